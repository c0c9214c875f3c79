"""GPU parity of the one-launch low-latency dispatch (static per-expert
capacity) against the CPU oracle, through the C-ABI.

Bit-exact: layout counts, mask, invalid count, slots, the rows written (FP8
codes + scales, or BF16 bits), the per-expert received counts and the
overflow status.  Rows past an expert's count are not written (checked with
a canary fill).  The handle then serves combine, cached dispatch and both
backward calls like a dense one; a captured HIP graph of dispatch + combine
is replayed with new inputs and checked on every replay."""
import numpy as np
import pytest

import oracle
import workloads
from conftest import grad_w_rel_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _check_grad_w(got, ref, g, y, slot, H):
    """grad_w is reduced in a fixed fp32 order on the GPU and in double by the
    oracle: |gpu - exact| <= gamma_d * sum_j |g_j y_j| (d the reduction depth) plus the
    oracle's rounding to fp32; undispatched pairs are exactly 0."""
    gf = workloads.f32_from_bf16_bits(g).astype(np.float64)
    yf = workloads.f32_from_bf16_bits(y).astype(np.float64)
    T, K = slot.shape
    for t in range(T):
        for k in range(K):
            s = slot[t, k]
            if s < 0:
                assert got[t, k] == 0.0
                continue
            mag = np.abs(gf[t] * yf[s]).sum()
            tol = grad_w_rel_bound(H) * mag + 2.0 ** -24 * abs(float(ref[t, k])) + 1e-38
            assert abs(float(got[t, k]) - float(ref[t, k])) <= tol, (t, k, got[t, k], ref[t, k])


def _alloc(ep, T, H, K, E, P, cap, use_fp8, dev):
    """Receive buffers with a canary fill, layout outputs and a workspace."""
    rows = E * cap
    if use_fp8:
        recv = torch.full((rows, H), 0xA5, dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
        sc = torch.full((rows, H // 128), -7.0, dtype=torch.float32, device=dev)
    else:
        recv = torch.full((rows, H), 0x5A5A, dtype=torch.int16, device=dev).view(torch.bfloat16)
        sc = None
    ws = torch.empty(ep.ep_workspace_bytes(T, K, E, P), dtype=torch.uint8, device=dev)
    lay = ep.Layout(torch.full((P,), -9, dtype=torch.int32, device=dev),
                    torch.full((E,), -9, dtype=torch.int32, device=dev),
                    torch.full((T, P), 7, dtype=torch.uint8, device=dev),
                    torch.full((1,), -9, dtype=torch.int32, device=dev),
                    ep.Handle(ep.ep_handle_t(), ws))
    return recv, sc, lay


def _check_dispatch(ep, idx, w, x, E, P, cap, use_fp8, recv, sc, lay, canary=True):
    T, K = idx.shape
    H = x.shape[1]
    ref = oracle.run_low_latency(idx, w, x, E, P, use_fp8, cap)
    np.testing.assert_array_equal(lay.num_tokens_per_expert.cpu().numpy(), ref["num_tokens_per_expert"])
    np.testing.assert_array_equal(lay.num_tokens_per_partition.cpu().numpy(), ref["num_tokens_per_partition"])
    np.testing.assert_array_equal(lay.is_token_in_partition.cpu().numpy(), ref["is_token_in_partition"])
    assert int(lay.num_invalid.cpu()[0]) == ref["num_invalid"]
    h = lay.handle
    assert h.c.stage == 2 and h.c.static_cap == cap and h.c.capacity_rows == E * cap
    np.testing.assert_array_equal(h.slot.cpu().numpy(), ref["slot"])
    counts, n, status = ep.handle_recv_counts(h)
    want_counts = np.minimum(ref["num_tokens_per_expert"], cap)
    np.testing.assert_array_equal(np.array(counts), want_counts)
    assert n == int(want_counts.sum())
    if ref["overflow"]:
        assert status == ep.EP_ECAPACITY
    elif ref["num_invalid"]:
        assert status == ep.EP_EIDS
    else:
        assert status == ep.EP_OK
    # written rows: expert e's first min(count, cap) rows; the rest keep the canary
    written = np.zeros(E * cap, bool)
    for e in range(E):
        written[e * cap:e * cap + want_counts[e]] = True
    if use_fp8:
        got = recv.view(torch.uint8).cpu().numpy()
        gsc = sc.cpu().numpy()
        np.testing.assert_array_equal(got[written], ref["recv_x"][written])
        np.testing.assert_array_equal(gsc[written].view(np.uint32), ref["recv_scales"][written].view(np.uint32))
        if canary:
            assert (got[~written] == 0xA5).all()
            assert (gsc[~written] == -7.0).all()
    else:
        got = _bits(recv)
        np.testing.assert_array_equal(got[written], ref["recv_x"][written])
        if canary:
            assert (got[~written] == 0x5A5A).all()
    return ref


def _run(ep, idx, w, x, E, P, cap, use_fp8, pass_weights=True):
    dev = _dev()
    T, K = idx.shape
    H = x.shape[1]
    recv, sc, lay = _alloc(ep, T, H, K, E, P, cap, use_fp8, dev)
    t_idx = torch.from_numpy(idx).to(dev)
    t_w = torch.from_numpy(w).to(dev)
    t_x = _bf16(x, dev) if T > 0 else torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    ep.low_latency_dispatch(t_x, t_idx, t_w if pass_weights else None, E, P, cap, use_fp8,
                            out=(recv, sc, lay))
    return recv, sc, lay, t_w


@pytest.mark.parametrize("name,cap", [("decode", 32), ("tiny", 12)])
def test_small_workloads(name, cap):
    """The two batches of at most 256 tokens through the one-launch dispatch,
    then combine through the same handle: decode (H=7168, 256 experts,
    top-8, FP8) with 32 rows per expert, nothing dropped; tiny (H=256, 16
    experts, top-2, BF16) with 12 rows per expert, so the most popular
    experts drop pairs."""
    ep = pytest.importorskip("combine_get_dispatch_scan_amd")
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    recv, sc, lay, t_w = _run(ep, idx, w, x, wl.E, wl.P, cap, wl.use_fp8)
    ref = _check_dispatch(ep, idx, w, x, wl.E, wl.P, cap, wl.use_fp8, recv, sc, lay)
    counts = np.bincount(idx[idx >= 0], minlength=wl.E)
    assert ref["overflow"] == int(counts.max() > cap)
    if name == "decode":
        assert ref["overflow"] == 0
    else:
        assert ref["overflow"] == 1
    y = workloads.expert_outputs(wl, wl.E * cap)
    out = ep.combine(_bf16(y, _dev()), lay.handle)
    np.testing.assert_array_equal(_bits(out), oracle.combine(y, ref["slot"], w))


@pytest.mark.parametrize("T,H,K,E,P,cap,use_fp8,kind", [
    (0, 256, 8, 16, 4, 4, True, "clean"),
    (1, 128, 1, 1, 1, 1, True, "clean"),
    (1, 7168, 8, 256, 8, 1, True, "clean"),
    (37, 1152, 6, 64, 8, 8, True, "dirty"),
    (64, 2048, 4, 32, 4, 3, True, "clean"),          # capacity overflow
    (200, 7168, 8, 256, 8, 16, True, "clean"),
    (255, 136, 9, 48, 6, 40, False, "dirty"),
    (256, 4096, 16, 1024, 64, 2, False, "clean"),
    (256, 7168, 8, 256, 8, 64, False, "clean"),
    (129, 512, 2, 8, 2, 200, True, "dup"),
    (7, 32768, 4, 16, 4, 3, True, "clean"),          # maximum hidden size
])
def test_shapes_and_edge_cases(T, H, K, E, P, cap, use_fp8, kind):
    ep = pytest.importorskip("combine_get_dispatch_scan_amd")
    seed = 7000 + T + 3 * K + E
    if kind == "clean":
        idx, w = workloads.random_case(seed, T, E, K)
    elif kind == "dirty":
        idx, w = workloads.random_case(seed, T, E, K, mask_frac=0.1, invalid_frac=0.05, dup_frac=0.05)
    else:
        idx, w = workloads.random_case(seed, T, E, K, distinct=False)
    x = workloads.random_rows(seed, T, H, "wide" if use_fp8 else "bits")
    recv, sc, lay, t_w = _run(ep, idx, w, x, E, P, cap, use_fp8)
    ref = _check_dispatch(ep, idx, w, x, E, P, cap, use_fp8, recv, sc, lay)
    if T > 0:
        y = workloads.random_rows(seed + 1, E * cap, H)
        out = ep.combine(_bf16(y, _dev()), lay.handle)
        np.testing.assert_array_equal(_bits(out), oracle.combine(y, ref["slot"], w))


def test_cached_dispatch_and_backward_use_the_static_handle():
    ep = pytest.importorskip("combine_get_dispatch_scan_amd")
    dev = _dev()
    T, H, K, E, P, cap = 96, 1024, 4, 32, 4, 6        # some experts overflow
    idx, w = workloads.random_case(71, T, E, K, mask_frac=0.05)
    x = workloads.random_rows(71, T, H)
    recv, sc, lay, t_w = _run(ep, idx, w, x, E, P, cap, False)
    ref = _check_dispatch(ep, idx, w, x, E, P, cap, False, recv, sc, lay)
    slot = ref["slot"]
    h = lay.handle
    # cached dispatch of new rows reuses the slots (BF16: the mode is the handle's)
    x2 = workloads.random_rows(72, T, H, "bits")
    r2 = torch.zeros((E * cap, H), dtype=torch.bfloat16, device=dev)
    ep.dispatch_cached(_bf16(x2, dev), h, r2)
    want, _ = oracle.dispatch(x2, slot, E * cap, False)
    np.testing.assert_array_equal(_bits(r2), want)
    # backward of dispatch: grad_x[t] = sum of its received rows' gradients
    g_recv = workloads.random_rows(73, E * cap, H)
    gx = ep.dispatch_backward(_bf16(g_recv, dev), h)
    np.testing.assert_array_equal(_bits(gx), oracle.dispatch_backward(g_recv, slot))
    # backward of combine, grad_w included
    g_out = workloads.random_rows(74, T, H)
    y = workloads.random_rows(75, E * cap, H)
    gy0 = torch.full((E * cap, H), 0x3F80, dtype=torch.int16, device=dev).view(torch.bfloat16)
    gy, gw = ep.combine_backward(_bf16(g_out, dev), h, y=_bf16(y, dev), grad_y=gy0)
    want_gy, want_gw = oracle.combine_backward(g_out, y, slot, w, E * cap, fill=0x3F80)
    np.testing.assert_array_equal(_bits(gy), want_gy)
    _check_grad_w(gw.cpu().numpy(), want_gw, g_out, y, slot, H)


def test_graph_capture_replays_match_the_oracle():
    """Dispatch + combine captured once in a HIP graph (no memset nodes),
    replayed on three new batches with eager work between the replays."""
    ep = pytest.importorskip("combine_get_dispatch_scan_amd")
    dev = _dev()
    T, H, K, E, P, cap = 128, 7168, 8, 256, 8, 24
    s_idx = torch.empty((T, K), dtype=torch.int64, device=dev)
    s_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    s_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    s_y = torch.empty((E * cap, H), dtype=torch.bfloat16, device=dev)
    s_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    recv, sc, lay = _alloc(ep, T, H, K, E, P, cap, True, dev)

    def step():
        ep.low_latency_dispatch(s_x, s_idx, s_w, E, P, cap, True, out=(recv, sc, lay))
        ep.combine(s_y, lay.handle, out=s_out)

    cases = []
    for r in range(4):
        idx, w = workloads.random_case(900 + r, T, E, K)
        x = workloads.random_rows(900 + r, T, H, "wide")
        y = workloads.random_rows(950 + r, E * cap, H)
        cases.append((idx, w, x, y))

    def load(c):
        idx, w, x, y = c
        s_idx.copy_(torch.from_numpy(idx))
        s_w.copy_(torch.from_numpy(w))
        s_x.copy_(_bf16(x, dev))
        s_y.copy_(_bf16(y, dev))

    load(cases[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                    # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for c in cases[1:]:
        load(c)
        junk = torch.randn(1 << 20, device=dev).sum()     # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        idx, w, x, y = c
        ref = _check_dispatch(ep, idx, w, x, E, P, cap, True, recv, sc, lay, canary=False)
        np.testing.assert_array_equal(_bits(s_out), oracle.combine(y, ref["slot"], w))
        del junk
