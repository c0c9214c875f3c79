"""GPU parity of the GEMM-facing dispatch options against the CPU oracle,
through the C-ABI: expert blocks aligned to a row tile (zeroed padding rows),
column-major block scales, and pre-quantised FP8 input passed through.

Everything here is integer or byte work, so the bar is bit-exact; rows the
definition leaves unwritten keep a canary pattern."""
import numpy as np
import pytest

import oracle
import workloads

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


def _run(ep, idx, w, x, E, P, A, use_fp8, cap=None, x_scales=None, col_major=False, guard=5):
    """layout (aligned) -> dispatch_ex into canary-filled buffers."""
    dev = _dev()
    T, K = idx.shape
    H = x.shape[1]
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), E, P, expert_alignment=A)
    h = lay.handle
    cap = T * K + E * (A - 1) if cap is None else cap
    rows_alloc = cap + guard
    ld = (cap + 3) // 4 * 4 if col_major else 0
    if use_fp8:
        recv = torch.full((rows_alloc, H), 0xA5, dtype=torch.uint8, device=dev)
        if col_major:
            sc = torch.full((H // 128, ld), -7.0, dtype=torch.float32, device=dev)
        else:
            sc = torch.full((rows_alloc, H // 128), -7.0, dtype=torch.float32, device=dev)
    else:
        recv = torch.full((rows_alloc, H), 0x5A5A, dtype=torch.int16, device=dev)
        sc = None
    if x_scales is not None:
        t_x = torch.from_numpy(x).to(dev)
        t_xs = torch.from_numpy(x_scales).to(dev)
    else:
        t_x = _bf16(x, dev)
        t_xs = None
    rc = ep.ep_dispatch_ex(t_x.data_ptr(), None if t_xs is None else t_xs.data_ptr(),
                           torch.from_numpy(w).to(dev).data_ptr(), H, int(use_fp8), ld,
                           recv.data_ptr(), None if sc is None else sc.data_ptr(), cap, h.c,
                           ep._stream())
    assert rc == ep.EP_OK, ep.ep_last_error()
    return lay, h, recv, sc, cap, t_x, t_xs


def _check(ep, lay, h, recv, sc, cap, ref, use_fp8, col_major=False):
    E = h.c.num_experts
    np.testing.assert_array_equal(lay.num_tokens_per_expert.cpu().numpy(), ref["num_tokens_per_expert"])
    np.testing.assert_array_equal(lay.num_tokens_per_partition.cpu().numpy(), ref["num_tokens_per_partition"])
    np.testing.assert_array_equal(lay.is_token_in_partition.cpu().numpy(), ref["is_token_in_partition"])
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), ref["expert_offset"])
    np.testing.assert_array_equal(h.slot.cpu().numpy(), ref["slot"])
    counts, n, status = ep.handle_recv_counts(h)
    np.testing.assert_array_equal(np.array(counts), np.diff(ref["expert_offset"]))
    assert n == int(ref["expert_offset"][-1])
    assert status == (ep.EP_ECAPACITY if ref["overflow"] else
                      (ep.EP_EIDS if ref["num_invalid"] else ep.EP_OK))
    rows = ref["rows"]
    got = recv.cpu().numpy()
    if use_fp8:
        np.testing.assert_array_equal(got[:rows], ref["recv_x"])
        assert (got[rows:] == 0xA5).all()
        g = sc.cpu().numpy()
        if col_major:
            np.testing.assert_array_equal(g[:, :rows].T.view(np.uint32), ref["recv_scales"].view(np.uint32))
            assert (g[:, rows:] == -7.0).all()
        else:
            np.testing.assert_array_equal(g[:rows].view(np.uint32), ref["recv_scales"].view(np.uint32))
            assert (g[rows:] == -7.0).all()
    else:
        got = got.view(np.uint16)
        np.testing.assert_array_equal(got[:rows], ref["recv_x"])
        assert (got[rows:] == 0x5A5A).all()


@pytest.mark.parametrize("name,A,col_major", [("v3", 128, False), ("v3", 128, True),
                                              ("skewed", 64, False), ("decode", 16, True),
                                              ("tiny", 4, False), ("large", 128, True)])
def test_aligned_layout_full_workloads(ep, name, A, col_major):
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    lay, h, recv, sc, cap, _, _ = _run(ep, idx, w, x, wl.E, wl.P, A, wl.use_fp8, col_major=col_major)
    ref = oracle.run_all(idx, w, x, wl.E, wl.P, wl.use_fp8, align=A)
    _check(ep, lay, h, recv, sc, cap, ref, wl.use_fp8, col_major)
    assert h.src_token.numel() == 0                 # no source-token table for aligned layouts
    if name == "v3":
        return                                      # combine at V3 is covered on the dense layout
    # combine through the aligned handle
    y = workloads.expert_outputs(wl, cap, seed_offset=1)
    out = ep.combine(_bf16(y, _dev()), h)
    np.testing.assert_array_equal(_bits(out), oracle.combine(y, ref["slot"], w))


@pytest.mark.parametrize("T,H,K,E,P,A,col_major,mask", [
    (1, 128, 1, 1, 1, 1, False, 0.0),
    (300, 1152, 6, 40, 8, 1, True, 0.1),
    (257, 512, 8, 64, 4, 32, True, 0.05),
    (96, 7168, 4, 256, 8, 128, False, 0.0),
    (2000, 256, 16, 1024, 64, 7, True, 0.02)])
def test_fp8_input_passthrough(ep, T, H, K, E, P, A, col_major, mask):
    rng = np.random.default_rng(T + H)
    idx, w = workloads.random_case(T + 9, T, E, K, mask_frac=mask)
    xq = rng.integers(0, 256, (T, H), dtype=np.uint32).astype(np.uint8)
    xs = rng.standard_normal((T, H // 128)).astype(np.float32)
    lay, h, recv, sc, cap, t_x, t_xs = _run(ep, idx, w, xq, E, P, A, True, x_scales=xs,
                                            col_major=col_major)
    ref = oracle.run_all(idx, w, None, E, P, True, align=A)
    recv_ref, sc_ref = oracle.dispatch_fp8_input(xq, xs, ref["slot"], ref["rows"])
    ref.update(recv_x=recv_ref, recv_scales=sc_ref)
    _check(ep, lay, h, recv, sc, cap, ref, True, col_major)
    # cached dispatch of new codes along the same routing (x_scales required)
    xq2 = rng.integers(0, 256, (T, H), dtype=np.uint32).astype(np.uint8)
    xs2 = rng.standard_normal((T, H // 128)).astype(np.float32)
    r2, s2 = ep.dispatch_cached(torch.from_numpy(xq2).to(t_x.device), h,
                                x_scales=torch.from_numpy(xs2).to(t_x.device))
    want_q, want_s = oracle.dispatch_fp8_input(xq2, xs2, ref["slot"], ref["rows"])
    rows = ref["rows"]
    np.testing.assert_array_equal(r2.view(torch.uint8).cpu().numpy()[:rows], want_q)
    g2 = s2.cpu().numpy()
    g2 = g2[:, :rows].T if col_major else g2[:rows]
    np.testing.assert_array_equal(g2.view(np.uint32), want_s.view(np.uint32))
    with pytest.raises(ep.EpError):
        ep.dispatch_cached(torch.from_numpy(xq2).to(t_x.device), h)


def test_aligned_capacity_drops(ep):
    """A capacity below the aligned total drops the pairs ranked past it; the
    padding rows past the capacity are not written."""
    T, H, K, E, A = 500, 256, 4, 32, 32
    idx, w = workloads.random_case(91, T, E, K)
    x = workloads.random_rows(92, T, H, "wide")
    total = int(oracle.expert_offsets(np.bincount(idx.reshape(-1), minlength=E), A)[-1])
    cap = total - 3 * A - 5
    lay, h, recv, sc, cap, _, _ = _run(ep, idx, w, x, E, 4, A, True, cap=cap)
    ref = oracle.run_all(idx, w, x, E, 4, True, capacity=cap, align=A)
    assert ref["overflow"] == 1 and ref["rows"] == cap
    _check(ep, lay, h, recv, sc, cap, ref, True)


def test_option_validation(ep):
    dev = _dev()
    idx, w = workloads.random_case(5, 64, 16, 2)
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), 16, 4, expert_alignment=8)
    h = lay.handle
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device=dev)
    r = torch.empty((64 * 2 + 16 * 7, 256), dtype=torch.uint8, device=dev)
    s = torch.empty((2, 64 * 2 + 16 * 7), dtype=torch.float32, device=dev)
    cap = 64 * 2 + 16 * 7
    # scale_ld below the capacity, not a multiple of 4, or in BF16 mode
    for ld, fp8 in [(cap - 4, 1), (cap + 2, 1), (cap, 0)]:
        rc = ep.ep_dispatch_ex(x.data_ptr(), None, None, 256, fp8, ld, r.data_ptr(),
                               s.data_ptr(), cap, h.c, ep._stream())
        assert rc == ep.EP_EINVAL and "scale_ld" in ep.ep_last_error()
    # x_scales in BF16 mode; capacity above the aligned worst case
    rc = ep.ep_dispatch_ex(x.data_ptr(), s.data_ptr(), None, 256, 0, 0, r.data_ptr(), None, cap,
                           h.c, ep._stream())
    assert rc == ep.EP_EINVAL and "x_scales" in ep.ep_last_error()
    rc = ep.ep_dispatch_ex(x.data_ptr(), None, None, 256, 1, 0, r.data_ptr(), s.data_ptr(),
                           cap + 1, h.c, ep._stream())
    assert rc == ep.EP_EINVAL and "capacity_rows" in ep.ep_last_error()
    with pytest.raises(ep.EpError):
        ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), 16, 4, expert_alignment=0)
    with pytest.raises(ep.EpError):
        ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), 16, 4, expert_alignment=2048)


def test_fp8_cached_combine_and_backward_on_aligned_and_static_handles(ep):
    """The calls that take a handle work the same on an aligned (padded) and a
    low-latency (static) handle: FP8 cached dispatch, FP8 combine, the backward
    of combine (padding rows keep their contents) -- each against the oracle."""
    dev = _dev()
    T, H, K, E, P, A, cap = 120, 1024, 4, 16, 4, 32, 40
    idx, w = workloads.random_case(131, T, E, K, mask_frac=0.05)
    x = workloads.random_rows(132, T, H, "wide")
    t_idx, t_w = torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev)
    handles = []
    lay = ep.get_dispatch_layout(t_idx, E, P, expert_alignment=A)
    recv_a, sc_a, h_a = ep.dispatch(_bf16(x, dev), t_w, lay, True)
    handles.append(("aligned", h_a, h_a.c.capacity_rows))
    recv_s, sc_s, lay_s = ep.low_latency_dispatch(_bf16(x, dev), t_idx, t_w, E, P, cap, True)
    handles.append(("static", lay_s.handle, E * cap))
    for name, h, rows in handles:
        slot = h.slot.cpu().numpy()
        # cached FP8 dispatch of new rows
        x2 = workloads.random_rows(133, T, H, "normal")
        r2, s2 = ep.dispatch_cached(_bf16(x2, dev), h)
        ref = oracle.dispatch(x2, slot, rows, True)
        used = slot[slot >= 0]
        assert np.array_equal(r2.view(torch.uint8).cpu().numpy()[used], ref[0][used]), name
        assert np.array_equal(s2.cpu().numpy()[used].view(np.uint32), ref[1][used].view(np.uint32)), name
        # FP8 combine of those rows
        out = ep.combine_fp8(r2, s2, h)
        q = r2.view(torch.uint8).cpu().numpy()
        assert np.array_equal(_bits(out), oracle.combine_fp8(q, s2.cpu().numpy(), slot, w)), name
        # and its unit-weight form, the dequantising backward of dispatch
        gx = ep.dispatch_backward_fp8(r2, s2, h)
        assert np.array_equal(_bits(gx), oracle.combine_fp8(q, s2.cpu().numpy(), slot, None)), name
        # backward of combine: rows no pair maps to keep the fill
        g = workloads.random_rows(134, T, H)
        gy0 = torch.full((rows, H), 0x1234, dtype=torch.int16, device=dev).view(torch.bfloat16)
        gy, _ = ep.combine_backward(_bf16(g, dev), h, grad_y=gy0)
        want, _ = oracle.combine_backward(g, None, slot, w, rows, fill=0x1234)
        assert np.array_equal(_bits(gy), want), name


@pytest.mark.parametrize("A,extra_ld", [(1, 0), (16, 8)])
def test_fp8_combine_on_column_major_scales(ep, A, extra_ld):
    """FP8 combine and the dequantising backward of dispatch read the scales
    in the layout the handle's dispatch wrote them: column-major [H/128][ld]
    here (ld past the capacity when extra_ld > 0).  Checked on dispatch's own
    rows, on a cached dispatch of new rows, and on random codes with random
    scales, each against the oracle on the same scales transposed to rows."""
    dev = _dev()
    T, H, K, E, P = 150, 2048, 6, 32, 8
    idx, w = workloads.random_case(141 + A, T, E, K, mask_frac=0.05)
    x = workloads.random_rows(142, T, H, "wide")
    t_idx, t_w = torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev)
    lay = ep.get_dispatch_layout(t_idx, E, P, expert_alignment=A)
    h = lay.handle
    cap = T * K + E * (A - 1)
    ld = (cap + 3) // 4 * 4 + extra_ld
    nb = H // 128
    recv = torch.empty((cap, H), dtype=torch.uint8, device=dev)
    sc = torch.full((nb, ld), -7.0, dtype=torch.float32, device=dev)
    rc = ep.ep_dispatch_ex(_bf16(x, dev).data_ptr(), None, t_w.data_ptr(), H, 1, ld, recv.data_ptr(),
                           sc.data_ptr(), cap, h.c, ep._stream())
    assert rc == ep.EP_OK, ep.ep_last_error()
    assert h.c.scale_ld == ld
    slot = h.slot.cpu().numpy()
    rng = np.random.default_rng(143)
    q_rand = rng.integers(0, 256, (cap, H), dtype=np.uint32).astype(np.uint8)
    q_rand[(q_rand & 0x7F) == 0x7F] ^= 0x01
    s_rand = (rng.standard_normal((nb, ld)).astype(np.float32) *
              np.ldexp(np.float32(1), rng.integers(-20, 21, (nb, ld))).astype(np.float32))
    x2 = workloads.random_rows(144, T, H, "normal")
    r2, s2 = ep.dispatch_cached(_bf16(x2, dev), h)
    assert s2.shape == (nb, ld)
    cases = [("dispatch rows", recv, sc), ("cached rows", r2, s2),
             ("random codes", torch.from_numpy(q_rand).to(dev), torch.from_numpy(s_rand).to(dev))]
    for name, q_t, s_t in cases:
        print(f"[gemm] fp8 combine column-major A={A} ld={ld} {name}", flush=True)
        out = ep.combine_fp8(q_t, s_t, h)
        gx = ep.dispatch_backward_fp8(q_t, s_t, h)
        q = q_t.view(torch.uint8).cpu().numpy()
        s_rows = np.ascontiguousarray(s_t.cpu().numpy()[:, :cap].T)     # [cap][H/128]
        assert np.array_equal(_bits(out), oracle.combine_fp8(q, s_rows, slot, w)), name
        assert np.array_equal(_bits(gx), oracle.combine_fp8(q, s_rows, slot, None)), name
