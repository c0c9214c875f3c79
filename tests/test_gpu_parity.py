"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Bit-exact for the layout outputs, slots, source tokens, FP8 codes, scales and
BF16 rows; combine within 1 BF16 ulp (and expected bit-exact, since both
sides run the same fp32 fma chain).  Full-size cases run the five workloads
in the launch configuration the benchmark uses."""
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


def _bf16_tensor(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _ulp_diff(a_bits, b_bits):
    """Distance in BF16 ulps (ordered-integer mapping, +0 == -0)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def run_gpu(ep, idx, w, x, y, E, P, use_fp8, capacity=None, guard_rows=3, pass_weights=True,
            combine_weights=None):
    """layout -> dispatch -> counts -> combine on the GPU; returns numpy."""
    dev = _dev()
    T, K = idx.shape
    H = x.shape[1]
    cap = T * K if capacity is None else capacity
    t_idx = torch.from_numpy(idx).to(dev)
    t_w = torch.from_numpy(w).to(dev)
    t_x = _bf16_tensor(x, dev)
    lay = ep.get_dispatch_layout(t_idx, E, P)
    # receive buffers with guard rows filled with a canary pattern
    if use_fp8:
        recv_full = torch.full((cap + guard_rows, H), 0xA5, dtype=torch.uint8, device=dev)
        sc_full = torch.full((cap + guard_rows, H // 128), -7.0, dtype=torch.float32, device=dev)
        recv = recv_full[:cap].view(torch.float8_e4m3fn)
        sc = sc_full[:cap]
    else:
        recv_full = torch.full((cap + guard_rows, H), 0x5A5A, dtype=torch.int16, device=dev)
        sc_full = None
        recv = recv_full[:cap].view(torch.bfloat16)
        sc = None
    h = lay.handle
    rc = ep.ep_dispatch(t_x.data_ptr(), t_w.data_ptr() if pass_weights else None, H, int(use_fp8),
                        recv.data_ptr(), sc.data_ptr() if sc is not None else None, cap, h.c,
                        ep._stream())
    assert rc == ep.EP_OK, ep.ep_last_error()
    counts, n, status = ep.handle_recv_counts(h)
    res = dict(
        num_tokens_per_partition=lay.num_tokens_per_partition.cpu().numpy(),
        num_tokens_per_expert=lay.num_tokens_per_expert.cpu().numpy(),
        is_token_in_partition=lay.is_token_in_partition.cpu().numpy(),
        num_invalid=int(lay.num_invalid.cpu().numpy()[0]),
        counts=np.array(counts, np.int32), N=n, status=status,
        slot=h.slot.cpu().numpy(), expert_offset=h.expert_offset.cpu().numpy(),
        src_token=h.src_token.cpu().numpy(), handle=h, lay=lay,
        recv_full=recv_full.cpu().numpy(), sc_full=None if sc_full is None else sc_full.cpu().numpy(),
    )
    if y is not None:
        # a receive-row buffer even when no pair was dispatched (the library
        # needs one whenever the capacity is not 0)
        t_y = _bf16_tensor(y, dev) if y.shape[0] > 0 else torch.zeros((1, H), dtype=torch.bfloat16, device=dev)
        cw = None if combine_weights is None else torch.from_numpy(combine_weights).to(dev)
        out = torch.full((T, H), 0x7777, dtype=torch.int16, device=dev).view(torch.bfloat16)
        ep.combine(t_y, h, topk_weights=cw, out=out)
        res["out"] = _bits(out)
    torch.cuda.synchronize()
    return res


def check(ep, idx, w, x, E, P, use_fp8, capacity=None, y=None, with_combine=True, tag=""):
    T, K = idx.shape
    H = x.shape[1]
    print(f"[parity] {tag} T={T} H={H} E={E} K={K} P={P} fp8={use_fp8} cap={capacity}", flush=True)
    ref = oracle.run_all(idx, w, x, E, P, use_fp8, capacity=capacity)
    rows = ref["rows"]
    if with_combine and y is None:
        y = workloads.random_rows(T * 31 + H, rows, H, "normal")
    got = run_gpu(ep, idx, w, x, y if with_combine else None, E, P, use_fp8, capacity=capacity)
    for key in ("num_tokens_per_partition", "num_tokens_per_expert", "is_token_in_partition"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["num_invalid"] == ref["num_invalid"]
    assert np.array_equal(got["counts"], ref["num_tokens_per_expert"])
    assert got["N"] == ref["N"]
    assert np.array_equal(got["expert_offset"], ref["expert_offset"])
    assert np.array_equal(got["slot"], ref["slot"])
    assert np.array_equal(got["src_token"][:rows], ref["src_token"])
    exp_status = ep.EP_ECAPACITY if ref["overflow"] else (ep.EP_EIDS if ref["num_invalid"] else ep.EP_OK)
    assert got["status"] == exp_status
    cap = T * K if capacity is None else capacity
    recv_full = got["recv_full"]
    if use_fp8:
        assert np.array_equal(recv_full[:rows], ref["recv_x"])
        assert np.array_equal(got["sc_full"][:rows].view(np.uint32), ref["recv_scales"].view(np.uint32))
        # rows past N and the guard rows are never written
        assert np.all(recv_full[rows:] == 0xA5)
        assert np.all(got["sc_full"][rows:] == -7.0)
    else:
        assert np.array_equal(recv_full[:rows].view(np.uint16), ref["recv_x"])
        assert np.all(recv_full[rows:] == 0x5A5A)
    if with_combine:
        ref_out = oracle.combine(y, ref["slot"], w)
        d = _ulp_diff(got["out"], ref_out)
        assert d.max(initial=0) <= 1, f"combine max ulp {d.max()}"
        assert np.array_equal(got["out"], ref_out), f"combine: {(d > 0).sum()} elements differ by 1 ulp"
    return ref, got


# ----------------------------------------------------------------------------
# the five workloads at full size
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "decode", "skewed", "v3", "large"])
def test_workload_full_size(ep, name):
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    y = workloads.expert_outputs(wl, N)
    check(ep, idx, w, x, wl.E, wl.P, wl.use_fp8, y=y, tag=name)


# ----------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------

SHAPES = [
    # T, H, E, K, P, fp8
    (1, 128, 1, 1, 1, True),
    (1, 8, 4, 2, 2, False),
    (63, 24, 8, 3, 2, False),
    (257, 520, 16, 4, 4, False),
    (300, 1152, 32, 6, 8, True),
    (513, 2176, 64, 8, 16, True),
    (700, 256, 1024, 16, 64, True),
    (1000, 384, 5, 5, 5, True),
    (2049, 4096, 256, 8, 8, True),
    (33000, 128, 256, 4, 8, True),      # > 128 chunks: separate scan kernel, tables in HBM
    (3, 32768, 16, 8, 4, True),         # maximum hidden size
    (5, 32760, 16, 16, 16, False),      # maximum BF16 hidden (a multiple of 8), K = E
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T%d_H%d_E%d_K%d_P%d_%s" % (*s[:5], "fp8" if s[5] else "bf16"))
@pytest.mark.parametrize("mode", ["clean", "dirty"])
def test_shapes(ep, shape, mode):
    T, H, E, K, P, fp8 = shape
    kw = {} if mode == "clean" else dict(distinct=False, mask_frac=0.1, invalid_frac=0.05, dup_frac=0.1)
    idx, w = workloads.random_case(T * 7 + H, T, E, K, **kw)
    x = workloads.random_rows(T + H, T, H, "normal")
    check(ep, idx, w, x, E, P, fp8, tag=f"shape-{mode}")


@pytest.mark.parametrize("kind", ["wide", "bits", "zeros", "subnormal", "ties"])
def test_fp8_value_mixes(ep, kind):
    T, H, E, K, P = 130, 1024, 16, 4, 4
    idx, w = workloads.random_case(5, T, E, K)
    x = workloads.random_rows(6, T, H, kind)
    check(ep, idx, w, x, E, P, True, tag=f"fp8-{kind}", with_combine=False)


@pytest.mark.parametrize("kind", ["wide", "bits", "subnormal"])
def test_combine_value_mixes(ep, kind):
    T, H, E, K, P = 200, 512, 32, 8, 4
    idx, w = workloads.random_case(8, T, E, K, mask_frac=0.1)
    x = workloads.random_rows(9, T, H, "normal")
    N = int((idx >= 0).sum())
    y = workloads.random_rows(10, N, H, kind)
    if kind == "bits":
        # keep sums finite: clear the top exponent bit
        y = (y & np.uint16(0xBFFF)).astype(np.uint16)
    check(ep, idx, w, x, E, P, False, y=y, tag=f"combine-{kind}")


def test_empty_input(ep):
    dev = _dev()
    E, P, K, H = 16, 4, 4, 256
    idx = np.zeros((0, K), np.int64)
    t_idx = torch.empty((0, K), dtype=torch.int64, device=dev)
    lay = ep.get_dispatch_layout(t_idx, E, P)
    x = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    w = torch.empty((0, K), dtype=torch.float32, device=dev)
    recv, sc, h = ep.dispatch(x, w, lay, True)
    counts, n, st = ep.handle_recv_counts(h)
    out = ep.combine(torch.empty((0, H), dtype=torch.bfloat16, device=dev), h)
    torch.cuda.synchronize()
    assert n == 0 and st == ep.EP_OK and sum(counts) == 0
    assert lay.num_tokens_per_partition.cpu().sum().item() == 0
    assert lay.num_invalid.cpu().item() == 0
    assert out.shape == (0, H) and recv.shape == (0, H)
    del idx


@pytest.mark.parametrize("cap_kind", ["exact", "minus7", "half", "zero"])
def test_capacity(ep, cap_kind):
    T, H, E, K, P = 333, 1024, 32, 4, 4
    idx, w = workloads.random_case(21, T, E, K, mask_frac=0.05)
    x = workloads.random_rows(22, T, H, "normal")
    N = int((idx >= 0).sum())
    cap = dict(exact=N, minus7=N - 7, half=N // 2, zero=0)[cap_kind]
    for fp8 in (False, True):
        check(ep, idx, w, x, E, P, fp8, capacity=cap, tag=f"cap-{cap_kind}")


def test_all_masked_tokens(ep):
    T, H, E, K, P = 100, 256, 8, 2, 2
    idx, w = workloads.random_case(31, T, E, K)
    idx[::3] = -1
    x = workloads.random_rows(32, T, H, "normal")
    ref, got = check(ep, idx, w, x, E, P, False, tag="masked-rows")
    assert np.all(got["out"][::3] == 0)


def test_cached_dispatch_is_bit_identical(ep):
    dev = _dev()
    for fp8 in (False, True):
        T, H, E, K, P = 500, 2048, 64, 6, 8
        idx, w = workloads.random_case(41, T, E, K, mask_frac=0.05)
        x1 = workloads.random_rows(42, T, H, "normal")
        x2 = workloads.random_rows(43, T, H, "wide")
        lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), E, P)
        t_w = torch.from_numpy(w).to(dev)
        recv1, sc1, h = ep.dispatch(_bf16_tensor(x1, dev), t_w, lay, fp8)
        recv2c, sc2c = ep.dispatch_cached(_bf16_tensor(x2, dev), h)
        lay2 = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), E, P)
        recv2f, sc2f, _ = ep.dispatch(_bf16_tensor(x2, dev), t_w, lay2, fp8)
        torch.cuda.synchronize()
        N = int((idx >= 0).sum())
        a = recv2c[:N].view(torch.uint8).cpu().numpy()
        b = recv2f[:N].view(torch.uint8).cpu().numpy()
        assert np.array_equal(a, b)
        if fp8:
            assert np.array_equal(sc2c[:N].cpu().numpy(), sc2f[:N].cpu().numpy())
        ref = oracle.run_all(idx, w, x2, E, P, fp8)
        if fp8:
            assert np.array_equal(a, ref["recv_x"])
        else:
            assert np.array_equal(a.view(np.uint16), ref["recv_x"])


def test_combine_weight_sources(ep):
    dev = _dev()
    T, H, E, K, P = 128, 512, 16, 4, 4
    idx, w = workloads.random_case(51, T, E, K)
    x = workloads.random_rows(52, T, H, "normal")
    N = int((idx >= 0).sum())
    y = workloads.random_rows(53, N, H, "normal")
    w2 = np.ascontiguousarray(w[:, ::-1])
    # weights given at combine time override the dispatch copy
    ref = oracle.run_all(idx, w, x, E, P, False)
    got = run_gpu(ep, idx, w, x, y, E, P, False, combine_weights=w2)
    assert np.array_equal(got["out"], oracle.combine(y, ref["slot"], w2))
    # no weights at dispatch: combine without weights is rejected
    got = run_gpu(ep, idx, w, x, None, E, P, False, pass_weights=False)
    h = got["handle"]
    assert h.c.has_weights == 0
    rc = ep.ep_combine(_bf16_tensor(y, dev).data_ptr(), h.c, None,
                       torch.empty((T, H), dtype=torch.bfloat16, device=dev).data_ptr(), ep._stream())
    assert rc == ep.EP_EINVAL


def test_async_counts_match_sync(ep):
    dev = _dev()
    wl = workloads.config("skewed")
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    for cap in (wl.T * wl.K, N - 5):
        lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), wl.E, wl.P)
        recv, sc, h = ep.dispatch(_bf16_tensor(x, dev), torch.from_numpy(w).to(dev), lay, False,
                                  capacity_rows=cap)
        buf = torch.full((wl.E + 5,), -9, dtype=torch.int32, pin_memory=True)
        ep.handle_recv_counts_async(h, buf)
        ev = torch.cuda.Event()
        ev.record()
        ev.synchronize()
        a = ep.recv_counts_decode(h, buf)
        b = ep.handle_recv_counts(h)
        assert a == b
        assert a[1] == N and a[2] == (ep.EP_OK if cap >= N else ep.EP_ECAPACITY)
        assert np.array_equal(np.array(a[0]), np.bincount(idx[idx >= 0], minlength=wl.E))


def test_counts_copied_before_dispatch_on_a_side_stream(ep):
    """For a dense layout the counts can be read back right after the layout,
    on a second stream, overlapping dispatch; the decode still reports drops
    (N > capacity) once the handle is dispatched."""
    dev = _dev()
    wl = workloads.config("v3")
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    t_idx, t_w, t_x = torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev), _bf16_tensor(x, dev)
    for cap in (wl.T * wl.K, N - 1000):
        lay = ep.get_dispatch_layout(t_idx, wl.E, wl.P)
        laid = torch.cuda.Event()
        laid.record(main)
        buf = torch.full((wl.E + 5,), -9, dtype=torch.int32, pin_memory=True)
        side.wait_event(laid)
        with torch.cuda.stream(side):
            ep.handle_recv_counts_async(lay.handle, buf)
            ready = torch.cuda.Event()
            ready.record(side)
        recv, sc, h = ep.dispatch(t_x, t_w, lay, True, capacity_rows=cap)
        ready.synchronize()
        counts, n, st = ep.recv_counts_decode(h, buf)
        torch.cuda.synchronize()
        assert n == N and st == (ep.EP_OK if cap >= N else ep.EP_ECAPACITY)
        assert np.array_equal(np.array(counts), np.bincount(idx[idx >= 0], minlength=wl.E))
        assert (counts, n, st) == ep.handle_recv_counts(h)


def test_determinism(ep):
    """Ten runs of the whole path give bit-identical outputs (slots come
    from integer adds over LDS masks, never from the order of atomics)."""
    wl = workloads.config("skewed")
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    y = workloads.expert_outputs(wl, N)
    first = run_gpu(ep, idx, w, x, y, wl.E, wl.P, wl.use_fp8)
    for _ in range(9):
        again = run_gpu(ep, idx, w, x, y, wl.E, wl.P, wl.use_fp8)
        assert again["N"] == first["N"] == N
        # src_token rows at and beyond N are never written (workspace contents)
        assert np.array_equal(first["src_token"][:N], again["src_token"][:N])
        for key in ("slot", "recv_full", "out", "is_token_in_partition", "expert_offset"):
            assert np.array_equal(first[key], again[key]), key


def test_device_e4m3fn_encoder_exhaustive(ep):
    """Every fp32 bit pattern in [2^-11, 464] (both signs) and a sample below:
    the device encoder equals the oracle's."""
    dev = _dev()
    lo = int(np.float32(2.0 ** -11).view(np.uint32))
    hi = int(np.float32(464.0).view(np.uint32))
    step = 1 << 24
    for start in range(lo, hi + 1, step):
        u = np.arange(start, min(start + step, hi + 1), dtype=np.uint32)
        for sign in (0, 0x80000000):
            v = (u | np.uint32(sign)).view(np.float32)
            got = ep.e4m3fn_encode(torch.from_numpy(v).to(dev)).cpu().numpy()
            ref = oracle.e4m3fn_array(v)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, (v[bad[:4]], got[bad[:4]], ref[bad[:4]])
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    v = u.view(np.float32)
    got = ep.e4m3fn_encode(torch.from_numpy(v).to(dev)).cpu().numpy()
    assert np.array_equal(got, oracle.e4m3fn_array(v))


def test_graph_capture_of_the_dense_path(ep):
    """layout -> dispatch (FP8) -> combine captured once in a HIP graph (the
    library records no memset nodes) and replayed on three new batches with
    eager work between the replays; every replay matches the oracle."""
    dev = _dev()
    T, H, K, E, P = 700, 1024, 6, 64, 8
    cap = T * K
    s_idx = torch.empty((T, K), dtype=torch.int64, device=dev)
    s_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    s_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    s_y = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ep.ep_workspace_bytes(T, K, E, P), dtype=torch.uint8, device=dev)
    ntpp = torch.empty(P, dtype=torch.int32, device=dev)
    ntpe = torch.empty(E, dtype=torch.int32, device=dev)
    itip = torch.empty((T, P), dtype=torch.uint8, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    recv = torch.empty((cap, H), dtype=torch.uint8, device=dev)
    sc = torch.empty((cap, H // 128), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    h = ep.ep_handle_t()
    p = lambda t: t.data_ptr()

    def step():
        s = ep._stream()
        assert ep.ep_get_dispatch_layout(p(s_idx), T, K, E, P, p(ntpp), p(ntpe), p(itip), p(ninv),
                                         p(ws), ws.numel(), h, s) == ep.EP_OK
        assert ep.ep_dispatch(p(s_x), p(s_w), H, 1, p(recv), p(sc), cap, h, s) == ep.EP_OK
        assert ep.ep_combine(p(s_y), h, None, p(out), s) == ep.EP_OK

    cases = []
    for r in range(4):
        idx, w = workloads.random_case(600 + r, T, E, K, mask_frac=0.05)
        cases.append((idx, w, workloads.random_rows(600 + r, T, H, "wide"),
                      workloads.random_rows(650 + r, cap, H)))

    def load(c):
        s_idx.copy_(torch.from_numpy(c[0]))
        s_w.copy_(torch.from_numpy(c[1]))
        s_x.copy_(_bf16_tensor(c[2], dev))
        s_y.copy_(_bf16_tensor(c[3], dev))

    load(cases[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                        # warm-up outside capture
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
        ref = oracle.run_all(idx, w, x, E, P, True, y_bits=y)
        rows = ref["rows"]
        assert np.array_equal(ntpe.cpu().numpy(), ref["num_tokens_per_expert"])
        assert np.array_equal(itip.cpu().numpy(), ref["is_token_in_partition"])
        assert np.array_equal(recv.cpu().numpy()[:rows], ref["recv_x"])
        assert np.array_equal(sc.cpu().numpy()[:rows].view(np.uint32), ref["recv_scales"].view(np.uint32))
        assert np.array_equal(_bits(out), ref["out"])
        del junk


def test_two_host_threads_on_two_streams(ep):
    """The library keeps no shared mutable state (the last-error string is per
    thread, workspaces and handles belong to the caller): two host threads,
    each on its own stream and workspace, run the path concurrently and each
    gets the oracle's result."""
    import threading
    dev = _dev()
    jobs = []
    for j, (T, H, E, K, P, fp8) in enumerate([(1500, 1024, 64, 6, 8, True), (900, 776, 32, 4, 4, False)]):
        idx, w = workloads.random_case(800 + j, T, E, K, mask_frac=0.05)
        x = workloads.random_rows(810 + j, T, H, "wide" if fp8 else "normal")
        ref = oracle.run_all(idx, w, x, E, P, fp8)
        y = workloads.random_rows(820 + j, ref["rows"], H)
        jobs.append(dict(args=(idx, w, x, y, E, P, fp8), ref=ref, ref_out=oracle.combine(y, ref["slot"], w)))
    errors = []

    def worker(job):
        try:
            idx, w, x, y, E, P, fp8 = job["args"]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                t_idx = torch.from_numpy(idx).to(dev)
                t_w = torch.from_numpy(w).to(dev)
                t_x = _bf16_tensor(x, dev)
                t_y = _bf16_tensor(y, dev)
                for _ in range(5):
                    lay = ep.get_dispatch_layout(t_idx, E, P)
                    recv, sc, h = ep.dispatch(t_x, t_w, lay, fp8)
                    out = ep.combine(t_y, h)
                s.synchronize()
                rows = job["ref"]["rows"]
                got = recv.view(torch.uint8).cpu().numpy() if fp8 else _bits(recv)
                assert np.array_equal(got[:rows], job["ref"]["recv_x"])
                assert np.array_equal(h.slot.cpu().numpy(), job["ref"]["slot"])
                assert np.array_equal(_bits(out), job["ref_out"])
                # an error on this thread leaves the other thread's message alone
                assert ep.ep_dispatch(None, None, 0, 0, None, None, 0, ep.ep_handle_t(), None) == ep.EP_EINVAL
        except Exception as e:      # surfaced by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors


@pytest.mark.parametrize("fp8", [False, True])
def test_redispatch_on_the_same_handle(ep, fp8):
    """A dispatch that dropped pairs, then a dispatch with room for all of
    them on the same handle (no new layout), then a short one again: each
    reports its own overflow status and matches the oracle at its capacity
    (the handle carries the routing, GeekNews usage section)."""
    dev = _dev()
    T, H, E, K, P = 257, 1024, 32, 4, 4
    idx, w = workloads.random_case(71, T, E, K, mask_frac=0.05)
    x = workloads.random_rows(72, T, H, "normal")
    N = int((idx >= 0).sum())
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), E, P)
    t_x, t_w = _bf16_tensor(x, dev), torch.from_numpy(w).to(dev)
    for cap in (N - 7, T * K, N - 1, N):
        print(f"[parity] re-dispatch fp8={fp8} cap={cap} N={N}", flush=True)
        recv, sc, h = ep.dispatch(t_x, t_w, lay, fp8, capacity_rows=cap)
        counts, n, st = ep.handle_recv_counts(h)
        buf = torch.full((E + 5,), -9, dtype=torch.int32, pin_memory=True)
        ep.handle_recv_counts_async(h, buf)
        torch.cuda.synchronize()
        assert ep.recv_counts_decode(h, buf) == (counts, n, st)
        ref = oracle.run_all(idx, w, x, E, P, fp8, capacity=cap)
        assert st == (ep.EP_ECAPACITY if ref["overflow"] else ep.EP_OK), (cap, st)
        assert n == N and np.array_equal(np.array(counts), ref["num_tokens_per_expert"])
        assert np.array_equal(h.slot.cpu().numpy(), ref["slot"])
        rows = ref["rows"]
        assert np.array_equal(h.src_token.cpu().numpy()[:rows], ref["src_token"])
        got = recv[:rows].view(torch.uint8 if fp8 else torch.int16).cpu().numpy()
        assert np.array_equal(got if fp8 else got.view(np.uint16), ref["recv_x"])
        if fp8:
            assert np.array_equal(sc[:rows].cpu().numpy().view(np.uint32), ref["recv_scales"].view(np.uint32))
        y = workloads.random_rows(73, max(rows, 1), H, "normal")
        out = ep.combine(_bf16_tensor(y, dev), h)
        assert np.array_equal(_bits(out), oracle.combine(y[:rows], ref["slot"], w))
    assert h.c.dispatch_seq == 4


def test_no_writes_past_any_output(ep):
    """Canary bytes after the end of every layout output, and in the gaps of
    the workspace after the handle's arrays (pair codes, slots, source tokens,
    weight copy), stay untouched through layout, dispatch and combine."""
    dev = _dev()
    T, H, E, K, P = 333, 512, 24, 3, 6          # T*K = 999: arrays end inside a 256-byte region
    idx, w = workloads.random_case(81, T, E, K, mask_frac=0.1, invalid_frac=0.02, dup_frac=0.05,
                                   distinct=False)
    x = workloads.random_rows(82, T, H, "normal")
    G = 13
    itip = torch.full((T * P + G,), 0xC3, dtype=torch.uint8, device=dev)
    ntpp = torch.full((P + G,), -123, dtype=torch.int32, device=dev)
    ntpe = torch.full((E + G,), -123, dtype=torch.int32, device=dev)
    ninv = torch.full((1 + G,), -123, dtype=torch.int32, device=dev)
    nbytes = ep.ep_workspace_bytes(T, K, E, P)
    ws = torch.full((nbytes,), 0xE7, dtype=torch.uint8, device=dev)
    h = ep.ep_handle_t()
    rc = ep.ep_get_dispatch_layout(torch.from_numpy(idx).to(dev).data_ptr(), T, K, E, P, ntpp.data_ptr(),
                                   ntpe.data_ptr(), itip.data_ptr(), ninv.data_ptr(), ws.data_ptr(),
                                   nbytes, h, ep._stream())
    assert rc == ep.EP_OK, ep.ep_last_error()
    cap = T * K
    recv = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    t_w = torch.from_numpy(w).to(dev)
    rc = ep.ep_dispatch(_bf16_tensor(x, dev).data_ptr(), t_w.data_ptr(), H, 0, recv.data_ptr(), None,
                        cap, h, ep._stream())
    assert rc == ep.EP_OK, ep.ep_last_error()
    ref = oracle.run_all(idx, w, x, E, P, False)
    N = ref["N"]
    y = workloads.random_rows(83, max(N, 1), H, "normal")
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    assert ep.ep_combine(_bf16_tensor(y, dev).data_ptr(), h, None, out.data_ptr(), ep._stream()) == ep.EP_OK
    torch.cuda.synchronize()
    a = itip.cpu().numpy()
    assert np.array_equal(a[:T * P].reshape(T, P), ref["is_token_in_partition"])
    assert np.all(a[T * P:] == 0xC3)
    for t, n, want in ((ntpp, P, ref["num_tokens_per_partition"]), (ntpe, E, ref["num_tokens_per_expert"]),
                       (ninv, 1, np.array([ref["num_invalid"]]))):
        v = t.cpu().numpy()
        assert np.array_equal(v[:n], want) and np.all(v[n:] == -123)
    wsb = ws.cpu().numpy()
    base = ws.data_ptr()
    off = lambda p: p - base
    regions = sorted([(off(h.pair_code), T * K * 4), (off(h.slot), T * K * 4),
                      (off(h.src_token), N * 4), (off(h.weights), T * K * 4)])
    ends = [r[0] for r in regions[1:]] + [nbytes]
    for (start, used), end in zip(regions, ends):
        gap = wsb[start + used:end]
        if end > off(h.expert_offset) > start:           # offsets + status sit between two arrays
            gap = wsb[start + used:off(h.expert_offset)]
        assert np.all(gap == 0xE7), (start, used, end)
    assert np.array_equal(_bits(out), oracle.combine(y[:N], ref["slot"], w))


@pytest.mark.parametrize("T,H,K,E,P", [(1, 256, 4, 8, 2), (333, 1000, 16, 64, 8), (257, 7168, 8, 256, 8),
                                       (5, 32768, 2, 4, 1), (130, 4104, 6, 32, 4)])
def test_token_owner_form_of_combine(ep, monkeypatch, T, H, K, E, P):
    """The token-owner combine (whole tokens per workgroup, output staged in
    LDS; the default past 160 MB of output) forced on small shapes: ragged
    token tails, hidden sizes off the 512-channel step, one token of 32768
    channels per workgroup, K = 16, masked and invalid ids.  Combine and the
    backward of dispatch against the oracle, bit for bit."""
    monkeypatch.setenv("EP_COMBINE_OWNER", "1")
    dev = _dev()
    idx, w = workloads.random_case(T + H, T, E, K, mask_frac=0.1, invalid_frac=0.03, dup_frac=0.03,
                                   distinct=False)
    x = workloads.random_rows(T + 7, T, H, "wide" if H % 128 == 0 else "bits")
    ref, got = check(ep, idx, w, x, E, P, False, tag="owner-form")
    g = workloads.random_rows(T + 8, T * K, H, "normal")
    gx = ep.dispatch_backward(_bf16_tensor(g, dev), got["handle"])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(gx), oracle.dispatch_backward(g[:ref["rows"]], ref["slot"]))


def test_binding_refuses_views_wrong_types_and_host_tensors(ep):
    """The binding hands the library bare addresses of dense rows, so it
    refuses what would be misread: a non-contiguous view, an element type the
    call does not take, a tensor in host memory."""
    dev = _dev()
    idx, w = workloads.random_case(71, 64, 16, 4)
    t_idx = torch.from_numpy(idx).to(dev)
    with pytest.raises(TypeError):
        ep.get_dispatch_layout(t_idx.to(torch.int32), 16, 4)
    with pytest.raises(ValueError):
        ep.get_dispatch_layout(torch.from_numpy(idx), 16, 4)
    lay = ep.get_dispatch_layout(t_idx, 16, 4)
    x = torch.randn((256, 64), device=dev).to(torch.bfloat16)
    with pytest.raises(ValueError):
        ep.dispatch(x.t(), torch.from_numpy(w).to(dev), lay, False)          # [64, 256] view
    with pytest.raises(TypeError):
        ep.dispatch(x.t().contiguous().float(), torch.from_numpy(w).to(dev), lay, False)
    recv, _, h = ep.dispatch(x.t().contiguous(), torch.from_numpy(w).to(dev), lay, False)
    y = torch.zeros((recv.shape[0], 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(TypeError):
        ep.combine(y, h, torch.from_numpy(w).to(dev).double())
    with pytest.raises(ValueError):
        ep.combine(torch.zeros((256, recv.shape[0]), dtype=torch.bfloat16, device=dev).t(), h)
    out = ep.combine(y, h)
    torch.cuda.synchronize()
    assert out.shape == (64, 256) and not out.view(torch.int16).any()


def _random_cases(n=40, seed=2026):
    """Seeded shapes across the boundary's range: T up to 3000 (0 included),
    K up to 16, E up to 1024 in P up to 64 partitions, hidden sizes on and
    off the row steps, clean and dirty ids, full and reduced capacities."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        P = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        E = P * int(rng.integers(1, 1024 // P + 1))
        K = int(rng.integers(1, 17))
        T = 0 if i == 0 else int(np.exp(rng.uniform(0, np.log(3000))))
        fp8 = bool(rng.integers(0, 2))
        H = 128 * int(rng.integers(1, 25)) if fp8 else 8 * int(rng.integers(1, 601))
        dirty = bool(rng.integers(0, 2))
        cap_frac = float(rng.choice([1.0, 1.0, rng.uniform(0, 1)]))
        cases.append((i, T, H, E, K, P, fp8, dirty, cap_frac))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: "case%d" % c[0])
def test_random_shapes(ep, case):
    """Layout, slots, rows, scales and combine bit-exact, then both backward
    calls on the same handle, on seeded random shapes."""
    i, T, H, E, K, P, fp8, dirty, cap_frac = case
    kw = dict(distinct=K <= E and not dirty)
    if dirty:
        kw.update(mask_frac=0.1, invalid_frac=0.03, dup_frac=0.05)
    idx, w = workloads.random_case(5000 + i, T, E, K, **kw)
    x = workloads.random_rows(6000 + i, T, H, "normal")
    cap = None if cap_frac >= 1.0 else int(T * K * cap_frac)
    ref, got = check(ep, idx, w, x, E, P, fp8, capacity=cap, tag=f"random-{i}")
    if T == 0:
        return
    dev = _dev()
    h = got["handle"]
    rows_cap = T * K if cap is None else cap
    gr = workloads.random_rows(7000 + i, rows_cap, H, "normal")
    g = workloads.random_rows(8000 + i, T, H, "normal")
    empty = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    gx = ep.dispatch_backward(_bf16_tensor(gr, dev) if rows_cap else empty, h)
    yb = workloads.random_rows(9000 + i, rows_cap, H, "normal")
    gy, gw = ep.combine_backward(_bf16_tensor(g, dev), h, y=_bf16_tensor(yb, dev) if rows_cap else empty)
    torch.cuda.synchronize()
    rows = ref["rows"]
    assert np.array_equal(_bits(gx), oracle.dispatch_backward(gr[:rows], ref["slot"]))
    ref_gy, ref_gw = oracle.combine_backward(g, yb[:rows], ref["slot"], w, rows_cap)
    assert np.array_equal(_bits(gy)[:rows], ref_gy[:rows])
    if rows_cap == 0:
        assert not gw.cpu().numpy().any()           # nothing dispatched: every grad_w is 0
    else:
        from test_gpu_backward import _check_grad_w_all
        _check_grad_w_all(gw.cpu().numpy(), ref_gw, g, yb, ref["slot"], H)


def test_debug_launch_trace():
    """EP_DEBUG=1 makes every launch print its kernel, grid, block and LDS
    (read once per process, so a child process runs a small forward)."""
    import os
    import subprocess
    import sys
    _dev()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch, combine_get_dispatch_scan_amd as ep\n"
        "d = torch.device('cuda:0')\n"
        "idx = torch.randint(0, 32, (600, 4), device=d)\n"
        "lay = ep.get_dispatch_layout(idx, 32, 4)\n"
        "x = torch.randn((600, 256), device=d).to(torch.bfloat16)\n"
        "recv, sc, h = ep.dispatch(x, torch.rand((600, 4), device=d), lay, True)\n"
        "ep.combine(torch.zeros((recv.shape[0], 256), dtype=torch.bfloat16, device=d), h)\n"
        "torch.cuda.synchronize()\n" % root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, EP_DEBUG="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[moe_ep] ")]
    kernels = [l.split()[1] for l in lines]
    assert kernels[:4] == ["layout_chunk_kernel", "scan_kernel", "dispatch_fp8_kernel", "combine_kernel"], lines
    assert all("grid=(" in l and "block=(" in l and "lds=" in l for l in lines)


def test_hand_worked_examples_on_the_gpu(ep):
    """The hand-worked examples in tests/golden/ (layout, slots, combine,
    aligned and static layouts, both backward calls, the FP8 combine and the
    expert-parallel flow) straight on the HIP path, with no oracle between:
    every value is the one worked out by hand."""
    import json
    import os
    dev = _dev()
    gdir = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    g = json.load(open(os.path.join(gdir, "layout_worked_example.json")))
    T, K, E, P, H = g["T"], g["K"], g["E"], g["P"], 8
    t_idx = torch.tensor(g["topk_idx"], dtype=torch.int64, device=dev)
    w = torch.tensor(g["combine"]["weights"], dtype=torch.float32, device=dev)
    f32 = lambda t: workloads.f32_from_bf16_bits(_bits(t))

    lay = ep.get_dispatch_layout(t_idx, E, P)
    assert lay.num_tokens_per_expert.tolist() == g["num_tokens_per_expert"]
    assert lay.num_tokens_per_partition.tolist() == g["num_tokens_per_partition"]
    assert lay.is_token_in_partition.tolist() == g["is_token_in_partition"]
    assert int(lay.num_invalid[0]) == g["num_invalid"]
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    _, _, h = ep.dispatch(x, w, lay, False, capacity_rows=15)
    assert h.slot.tolist() == g["slot"]
    assert h.expert_offset.tolist() == g["expert_offset"]
    assert h.src_token.tolist()[:9] == g["src_token"]
    # y[r] = [r, -r] repeated over the 8 channels
    y = torch.tensor([[r, -r] * 4 for r in range(15)], dtype=torch.float32, device=dev).to(torch.bfloat16)
    out = f32(ep.combine(y, h))
    assert np.array_equal(out[:, :2], np.array(g["combine"]["out"], np.float32))
    assert np.array_equal(out[:, 2:], np.tile(out[:, :2], (1, 3)))
    # both backward calls (grad_out[t] = [1, 2] repeated)
    bw = g["backward"]
    gx = f32(ep.dispatch_backward(y, h))
    assert np.array_equal(gx[:, :2], np.array(bw["dispatch_backward"], np.float32))
    go = torch.tensor([[1.0, 2.0] * 4] * T, dtype=torch.float32, device=dev).to(torch.bfloat16)
    gy, gw = ep.combine_backward(go, h, y=y)
    assert np.array_equal(f32(gy)[:9, :2], np.array(bw["grad_y"], np.float32))
    assert np.array_equal(gw.cpu().numpy(), 4 * np.array(bw["grad_w"], np.float32))   # 4 channel pairs
    # capacity 6: drops and overflow
    lay6 = ep.get_dispatch_layout(t_idx, E, P)
    _, _, h6 = ep.dispatch(x, w, lay6, False, capacity_rows=6)
    assert h6.slot.tolist() == g["capacity_6"]["slot"]
    assert ep.handle_recv_counts(h6)[2] == ep.EP_ECAPACITY
    # aligned layout, A = 2
    lay2 = ep.get_dispatch_layout(t_idx, E, P, expert_alignment=2)
    _, _, h2 = ep.dispatch(x, w, lay2, False)
    assert h2.expert_offset.tolist() == g["aligned_2"]["expert_offset"]
    assert h2.slot.tolist() == g["aligned_2"]["slot"]
    # static low-latency layout, 2 rows per expert
    _, _, lls = ep.low_latency_dispatch(x, t_idx, w, E, P, 2, False)
    assert lls.handle.slot.tolist() == g["static_cap_2"]["slot"]
    assert ep.handle_recv_counts(lls.handle)[2] == ep.EP_ECAPACITY
    # FP8 combine: two blocks, scales 0.5 and 0.25
    c8 = g["combine_fp8"]
    codes = torch.tensor([int(c, 16) for c in c8["row_codes"]], dtype=torch.uint8, device=dev)
    q = codes[:, None].repeat(1, 256)
    q = torch.cat([q, torch.zeros((6, 256), dtype=torch.uint8, device=dev)])        # 15 rows
    sc = torch.tensor(c8["scales"], dtype=torch.float32, device=dev).repeat(15, 1)
    lay8 = ep.get_dispatch_layout(t_idx, E, P)
    _, _, h8 = ep.dispatch(torch.zeros((T, 256), dtype=torch.bfloat16, device=dev), w, lay8, True,
                           capacity_rows=15)
    assert h8.slot.tolist() == g["slot"]
    for wts, key in ((w, "out_weighted"), (None, "out_unit")):
        o = f32(ep.combine_fp8(q, sc, h8, wts) if wts is not None else ep.dispatch_backward_fp8(q, sc, h8))
        want = np.repeat(np.array(c8[key], np.float32), 128, axis=1)
        assert np.array_equal(o, want), key

    # the expert-parallel flow on its own worked example
    ge = json.load(open(os.path.join(gdir, "ep_worked_example.json")))
    we = torch.tensor(ge["topk_weights"], dtype=torch.float32, device=dev)
    send_x, _, li, lw, play, part = ep.pack_for_ranks(x, t_idx, we, E, P, use_fp8=False)
    assert part.tolist() == ge["part_idx"]
    assert play.handle.slot.tolist() == ge["pack_slot"]
    rows = sum(ge["pack_rows_per_destination"])
    assert li[:rows].tolist() == ge["local_idx"]
    assert np.array_equal(lw[:rows].cpu().numpy(), np.array(ge["local_w"], np.float32))
    off = np.concatenate([[0], np.cumsum(ge["pack_rows_per_destination"])])
    partial = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    for p in range(P):
        r0, r1 = int(off[p]), int(off[p + 1])
        ul = ep.get_dispatch_layout(li[r0:r1], E // P, 1)
        _, _, uh = ep.dispatch(send_x[r0:r1], lw[r0:r1], ul, False)
        assert uh.slot.tolist() == ge["unpack_slot"][p], p
        n = ge["expert_outputs"]["rows_per_destination"][p]
        yp = torch.tensor([[10 * p + u + 1, -(10 * p + u + 1)] * 4 for u in range(n)],
                          dtype=torch.float32, device=dev).to(torch.bfloat16)
        ep.combine(yp, uh, out=partial[r0:r1])
    assert np.array_equal(f32(partial)[:, :2], np.array(ge["partials"], np.float32))
    out_ep = f32(ep.dispatch_backward(partial, play.handle))
    assert np.array_equal(out_ep[:, :2], np.array(ge["out"], np.float32))


def test_nothing_dispatched_still_needs_a_row_buffer(ep):
    """Every id masked: N = 0 rows, capacity T*K.  combine gives +0 rows from
    a receive buffer of any size; an empty (NULL) buffer is refused with a
    message, since the host cannot know N without a sync."""
    dev = _dev()
    T, K, E, P, H = 3, 2, 8, 2, 64
    t_idx = torch.full((T, K), -1, dtype=torch.int64, device=dev)
    lay = ep.get_dispatch_layout(t_idx, E, P)
    x = torch.randn((T, H), device=dev).to(torch.bfloat16)
    _, _, h = ep.dispatch(x, torch.ones((T, K), device=dev), lay, False)
    assert ep.handle_recv_counts(h)[1] == 0
    out = ep.combine(torch.zeros((1, H), dtype=torch.bfloat16, device=dev), h)
    torch.cuda.synchronize()
    assert not _bits(out).any()
    with pytest.raises(ep.EpError, match="also when no pair was dispatched"):
        ep.combine(torch.empty((0, H), dtype=torch.bfloat16, device=dev), h)


def test_library_loaded_before_torch():
    """Loading the library before the caller imports torch still gives one
    HIP runtime (load() imports torch first): a small forward in a child
    process that does exactly that."""
    import os
    import subprocess
    import sys
    _dev()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import combine_get_dispatch_scan_amd as ep\n"
        "ep.load()\n"
        "import torch\n"
        "d = torch.device('cuda:0')\n"
        "lay = ep.get_dispatch_layout(torch.randint(0, 16, (40, 2), device=d), 16, 4)\n"
        "recv, sc, h = ep.dispatch(torch.ones((40, 128), device=d).to(torch.bfloat16), None, lay, True)\n"
        "print('N', ep.handle_recv_counts(h)[1])\n" % root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "N " in r.stdout


@pytest.mark.parametrize("T,H,K,E,P,fp8,dirty", [(1, 128, 1, 1, 1, False, False),
                                                 (3000, 512, 16, 1024, 64, True, True),
                                                 (257, 256, 8, 32, 4, False, True),
                                                 (1500, 2048, 8, 256, 8, True, False)])
def test_graph_capture_of_every_call(ep, T, H, K, E, P, fp8, dirty):
    """layout, dispatch, the asynchronous count readback (a copy node),
    combine and both backward calls captured once in one HIP graph, then
    replayed on three new batches with eager work between the replays; every
    replay against the oracle."""
    dev = _dev()
    cap = T * K
    s_idx = torch.empty((T, K), dtype=torch.int64, device=dev)
    s_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    s_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    s_y = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    s_g = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ep.ep_workspace_bytes(T, K, E, P), dtype=torch.uint8, device=dev)
    ntpp = torch.empty(P, dtype=torch.int32, device=dev)
    ntpe = torch.empty(E, dtype=torch.int32, device=dev)
    itip = torch.empty((T, P), dtype=torch.uint8, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    recv = torch.empty((cap, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    sc = torch.empty((cap, H // 128), dtype=torch.float32, device=dev) if fp8 else None
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    gx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    gy = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((T, K), dtype=torch.float32, device=dev)
    host = torch.empty(E + 5, dtype=torch.int32, pin_memory=True)
    h = ep.ep_handle_t()
    p = lambda t: None if t is None else t.data_ptr()

    def step():
        s = ep._stream()
        assert ep.ep_get_dispatch_layout(p(s_idx), T, K, E, P, p(ntpp), p(ntpe), p(itip), p(ninv),
                                         p(ws), ws.numel(), h, s) == ep.EP_OK
        assert ep.ep_dispatch(p(s_x), p(s_w), H, int(fp8), p(recv), p(sc), cap, h, s) == ep.EP_OK
        assert ep.ep_handle_recv_counts_async(h, host.data_ptr(), s) == ep.EP_OK
        assert ep.ep_combine(p(s_y), h, None, p(out), s) == ep.EP_OK
        assert ep.ep_dispatch_backward(p(s_y), h, p(gx), s) == ep.EP_OK
        assert ep.ep_combine_backward(p(s_g), p(s_y), h, None, p(gy), p(gw), s) == ep.EP_OK

    kw = dict(distinct=K <= E and not dirty)
    if dirty:
        kw.update(mask_frac=0.1, invalid_frac=0.03, dup_frac=0.05)
    cases = []
    for r in range(4):
        idx, w = workloads.random_case(700 + 10 * r + T % 7, T, E, K, **kw)
        cases.append((idx, w, workloads.random_rows(710 + r, T, H, "normal"),
                      workloads.random_rows(720 + r, cap, H, "normal"),
                      workloads.random_rows(730 + r, T, H, "normal")))

    def load(c):
        s_idx.copy_(torch.from_numpy(c[0]))
        s_w.copy_(torch.from_numpy(c[1]))
        s_x.copy_(_bf16_tensor(c[2], dev))
        s_y.copy_(_bf16_tensor(c[3], dev))
        s_g.copy_(_bf16_tensor(c[4], dev))

    load(cases[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                        # warm-up outside capture
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
        idx, w, x, y, go = c
        ref = oracle.run_all(idx, w, x, E, P, fp8)
        rows = ref["rows"]
        assert np.array_equal(np.diff(host.numpy()[:E + 1]), ref["num_tokens_per_expert"])
        assert np.array_equal(ntpe.cpu().numpy(), ref["num_tokens_per_expert"])
        got = recv.view(torch.uint8).cpu().numpy() if fp8 else _bits(recv)
        assert np.array_equal(got[:rows], ref["recv_x"])
        assert np.array_equal(_bits(out), oracle.combine(y[:rows], ref["slot"], w))
        assert np.array_equal(_bits(gx), oracle.dispatch_backward(y[:rows], ref["slot"]))
        ref_gy, _ = oracle.combine_backward(go, y[:rows], ref["slot"], w, cap)
        assert np.array_equal(_bits(gy)[:rows], ref_gy[:rows])
        del junk
