"""Seeded random shapes through the paths beside the dense forward, each
against the CPU oracle: the one-launch low-latency dispatch (then combine on
its static handle), GEMM-aligned layouts (column-major scales and FP8 input
included), and the expert-parallel flow over ranks.  Bit-exact throughout."""
import numpy as np
import pytest

import oracle
import workloads
import test_gpu_gemm_layout as gl
import test_gpu_low_latency as ll
import test_gpu_ranks as rk

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _routing(rng, E_max=1024):
    P = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    E = P * int(rng.integers(1, max(1, E_max // P) + 1))
    K = int(rng.integers(1, 17))
    return E, K, P


def _ids(seed, T, E, K, dirty):
    kw = dict(distinct=K <= E and not dirty)
    if dirty:
        kw.update(mask_frac=0.1, invalid_frac=0.03, dup_frac=0.05)
    return workloads.random_case(seed, T, E, K, **kw)


def _ll_cases(n=15, seed=11):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E, K, P = _routing(rng)
        T = 0 if i == 0 else int(rng.integers(1, 257))
        fp8 = bool(rng.integers(0, 2))
        H = 128 * int(rng.integers(1, 17)) if fp8 else 8 * int(rng.integers(1, 401))
        cap = int(rng.integers(1, 65))
        out.append((i, T, H, E, K, P, fp8, bool(rng.integers(0, 2)), cap))
    return out


@pytest.mark.parametrize("case", _ll_cases(), ids=lambda c: "ll%d" % c[0])
def test_low_latency_random(ep, case):
    i, T, H, E, K, P, fp8, dirty, cap = case
    print(f"[random] low-latency {case}", flush=True)
    idx, w = _ids(9100 + i, T, E, K, dirty)
    x = workloads.random_rows(9200 + i, T, H, "normal")
    recv, sc, lay, t_w = ll._run(ep, idx, w, x, E, P, cap, fp8)
    ref = ll._check_dispatch(ep, idx, w, x, E, P, cap, fp8, recv, sc, lay)
    if T == 0:
        return
    y = workloads.random_rows(9300 + i, E * cap, H, "normal")
    out = ep.combine(ll._bf16(y, ll._dev()), lay.handle)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ll._bits(out), oracle.combine(y, ref["slot"], w))


def _aligned_cases(n=15, seed=12):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E, K, P = _routing(rng, E_max=256)
        T = int(rng.integers(1, 2001))
        fp8 = bool(rng.integers(0, 2))
        H = 128 * int(rng.integers(1, 17)) if fp8 else 8 * int(rng.integers(1, 257))
        A = int(rng.choice([2, 3, 16, 64, 128]))
        A = max(2, min(A, 1 + 32768 // E))              # at most 32768 padding rows
        col_major = fp8 and bool(rng.integers(0, 2))
        fp8_input = fp8 and bool(rng.integers(0, 2))
        out.append((i, T, H, E, K, P, fp8, bool(rng.integers(0, 2)), A, col_major, fp8_input))
    return out


@pytest.mark.parametrize("case", _aligned_cases(), ids=lambda c: "aligned%d" % c[0])
def test_aligned_layout_random(ep, case):
    i, T, H, E, K, P, fp8, dirty, A, col_major, fp8_input = case
    print(f"[random] aligned {case}", flush=True)
    idx, w = _ids(9400 + i, T, E, K, dirty)
    if fp8_input:
        rng = np.random.default_rng(9500 + i)
        xq = rng.integers(0, 256, (T, H), dtype=np.uint32).astype(np.uint8)
        xq[(xq & 0x7F) == 0x7F] ^= 1                   # finite codes only (NaN is outside the contract)
        xs = rng.standard_normal((T, H // 128)).astype(np.float32)
        lay, h, recv, sc, cap, _, _ = gl._run(ep, idx, w, xq, E, P, A, True, x_scales=xs,
                                              col_major=col_major)
        ref = oracle.run_all(idx, w, None, E, P, True, align=A)
        q, s = oracle.dispatch_fp8_input(xq, xs, ref["slot"], ref["rows"])
        ref.update(recv_x=q, recv_scales=s)
    else:
        x = workloads.random_rows(9600 + i, T, H, "normal")
        lay, h, recv, sc, cap, _, _ = gl._run(ep, idx, w, x, E, P, A, fp8, col_major=col_major)
        ref = oracle.run_all(idx, w, x, E, P, fp8, align=A)
    gl._check(ep, lay, h, recv, sc, cap, ref, fp8, col_major)
    # combine through the aligned handle: padding rows are never gathered
    y = workloads.random_rows(9700 + i, cap, H, "normal")
    out = ep.combine(gl._bf16(y, gl._dev()), h)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gl._bits(out), oracle.combine(y, ref["slot"], w))
    if fp8:
        # the FP8 rows and scales as dispatch wrote them (column-major when
        # asked), through the FP8 combine and the FP8 dispatch backward
        out8 = ep.combine_fp8(recv[:cap], sc, h)
        gx8 = ep.dispatch_backward_fp8(recv[:cap], sc, h)
        torch.cuda.synchronize()
        rows = ref["rows"]
        q = recv[:rows].cpu().numpy()
        s_rm = (sc.cpu().numpy()[:, :rows].T if col_major else sc.cpu().numpy()[:rows])
        np.testing.assert_array_equal(gl._bits(out8), oracle.combine_fp8(q, np.ascontiguousarray(s_rm), ref["slot"], w))
        np.testing.assert_array_equal(gl._bits(gx8), oracle.combine_fp8(q, np.ascontiguousarray(s_rm), ref["slot"], None))


def _ranks_cases(n=15, seed=13):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E, K, P = _routing(rng, E_max=512)
        T = int(rng.integers(1, 1501))
        fp8 = bool(rng.integers(0, 2))
        H = 128 * int(rng.integers(1, 17)) if fp8 else 8 * int(rng.integers(1, 257))
        out.append((i, T, H, E, K, P, fp8, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _ranks_cases(), ids=lambda c: "ranks%d" % c[0])
def test_rank_flow_random(ep, case):
    i, T, H, E, K, P, fp8, dirty = case
    print(f"[random] ranks {case}", flush=True)
    idx, w = _ids(9800 + i, T, E, K, dirty)
    x = workloads.random_rows(9900 + i, T, H, "normal")
    got, partials, out, ref = rk._flow(ep, (idx, w, x, E, P), fp8, 10000 + 100 * i)
    for p, (g, d) in enumerate(zip(got, ref["dest"])):
        u = d["unpack"]
        assert g["n"] == u["rows"], p
        assert np.array_equal(g["slot"], u["slot"]), p
        assert np.array_equal(g["rows"], u["recv_x"][:u["rows"]]), p
    assert np.array_equal(partials, ref["partials"])
    assert np.array_equal(out, ref["out"])


def _bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_call_sequences_on_one_handle(ep, seed):
    """Random sequences of calls on one handle, each step against the oracle:
    re-dispatch with changing capacity (0, N - 1, N, T*K, any) and payload
    mode, cached dispatch of new rows, combine, dispatch backward, and the
    asynchronous count readback.  The overflow status always belongs to the
    latest dispatch."""
    dev = ll._dev()
    bf = lambda b: ll._bf16(b, dev)
    rng = np.random.default_rng(seed)
    for case in range(10):
        P = int(rng.choice([1, 2, 4, 8, 16]))
        E = P * int(rng.integers(1, 256 // P + 1))
        K = int(rng.integers(1, 9))
        T = int(rng.integers(1, 1500))
        H = 128 * int(rng.integers(1, 9))
        idx, w = _ids(int(rng.integers(1 << 30)), T, E, K, bool(rng.integers(0, 2)))
        print(f"[random] sequence seed={seed} case={case} T={T} H={H} E={E} K={K} P={P}", flush=True)
        t_idx, t_w = torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev)
        lay = ep.get_dispatch_layout(t_idx, E, P)
        h = lay.handle
        N = oracle.run_all(idx, w, None, E, P, False)["N"]
        host_buf = torch.empty(E + 5, dtype=torch.int32, pin_memory=True)
        cur = None
        for step in range(int(rng.integers(3, 8))):
            op = "dispatch" if cur is None else str(rng.choice(
                ["dispatch", "dispatch", "cached", "combine", "backward", "counts_async"]))
            if op == "dispatch":
                fp8 = bool(rng.integers(0, 2))
                cap = int(rng.choice([T * K, N, max(0, N - 1), int(rng.integers(0, N + 1)), 0]))
                x = workloads.random_rows(int(rng.integers(1 << 30)), T, H, "normal")
                recv, sc, _ = ep.dispatch(bf(x), t_w, lay, fp8, capacity_rows=cap)
                ref = oracle.run_all(idx, w, x, E, P, fp8, capacity=cap)
                assert np.array_equal(h.slot.cpu().numpy(), ref["slot"])
                rows = ref["rows"]
                got = recv.view(torch.uint8).cpu().numpy() if fp8 else _bits16(recv)
                assert np.array_equal(got[:rows], ref["recv_x"])
                if fp8:
                    assert np.array_equal(sc[:rows].cpu().numpy().view(np.uint32), ref["recv_scales"].view(np.uint32))
                _, n, st = ep.handle_recv_counts(h)
                cur = (fp8, cap, ref)
            else:
                fp8, cap, ref = cur
                if op == "cached":
                    x2 = workloads.random_rows(int(rng.integers(1 << 30)), T, H, "normal")
                    r2, _ = ep.dispatch_cached(bf(x2), h)
                    ref2 = oracle.run_all(idx, w, x2, E, P, fp8, capacity=cap)
                    got = r2.view(torch.uint8).cpu().numpy() if fp8 else _bits16(r2)
                    assert np.array_equal(got[:ref2["rows"]], ref2["recv_x"])
                elif op == "combine":
                    y = workloads.random_rows(int(rng.integers(1 << 30)), max(cap, 1), H, "normal")
                    assert np.array_equal(_bits16(ep.combine(bf(y), h)),
                                          oracle.combine(y[:ref["rows"]], ref["slot"], w))
                elif op == "backward":
                    gr = workloads.random_rows(int(rng.integers(1 << 30)), max(cap, 1), H, "normal")
                    assert np.array_equal(_bits16(ep.dispatch_backward(bf(gr), h)),
                                          oracle.dispatch_backward(gr[:ref["rows"]], ref["slot"]))
                else:
                    ev = torch.cuda.Event()
                    ep.handle_recv_counts_async(h, host_buf)
                    ev.record()
                    ev.synchronize()
                    _, n, st = ep.recv_counts_decode(h, host_buf)
            if op in ("dispatch", "counts_async"):
                want = ep.EP_ECAPACITY if cur[2]["overflow"] else (ep.EP_EIDS if cur[2]["num_invalid"] else ep.EP_OK)
                assert st == want and n == N, (op, st, want)
