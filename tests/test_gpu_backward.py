"""GPU parity of the backward calls against the CPU oracle.

grad_x and grad_y are bit-exact (same fp32 operations); grad_w is an fp32
dot product reduced in a fixed order on the GPU and in double by the oracle,
so it is compared within the bound that order implies:
|gpu - exact| <= gamma_d * sum_j |g_j y_j| (d the reduction depth)  (+ the oracle's own
rounding to fp32), and it must be bit-identical from run to run."""
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


def _forward(ep, idx, w, x, E, P, fp8, cap=None):
    dev = _dev()
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), E, P)
    recv, sc, h = ep.dispatch(_bf16(x, dev), torch.from_numpy(w).to(dev), lay, fp8, capacity_rows=cap)
    return h


def _check_grad_w(got, ref_exact_f32, g, y, slot, H):
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
            tol = grad_w_rel_bound(H) * mag + 2.0 ** -24 * abs(float(ref_exact_f32[t, k])) + 1e-38
            assert abs(float(got[t, k]) - float(ref_exact_f32[t, k])) <= tol, (t, k, got[t, k], ref_exact_f32[t, k])


CASES = [
    ("tiny", None),
    ("skewed", None),
    ("decode", None),
    ("v3", None),
    ("large", None),
]


def _check_grad_w_all(got, ref, g, y, slot, H, chunk=256):
    """grad_w on every pair, vectorised over chunks of tokens: within
    gamma_d * sum_j |g_j y_j| of the oracle's (exactly rounded) dot product,
    plus half an fp32 ulp of it; 0 for pairs that were not dispatched.  The
    magnitude sum is taken in fp32 (relative error < H * 2^-24), so the bound
    is widened by 1%."""
    T, K = slot.shape
    valid = slot >= 0
    assert np.all(got[~valid] == 0.0)
    gabs = np.abs(workloads.f32_from_bf16_bits(g))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        s = slot[t0:t1]
        ya = np.abs(workloads.f32_from_bf16_bits(y[np.maximum(s, 0)]))       # [c, K, H]
        mag = np.einsum("tj,tkj->tk", gabs[t0:t1], ya, dtype=np.float32).astype(np.float64)
        r = ref[t0:t1].astype(np.float64)
        tol = grad_w_rel_bound(H) * mag * 1.01 + 2.0 ** -24 * np.abs(r) + 1e-38
        err = np.abs(got[t0:t1].astype(np.float64) - r)
        bad = valid[t0:t1] & (err > tol)
        assert not bad.any(), (t0 + np.argwhere(bad)[:4, 0], err[bad][:4], tol[bad][:4])


@pytest.mark.parametrize("name,cap", CASES)
def test_dispatch_backward_matches_oracle(ep, name, cap):
    dev = _dev()
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    print(f"[bwd] dispatch_backward {name}", flush=True)
    ref = oracle.run_all(idx, w, None, wl.E, wl.P, wl.use_fp8)
    h = _forward(ep, idx, w, x, wl.E, wl.P, wl.use_fp8)
    g = workloads.random_rows(17, wl.T * wl.K, wl.H, "normal")
    gx = ep.dispatch_backward(_bf16(g, dev), h)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(gx), oracle.dispatch_backward(g[:ref["rows"]], ref["slot"]))


@pytest.mark.parametrize("name", ["tiny", "skewed", "decode", "v3", "large"])
def test_combine_backward_matches_oracle(ep, name):
    dev = _dev()
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    print(f"[bwd] combine_backward {name}", flush=True)
    ref = oracle.run_all(idx, w, None, wl.E, wl.P, wl.use_fp8)
    rows = ref["rows"]
    h = _forward(ep, idx, w, x, wl.E, wl.P, wl.use_fp8)
    cap = wl.T * wl.K
    y = workloads.random_rows(18, cap, wl.H, "normal")
    g = workloads.random_rows(19, wl.T, wl.H, "normal")
    t_y, t_g = _bf16(y, dev), _bf16(g, dev)
    gy_t = torch.full((cap, wl.H), 0x7777, dtype=torch.int16, device=dev).view(torch.bfloat16)
    gy, gw = ep.combine_backward(t_g, h, y=t_y, grad_y=gy_t)
    ref_gy, ref_gw = oracle.combine_backward(g, y[:rows], ref["slot"], w, cap, fill=0x7777)
    assert np.array_equal(_bits(gy), ref_gy)
    del gy_t, gy
    gy2, gw2 = ep.combine_backward(t_g, h, y=t_y)
    assert np.array_equal(_bits(gy2)[:rows], ref_gy[:rows])
    del gy2
    gy3, gw3 = ep.combine_backward(t_g, h)          # grad_y only (segmented launch)
    assert np.array_equal(_bits(gy3)[:rows], ref_gy[:rows])
    assert gw3 is None
    del gy3, ref_gy
    got = gw.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), gw2.cpu().numpy().view(np.uint32))   # deterministic
    _check_grad_w_all(got, ref_gw, g, y, ref["slot"], wl.H)


def test_backward_with_masks_and_capacity(ep):
    dev = _dev()
    T, H, E, K, P = 300, 1024, 32, 6, 8
    idx, w = workloads.random_case(61, T, E, K, mask_frac=0.15, invalid_frac=0.05, dup_frac=0.05,
                                   distinct=False)
    x = workloads.random_rows(62, T, H, "normal")
    N = int(oracle.layout(idx, E, P)["valid"].sum())
    for cap in (T * K, N - 11):
        ref = oracle.run_all(idx, w, None, E, P, False, capacity=cap)
        h = _forward(ep, idx, w, x, E, P, False, cap=cap)
        y = workloads.random_rows(63, cap, H, "wide")
        g = workloads.random_rows(64, T, H, "wide")
        gr = workloads.random_rows(65, cap, H, "normal")
        gx = ep.dispatch_backward(_bf16(gr, dev), h)
        gy, gw = ep.combine_backward(_bf16(g, dev), h, y=_bf16(y, dev))
        torch.cuda.synchronize()
        assert np.array_equal(_bits(gx), oracle.dispatch_backward(gr, ref["slot"]))
        ref_gy, ref_gw = oracle.combine_backward(g, y, ref["slot"], w, cap)
        used = np.zeros(cap, bool)
        used[ref["slot"][ref["slot"] >= 0]] = True
        assert np.array_equal(_bits(gy)[used], ref_gy[used])
        _check_grad_w(gw.cpu().numpy(), ref_gw, g, y, ref["slot"], H)


@pytest.mark.parametrize("T,H,E,K,P,fp8", [
    (0, 256, 16, 4, 4, True),            # no tokens
    (1, 8, 4, 1, 1, False),              # the smallest row, one expert per token
    (5, 32768, 8, 4, 2, True),           # the largest hidden size
    (133, 776, 1024, 16, 64, False),     # K = 16 over 1024 experts in 64 partitions, H off the 512 step
    (257, 4224, 64, 6, 8, True),         # a ragged token tail, H off the 1024-channel FP8 step
])
def test_backward_at_the_boundary_limits(ep, T, H, E, K, P, fp8):
    """Both backward calls (and the FP8 dispatch backward) at the extremes the
    boundary accepts, with masked, out-of-range and repeated ids: grad_x and
    grad_y bit-exact, grad_w within the fp32 bound."""
    dev = _dev()
    idx, w = workloads.random_case(900 + T + H, T, E, K, distinct=False, mask_frac=0.1,
                                   invalid_frac=0.03, dup_frac=0.05)
    x = workloads.random_rows(901 + T, T, H, "normal")
    print(f"[bwd] limits T={T} H={H} E={E} K={K} P={P} fp8={fp8}", flush=True)
    ref = oracle.run_all(idx, w, None, E, P, fp8)
    rows = ref["rows"]
    h = _forward(ep, idx, w, x, E, P, fp8)
    cap = T * K
    gr = workloads.random_rows(902 + T, cap, H, "normal")
    y = workloads.random_rows(903 + T, cap, H, "normal")
    g = workloads.random_rows(904 + T, T, H, "normal")
    gx = ep.dispatch_backward(_bf16(gr, dev), h)
    gy, gw = ep.combine_backward(_bf16(g, dev), h, y=_bf16(y, dev))
    torch.cuda.synchronize()
    assert gx.shape == (T, H) and gy.shape == (cap, H) and gw.shape == (T, K)
    assert np.array_equal(_bits(gx), oracle.dispatch_backward(gr[:rows], ref["slot"]))
    ref_gy, ref_gw = oracle.combine_backward(g, y[:rows], ref["slot"], w, cap)
    assert np.array_equal(_bits(gy)[:rows], ref_gy[:rows])
    _check_grad_w_all(gw.cpu().numpy(), ref_gw, g, y, ref["slot"], H)
    if fp8 and T > 0:
        # FP8 dispatch backward on E4M3FN rows (random finite codes) with
        # random positive block scales, unit weights, against the oracle
        rng = np.random.default_rng(905 + T)
        q = rng.integers(0, 256, (rows, H), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] ^= 1                       # no NaN codes
        sc = np.ldexp(rng.random((rows, H // 128)) + 0.5, rng.integers(-20, 20, (rows, H // 128)))
        sc = sc.astype(np.float32)
        t_q, t_s = torch.from_numpy(q).to(dev), torch.from_numpy(sc).to(dev)
        gx8 = ep.dispatch_backward_fp8(t_q, t_s, h)
        out8 = ep.combine_fp8(t_q, t_s, h)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(gx8), oracle.combine_fp8(q, sc, ref["slot"], None))
        assert np.array_equal(_bits(out8), oracle.combine_fp8(q, sc, ref["slot"], w))
