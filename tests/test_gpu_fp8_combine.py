"""GPU parity of combine / backward of dispatch on FP8 rows (the dequantising
option) against the CPU oracle, through the C-ABI.

Each gathered element is decode(q) * scale in one fp32 multiply, then the
same fp32 fma chain as combine, so results are expected bit-exact (the
tolerance allows 1 BF16 ulp).  Cases: the FP8 round trip on the decode and
V3 workloads (rows and scales straight from dispatch), every finite code
with random scales, ragged hidden sizes, masked tokens and capacity drops."""
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


def _ulp(a, b):
    def o(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(o(a) - o(b))


def _codes(rng, shape):
    q = rng.integers(0, 256, shape, dtype=np.uint32).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01          # no NaN codes (outside the contract)
    return q


@pytest.mark.parametrize("name", ["decode", "v3", "large"])
def test_round_trip_from_dispatch(ep, name):
    """dispatch (FP8) -> combine_fp8 (weights) and dispatch_backward_fp8 (unit)
    on the rows and scales dispatch produced."""
    dev = _dev()
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), wl.E, wl.P)
    recv, sc, h = ep.dispatch(_bf16(x, dev), torch.from_numpy(w).to(dev), lay, True)
    out = ep.combine_fp8(recv, sc, h)
    gx = ep.dispatch_backward_fp8(recv, sc, h)
    slot = h.slot.cpu().numpy()
    q = recv.view(torch.uint8).cpu().numpy()
    s = sc.cpu().numpy()
    ref = oracle.combine_fp8(q, s, slot, w)            # every token, at full size
    ref_u = oracle.combine_fp8(q, s, slot, None)
    got, got_u = _bits(out), _bits(gx)
    assert _ulp(got, ref).max() <= 1 and _ulp(got_u, ref_u).max() <= 1
    assert np.array_equal(got, ref), "expected bit-exact (same fp32 operations)"
    assert np.array_equal(got_u, ref_u)


@pytest.mark.parametrize("T,H,K,E,mask", [(64, 128, 1, 8, 0.0), (100, 1152, 6, 32, 0.1),
                                          (37, 7168, 8, 256, 0.2), (256, 2048, 16, 64, 0.05),
                                          (4, 32768, 4, 8, 0.0)])
def test_every_code_random_scales(ep, T, H, K, E, mask):
    dev = _dev()
    idx, w = workloads.random_case(400 + T, T, E, K, mask_frac=mask)
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), E, max(1, E // 8))
    x = workloads.random_rows(401 + T, T, H)
    _, _, h = ep.dispatch(_bf16(x, dev), torch.from_numpy(w).to(dev), lay, False)
    rows = h.c.capacity_rows
    rng = np.random.default_rng(T * 7 + H)
    q = _codes(rng, (rows, H))
    s = (rng.standard_normal((rows, H // 128)).astype(np.float32) *
         np.ldexp(np.float32(1), rng.integers(-30, 31, (rows, H // 128))).astype(np.float32))
    t_q = torch.from_numpy(q).to(dev).view(torch.float8_e4m3fn)
    t_s = torch.from_numpy(s).to(dev)
    slot = h.slot.cpu().numpy()
    out = ep.combine_fp8(t_q, t_s, h)
    gx = ep.dispatch_backward_fp8(t_q, t_s, h)
    assert np.array_equal(_bits(out), oracle.combine_fp8(q, s, slot, w))
    assert np.array_equal(_bits(gx), oracle.combine_fp8(q, s, slot, None))
    # explicit weights override the handle's copy
    w2 = (w * 0.5).astype(np.float32)
    out2 = ep.combine_fp8(t_q, t_s, h, torch.from_numpy(w2).to(dev))
    assert np.array_equal(_bits(out2), oracle.combine_fp8(q, s, slot, w2))


def test_capacity_drops_and_empty(ep):
    dev = _dev()
    T, H, K, E = 96, 256, 4, 8
    idx, w = workloads.random_case(77, T, E, K)
    x = workloads.random_rows(78, T, H)
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), E, 2)
    cap = 150
    recv, sc, h = ep.dispatch(_bf16(x, dev), torch.from_numpy(w).to(dev), lay, True, capacity_rows=cap)
    slot = h.slot.cpu().numpy()
    assert (slot < 0).any()
    out = ep.combine_fp8(recv, sc, h)
    ref = oracle.combine_fp8(recv.view(torch.uint8).cpu().numpy(), sc.cpu().numpy(), slot, w)
    assert np.array_equal(_bits(out), ref)
    # dropped pairs read nothing in the unit-weight form either
    gx = ep.dispatch_backward_fp8(recv, sc, h)
    ref_u = oracle.combine_fp8(recv.view(torch.uint8).cpu().numpy(), sc.cpu().numpy(), slot, None)
    assert np.array_equal(_bits(gx), ref_u)
    # T = 0: nothing to do, no error
    lay0 = ep.get_dispatch_layout(torch.empty((0, K), dtype=torch.int64, device=dev), E, 2)
    _, _, h0 = ep.dispatch(torch.empty((0, H), dtype=torch.bfloat16, device=dev), None, lay0, True)
    assert ep.dispatch_backward_fp8(recv, sc, h0).shape == (0, H)


def test_device_decoder_on_every_code(ep):
    """K = 1, w = 1, scale 1: each output is bf16(decode(q)), and every finite
    E4M3FN value is exact in bf16 -- so this checks the device's decoder on
    all 254 finite codes against the oracle's formula."""
    dev = _dev()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    H = 256
    T = 8
    q = np.resize(codes, (T, H)).astype(np.uint8)
    q[T // 2:] = q[T // 2:, ::-1]
    idx = np.arange(T, dtype=np.int64).reshape(T, 1)
    w = np.ones((T, 1), np.float32)
    lay = ep.get_dispatch_layout(torch.from_numpy(idx).to(dev), T, 1)
    x = workloads.random_rows(3, T, H)
    _, _, h = ep.dispatch(_bf16(x, dev), torch.from_numpy(w).to(dev), lay, True)
    slot = h.slot.cpu().numpy()
    rows = np.empty_like(q)
    rows[slot[:, 0]] = q                        # token t's codes sit in its receive row
    s = np.ones((T, H // 128), np.float32)
    out = ep.combine_fp8(torch.from_numpy(rows).to(dev), torch.from_numpy(s).to(dev), h)
    want = np.array([[oracle.e4m3fn_decode(int(c)) for c in r] for r in q], np.float32)
    got = workloads.f32_from_bf16_bits(_bits(out))
    assert np.array_equal(got.view(np.uint32) & 0x7FFFFFFF, want.view(np.uint32) & 0x7FFFFFFF)
    nz = want != 0                               # signs (zeros come out +0: the sum starts at +0)
    assert np.array_equal(np.signbit(got[nz]), np.signbit(want[nz]))
