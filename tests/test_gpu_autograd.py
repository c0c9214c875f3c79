"""GPU checks of the autograd wrappers: the gradients that reach x, y and the
weights are the oracle's backward of dispatch and combine (grad_x, grad_y bit
for bit; grad_w within the bound of its fp32 reduction order), and a
two-layer chain dispatch -> expert -> combine backpropagates end to end."""
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
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_dispatch_and_combine_gradients(ep):
    import combine_get_dispatch_scan_amd.autograd as A
    dev = _dev()
    T, H, E, K, P = 300, 512, 32, 4, 4
    idx, w = workloads.random_case(41, T, E, K, mask_frac=0.05)
    x_bits = workloads.random_rows(42, T, H)
    x = _bf16(x_bits, dev).requires_grad_(True)
    t_w = torch.from_numpy(w).to(dev).requires_grad_(True)
    recv, handle = A.dispatch(x, torch.from_numpy(idx).to(dev), t_w, E, P)
    ref = oracle.run_all(idx, w, x_bits, E, P, False)
    slot, rows = ref["slot"], ref["rows"]
    assert np.array_equal(_bits(recv)[:rows], ref["recv_x"])
    # backward of dispatch
    g_recv = workloads.random_rows(43, recv.shape[0], H)
    recv.backward(_bf16(g_recv, dev))
    assert np.array_equal(_bits(x.grad), oracle.dispatch_backward(g_recv, slot))
    # combine of independent expert outputs, gradients for y and the weights
    y_bits = workloads.random_rows(44, recv.shape[0], H)
    y = _bf16(y_bits, dev).requires_grad_(True)
    out = A.combine(y, handle, t_w)
    assert np.array_equal(_bits(out), oracle.combine(y_bits, slot, w))
    g_out = workloads.random_rows(45, T, H)
    out.backward(_bf16(g_out, dev))
    want_gy, want_gw = oracle.combine_backward(g_out, y_bits, slot, w, recv.shape[0], fill=0)
    assert np.array_equal(_bits(y.grad), want_gy)
    gw = t_w.grad.cpu().numpy()
    gf = workloads.f32_from_bf16_bits(g_out).astype(np.float64)
    yf = workloads.f32_from_bf16_bits(y_bits).astype(np.float64)
    for t in range(T):
        for k in range(K):
            s = slot[t, k]
            if s < 0:
                assert gw[t, k] == 0.0
                continue
            tol = grad_w_rel_bound(H) * np.abs(gf[t] * yf[s]).sum() + 2.0 ** -24 * abs(want_gw[t, k])
            assert abs(gw[t, k] - want_gw[t, k]) <= tol + 1e-38


def test_chain_through_an_expert(ep):
    """x -> dispatch -> (row scale, a stand-in expert) -> combine -> loss;
    x.grad equals the oracle's chain of the two backward definitions."""
    import combine_get_dispatch_scan_amd.autograd as A
    dev = _dev()
    T, H, E, K, P = 200, 256, 16, 2, 2
    idx, w = workloads.random_case(51, T, E, K)
    x_bits = workloads.random_rows(52, T, H)
    x = _bf16(x_bits, dev).requires_grad_(True)
    recv, handle = A.dispatch(x, torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev), E, P)
    y = recv * 2                                           # exact in bf16
    out = A.combine(y, handle)                             # weights from dispatch's copy
    g_out = workloads.random_rows(53, T, H)
    out.backward(_bf16(g_out, dev))
    ref = oracle.run_all(idx, w, x_bits, E, P, False)
    rows = recv.shape[0]
    gy, _ = oracle.combine_backward(g_out, None, ref["slot"], w, rows, fill=0)
    # d(2 * recv) / d recv: doubling bf16 values is exact
    g_recv = workloads.bf16_bits_from_f32(2 * workloads.f32_from_bf16_bits(gy))
    assert np.array_equal(_bits(x.grad), oracle.dispatch_backward(g_recv, ref["slot"]))


@pytest.mark.parametrize("read_counts", [True, False])
def test_combine_gradient_rows_no_pair_maps_to_are_zero(ep, read_counts):
    """With the pair count read on the host, the combine backward zeroes only
    the rows past it; without, every row first.  Either way the rows no pair
    maps to get a zero gradient and the others the oracle's."""
    import combine_get_dispatch_scan_amd.autograd as A
    dev = _dev()
    T, H, E, K, P = 200, 256, 16, 4, 4
    idx, w = workloads.random_case(51, T, E, K, mask_frac=0.2)
    x_bits = workloads.random_rows(52, T, H)
    t_w = torch.from_numpy(w).to(dev)
    recv, handle = A.dispatch(_bf16(x_bits, dev), torch.from_numpy(idx).to(dev), t_w, E, P)
    ref = oracle.run_all(idx, w, x_bits, E, P, False)
    assert ref["N"] < recv.shape[0]              # masked pairs leave rows past N
    if read_counts:
        _, n, _ = ep.handle_recv_counts(handle)
        assert n == ref["N"] and handle.num_recv == n
    # rows past N hold leftovers in the allocator's memory: fill them first
    y_bits = workloads.random_rows(53, recv.shape[0], H)
    y = _bf16(y_bits, dev).requires_grad_(True)
    out = A.combine(y, handle, None)
    g_out = workloads.random_rows(54, T, H)
    torch.empty_like(y).fill_(7.0)               # dirty the caching allocator's block
    out.backward(_bf16(g_out, dev))
    want_gy, _ = oracle.combine_backward(g_out, y_bits, ref["slot"], w, recv.shape[0], fill=0)
    assert np.array_equal(_bits(y.grad), want_gy)
    assert not _bits(y.grad)[ref["N"]:].any()
