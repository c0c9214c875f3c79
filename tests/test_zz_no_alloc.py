"""The allocation-free low-latency dispatch against the workspace form, through
the C ABI: two calls in a row, the second with a smaller input, each compared
bit for bit with ep_low_latency_dispatch on the same inputs (layout outputs,
received rows and scales, slots, counts and status) and, through each
handle, with combine; and against the oracle."""
import ctypes

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


def _outputs(T, H, E, P, cap, fp8, dev):
    """Canary-filled output buffers of one low-latency dispatch."""
    rows = E * cap
    if fp8:
        recv = torch.full((rows, H), 0xA5, dtype=torch.uint8, device=dev)
        sc = torch.full((rows, H // 128), -7.0, dtype=torch.float32, device=dev)
    else:
        recv = torch.full((rows, H), 0x5A5A, dtype=torch.int16, device=dev)
        sc = None
    return dict(recv=recv, sc=sc,
                ntpp=torch.full((P,), -1, dtype=torch.int32, device=dev),
                ntpe=torch.full((E,), -1, dtype=torch.int32, device=dev),
                itip=torch.full((T, P), 0xC3, dtype=torch.uint8, device=dev),
                ninv=torch.full((1,), -1, dtype=torch.int32, device=dev))


def _call(ep, noalloc, t_x, t_idx, t_w, T, H, K, E, P, fp8, cap, o, ws=None):
    h = ep.ep_handle_t()
    p = lambda t: None if t is None else t.data_ptr()
    args = (p(t_x), p(t_idx), p(t_w), T, H, K, E, P, int(fp8), cap, p(o["recv"]), p(o["sc"]),
            p(o["ntpp"]), p(o["ntpe"]), p(o["itip"]), p(o["ninv"]))
    if noalloc:
        rc = ep.ep_low_latency_dispatch_noalloc(*args, h, ep._stream())
    else:
        rc = ep.ep_low_latency_dispatch(*args, ws.data_ptr(), ws.numel(), h, ep._stream())
    assert rc == ep.EP_OK, ep.ep_last_error()
    return h


def _status(ep, h, E):
    counts = (ctypes.c_int32 * E)()
    n = ctypes.c_int32(-1)
    rc = ep.ep_handle_recv_counts(h, counts, ctypes.byref(n), ep._stream())
    return list(counts), n.value, rc


# the decode shape first, then a smaller batch with drops (BF16)
CALLS = [(128, 7168, 8, 256, 8, True, 128, 901), (40, 1024, 4, 32, 4, False, 3, 902)]


def test_noalloc_matches_the_workspace_form_on_two_calls(ep):
    dev = _dev()
    scratch_addr = None
    for T, H, K, E, P, fp8, cap, seed in CALLS:
        print(f"[noalloc] T={T} H={H} K={K} E={E} P={P} fp8={fp8} cap={cap}", flush=True)
        idx, w = workloads.random_case(seed, T, E, K, mask_frac=0.05, invalid_frac=0.02)
        x = workloads.random_rows(seed, T, H, "wide")
        t_x, t_idx, t_w = _bf16(x, dev), torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev)
        ws = torch.empty(ep.ep_workspace_bytes(T, K, E, P), dtype=torch.uint8, device=dev)
        a, b = _outputs(T, H, E, P, cap, fp8, dev), _outputs(T, H, E, P, cap, fp8, dev)
        ha = _call(ep, False, t_x, t_idx, t_w, T, H, K, E, P, fp8, cap, a, ws)
        hb = _call(ep, True, t_x, t_idx, t_w, T, H, K, E, P, fp8, cap, b)
        # the handle's arrays live in the library's per-GPU array, at one address
        assert hb.ws is not None and hb.ws != ws.data_ptr()
        assert hb.ws_bytes == ep.EP_NOALLOC_SCRATCH_BYTES
        if scratch_addr is not None:
            assert hb.ws == scratch_addr
        scratch_addr = hb.ws
        for key in ("recv", "sc", "ntpp", "ntpe", "itip", "ninv"):
            if a[key] is not None:
                assert torch.equal(a[key], b[key]), key
        sta, stb = _status(ep, ha, E), _status(ep, hb, E)
        assert sta == stb
        # the handles route the same: a cached dispatch of new rows and a
        # combine (with the weight copy each handle holds) through each
        x2 = workloads.random_rows(seed + 2, T, H, "normal")
        a2, b2 = _outputs(T, H, E, P, cap, fp8, dev), _outputs(T, H, E, P, cap, fp8, dev)
        p = lambda t: None if t is None else t.data_ptr()
        for h, o in ((ha, a2), (hb, b2)):
            assert ep.ep_dispatch_cached(_bf16(x2, dev).data_ptr(), h, p(o["recv"]), p(o["sc"]),
                                         ep._stream()) == ep.EP_OK
        y = workloads.random_rows(seed + 1, E * cap, H, "normal")
        t_y = _bf16(y, dev)
        out_a = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        out_b = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        assert ep.ep_combine(t_y.data_ptr(), ha, None, out_a.data_ptr(), ep._stream()) == ep.EP_OK
        assert ep.ep_combine(t_y.data_ptr(), hb, None, out_b.data_ptr(), ep._stream()) == ep.EP_OK
        torch.cuda.synchronize()
        assert torch.equal(a2["recv"], b2["recv"])
        if fp8:
            assert torch.equal(a2["sc"], b2["sc"])
        assert torch.equal(out_a, out_b)
        # and the oracle
        ref = oracle.run_low_latency(idx, w, x, E, P, fp8, cap)
        slot = ref["slot"]
        assert stb[0] == list(np.minimum(ref["num_tokens_per_expert"], cap))
        assert stb[2] == (ep.EP_ECAPACITY if ref["overflow"] else
                          (ep.EP_EIDS if ref["num_invalid"] else ep.EP_OK))
        assert np.array_equal(b["itip"].cpu().numpy(), ref["is_token_in_partition"])
        assert np.array_equal(b["ntpe"].cpu().numpy(), ref["num_tokens_per_expert"])
        used = slot[slot >= 0]
        got = b["recv"].cpu().numpy()
        want = ref["recv_x"]
        assert np.array_equal(got[used] if fp8 else got[used].view(np.uint16), want[used])
        if fp8:
            assert np.array_equal(b["sc"].cpu().numpy()[used].view(np.uint32),
                                  ref["recv_scales"][used].view(np.uint32))
        assert np.array_equal(_bits(out_b), oracle.combine(y, slot, w))


def test_noalloc_rejects_oversized_batches(ep):
    """More tokens than the low-latency limit: a clear error before any HIP call."""
    h = ep.ep_handle_t()
    rc = ep.ep_low_latency_dispatch_noalloc(None, None, None, ep.EP_MAX_LL_TOKENS + 1, 128, 2, 8, 2, 0,
                                            4, None, None, None, None, None, None, h, None)
    assert rc == ep.EP_EINVAL and "at most" in ep.ep_last_error()
