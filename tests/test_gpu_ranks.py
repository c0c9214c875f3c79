"""GPU parity of the expert-parallel flow over P ranks, one rank's share,
against the CPU oracle, through the C ABI: the destination routing, the
packed rows and their metadata (the sender), the expert-contiguous layout of
the received rows (the receiver), the expert rank's pre-reduction and the
origin's sum in rank order.  The exchange between ranks is the identity:
destination p receives the packed block p.  Everything is integer work or the
same fp32 operations as the oracle, so the bar is bit-exact."""
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


def _rows(t, fp8):
    return t.view(torch.uint8).cpu().numpy() if fp8 else _bits(t)


@pytest.mark.parametrize("mode", ["clean", "dirty"])
@pytest.mark.parametrize("T,H,E,K,P", [(50, 256, 16, 4, 4), (300, 1024, 64, 6, 8), (64, 512, 256, 8, 8),
                                       (33, 256, 8, 16, 2), (40, 128, 64, 3, 64), (0, 128, 16, 4, 4)])
def test_sender_matches_the_oracle(ep, T, H, E, K, P, mode):
    dev = _dev()
    kw = {} if mode == "clean" else dict(distinct=False, mask_frac=0.15, invalid_frac=0.05, dup_frac=0.1)
    idx, w = workloads.random_case(T + E + K, T, E, K, **kw)
    x = workloads.random_rows(T + 3, T, H, "wide")
    print(f"[ranks] sender T={T} H={H} E={E} K={K} P={P} {mode}", flush=True)
    ref = oracle.ep_one_source(idx, w, x, E, P, True)
    if T == 0:
        part = ep.rank_routing(torch.from_numpy(idx).to(dev), E, P)
        assert part.shape == (0, min(K, P))
        return
    send_x, send_sc, li, lw, lay, part = ep.pack_for_ranks(_bf16(x, dev), torch.from_numpy(idx).to(dev),
                                                          torch.from_numpy(w).to(dev), E, P, True)
    torch.cuda.synchronize()
    assert np.array_equal(part.cpu().numpy(), ref["part_idx"])
    pk = ref["pack"]
    rows = pk["rows"]
    assert np.array_equal(lay.handle.slot.cpu().numpy(), pk["slot"])
    assert np.array_equal(lay.num_tokens_per_expert.cpu().numpy(), pk["num_tokens_per_expert"])
    assert np.array_equal(send_x[:rows].view(torch.uint8).cpu().numpy(), pk["recv_x"])
    assert np.array_equal(send_sc[:rows].cpu().numpy().view(np.uint32), pk["recv_scales"].view(np.uint32))
    assert np.array_equal(li[:rows].cpu().numpy(), ref["local_idx"])
    assert np.array_equal(lw[:rows].cpu().numpy().view(np.uint32), ref["local_w"].view(np.uint32))
    assert np.all(li[rows:].cpu().numpy() == -1)              # rows past the last block: untouched


def _flow(ep, wl_or_case, use_fp8, seed):
    """The whole one-rank flow on the GPU and in the oracle; returns both."""
    dev = _dev()
    idx, w, x, E, P = wl_or_case
    T, K = idx.shape
    H = x.shape[1]
    epp = E // P
    send_x, send_sc, li, lw, lay, part = ep.pack_for_ranks(_bf16(x, dev), torch.from_numpy(idx).to(dev),
                                                          torch.from_numpy(w).to(dev), E, P, use_fp8)
    counts, n, st = ep.handle_recv_counts(lay.handle)
    assert st == ep.EP_OK
    off = np.concatenate([[0], np.cumsum(counts)])
    partials = torch.empty((max(lay.handle.c.capacity_rows, 1), H), dtype=torch.bfloat16, device=dev)
    got = []
    y_parts = []
    for p in range(P):
        r0, r1 = int(off[p]), int(off[p + 1])
        lay_p = ep.get_dispatch_layout(li[r0:r1], epp, 1)
        if use_fp8:
            recv, sc, h = ep.dispatch(send_x[r0:r1], lw[r0:r1], lay_p, True, x_scales=send_sc[r0:r1])
        else:
            recv, sc, h = ep.dispatch(send_x[r0:r1], lw[r0:r1], lay_p, False)
        _, n_p, st_p = ep.handle_recv_counts(h)
        y = workloads.random_rows(seed + p, max(n_p, 1), H, "normal")[:n_p]
        y_parts.append(y)
        if r1 > r0:
            ep.combine(_bf16(y, dev) if n_p else torch.empty((0, H), dtype=torch.bfloat16, device=dev),
                       h, out=partials[r0:r1])
        got.append(dict(slot=h.slot.cpu().numpy(), rows=_rows(recv[:n_p], use_fp8),
                        scales=sc[:n_p].cpu().numpy() if use_fp8 else None, n=n_p, status=st_p))
    out = ep.dispatch_backward(partials, lay.handle)
    torch.cuda.synchronize()
    ref = oracle.ep_one_source(idx, w, x, E, P, use_fp8, y_parts=y_parts)
    return got, _bits(partials[:n]), _bits(out), ref


@pytest.mark.parametrize("name", ["tiny", "skewed", "decode", "v3", "large"])
def test_flow_matches_the_oracle(ep, name):
    """Pack -> (identity exchange) -> unpack per destination -> pre-reduce with
    the received weights -> origin sum in rank order, each stage bit-exact."""
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    print(f"[ranks] flow {name}", flush=True)
    got, partials, out, ref = _flow(ep, (idx, w, x, wl.E, wl.P), wl.use_fp8, 7000)
    for p, (g, d) in enumerate(zip(got, ref["dest"])):
        u = d["unpack"]
        assert g["n"] == u["rows"], p
        assert np.array_equal(g["slot"], u["slot"]), p
        assert np.array_equal(g["rows"], u["recv_x"][:u["rows"]]), p
        if wl.use_fp8:
            assert np.array_equal(g["scales"].view(np.uint32), u["recv_scales"][:u["rows"]].view(np.uint32)), p
    assert np.array_equal(partials, ref["partials"])
    assert np.array_equal(out, ref["out"])


def test_flow_with_dirty_routing(ep):
    """Masked, out-of-range and repeated ids, K > P (a token can reach every
    rank), BF16 rows."""
    T, H, E, K, P = 257, 512, 32, 16, 4
    idx, w = workloads.random_case(611, T, E, K, distinct=False, mask_frac=0.1, invalid_frac=0.05, dup_frac=0.1)
    x = workloads.random_rows(612, T, H, "wide")
    got, partials, out, ref = _flow(ep, (idx, w, x, E, P), False, 8000)
    assert np.array_equal(partials, ref["partials"])
    assert np.array_equal(out, ref["out"])
    for p, (g, d) in enumerate(zip(got, ref["dest"])):
        assert np.array_equal(g["slot"], d["unpack"]["slot"]), p


def test_pack_metadata_validates_its_handle(ep):
    dev = _dev()
    idx, w = workloads.random_case(5, 20, 16, 4)
    t_idx = torch.from_numpy(idx).to(dev)
    part = ep.rank_routing(t_idx, 16, 4)
    lay = ep.get_dispatch_layout(t_idx, 16, 4)           # routed by expert, not by destination
    x = _bf16(workloads.random_rows(6, 20, 256, "normal"), dev)
    ep.dispatch(x, torch.from_numpy(w).to(dev), lay, True)
    buf_i = torch.empty((80, 4), dtype=torch.int64, device=dev)
    buf_w = torch.empty((80, 4), dtype=torch.float32, device=dev)
    rc = ep.ep_pack_metadata(t_idx.data_ptr(), torch.from_numpy(w).to(dev).data_ptr(), 4, 16, part.data_ptr(),
                             lay.handle.c, buf_i.data_ptr(), buf_w.data_ptr(), ep._stream())
    assert rc == ep.EP_EINVAL and "destinations" in ep.ep_last_error()
