"""Pins for the CPU oracle: every check compares it with something other than
itself -- torch's CPU codecs, brute-force search, a textbook stable sort,
numpy bincount / unique, hand-worked values, exact identities and error
bounds that hold for the mathematics."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(bits_u16):
    return workloads.f32_from_bf16_bits(bits_u16)


# ----------------------------------------------------------------------------
# BF16 rounding
# ----------------------------------------------------------------------------

def test_bf16_rne_matches_torch_on_random_and_ties():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]                       # finite only
    ties = (rng.integers(0, 1 << 16, 20000, dtype=np.uint32) << 16) | 0x8000
    ties = ties[((ties >> 23) & 0xFF) < 0xFE]                # stay clear of overflow
    near = np.concatenate([ties - 1, ties + 1])
    for arr in (u, ties.astype(np.uint32), near.astype(np.uint32)):
        f = arr.view(np.float32)
        ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = np.array([oracle.bf16_rne(v) for v in f[:5000]], dtype=np.uint16)
        assert np.array_equal(got, ref[:5000])


def test_bf16_widening_is_exact():
    for b in [0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4049]:
        assert np.float32(oracle.lib().oracle_bf16_to_f32(b)) == _f32(np.array([b], np.uint16))[0]


# ----------------------------------------------------------------------------
# FP8 E4M3FN codec
# ----------------------------------------------------------------------------

def _e4m3_table():
    """All 127 non-negative finite E4M3FN values, built from the bit layout."""
    vals, codes = [], []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append(v)
        codes.append(code)
    return np.array(vals), np.array(codes)


def _nearest_brute(v):
    """Nearest E4M3FN value by exhaustive search; ties to the even code;
    saturate at 448; keep the sign."""
    tv, tc = _e4m3_table()
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - tv[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates prefer an even code
    even = cand & ((tc[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    code = tc[pick].astype(np.uint8)
    code[a >= 448.0] = 0x7E
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def test_e4m3fn_hand_values():
    g = json.load(open(os.path.join(GOLDEN, "e4m3fn_values.json")))
    for v, code in g["cases"]:
        assert oracle.e4m3fn(np.float32(v)) == int(code, 16), (v, code)


def test_quant_block_hand_values():
    """Whole 128-channel blocks quantised by hand (golden/e4m3fn_values.json,
    "blocks"): the block's amax sets one inverse scale for every element."""
    g = json.load(open(os.path.join(GOLDEN, "e4m3fn_values.json")))["blocks"]
    for case in g["cases"]:
        v = np.zeros(128, np.float32)
        for j, val in case["values"].items():
            v[int(j)] = val
        codes, scale = oracle.quant_block(workloads.bf16_bits_from_f32(v))
        want = np.zeros(128, np.uint8)
        for j, c in case["codes"].items():
            want[int(j)] = int(c, 16)
        assert np.array_equal(np.asarray(codes, np.uint8), want), case
        if "scale" in case:
            assert np.float32(scale) == np.float32(case["scale"])


def test_e4m3fn_matches_brute_force_nearest():
    rng = np.random.default_rng(5)
    tv, _ = _e4m3_table()
    mids = (tv[1:] + tv[:-1]) / 2
    pts = np.concatenate([tv, mids]).astype(np.float32)
    # every value and midpoint, and the fp32 neighbours of each
    u = pts.view(np.uint32)
    around = np.concatenate([u, u + 1, np.maximum(u, 1) - 1]).view(np.float32)
    rnd = (rng.random(60000) * 500).astype(np.float32)
    tiny = (rng.random(20000) * 2 ** -5).astype(np.float32)
    v = np.concatenate([around, rnd, tiny, [464.0, 480.0, 1e30]]).astype(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.e4m3fn_array(v), _nearest_brute(v))


@pytest.mark.slow
def test_e4m3fn_exhaustive_against_torch():
    """Every fp32 bit pattern in [2^-11, 448] and its negative: the oracle's
    encoder equals torch's CPU float8_e4m3fn conversion (RNE, same format).
    Below 2^-11 both give signed zero (checked on a sample)."""
    lo = np.float32(2.0 ** -11).view(np.uint32)
    hi = np.float32(448.0).view(np.uint32)
    step = 1 << 24
    for start in range(int(lo), int(hi) + 1, step):
        u = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        for sign in (0, 0x80000000):
            v = (u | np.uint32(sign)).view(np.float32)
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            got = oracle.e4m3fn_array(v)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])
    rng = np.random.default_rng(3)
    small = rng.integers(0, int(lo), 1 << 20, dtype=np.uint64).astype(np.uint32)
    v = np.concatenate([small, small | np.uint32(0x80000000)]).view(np.float32)
    assert np.array_equal(oracle.e4m3fn_array(v), torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_e4m3fn_decode_roundtrip_and_bound():
    for code in range(256):
        if code & 0x7F == 0x7F:
            assert np.isnan(oracle.e4m3fn_decode(code))
            continue
        v = oracle.e4m3fn_decode(code)
        assert oracle.e4m3fn(v) == code
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(20000) * 40).astype(np.float32)
    v = v[np.abs(v) < 448]
    q = oracle.e4m3fn_array(v)
    dec = np.array([oracle.e4m3fn_decode(c) for c in q])
    a = np.abs(v.astype(np.float64))
    # half a quantum: 2^-4 relative in the normal range, 2^-10 absolute below 2^-6
    bound = np.where(a >= 2 ** -6, a * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(dec - v) <= bound)


# ----------------------------------------------------------------------------
# block quantisation
# ----------------------------------------------------------------------------

def _blocks(seed, kind, n=64):
    return workloads.random_rows(seed, n, 128, kind)


@pytest.mark.parametrize("kind", ["normal", "wide", "bits", "ties"])
def test_quant_block_properties(kind):
    for row in _blocks(21, kind):
        q, s = oracle.quant_block(row)
        v = _f32(row).astype(np.float64)
        amax = np.abs(v).max()
        a = max(amax, 2.0 ** -64)
        # scale is the closed form a / 448 rounded to fp32 (exact quotient
        # within half an fp32 ulp)
        assert abs(float(s) - a / 448.0) <= 2.0 ** -24 * (a / 448.0)
        # the element(s) equal to amax map to +-448 exactly
        if amax > 0:
            for i in np.nonzero(np.abs(v) == amax)[0]:
                assert q[i] & 0x7F == 0x7E
        dec = np.array([oracle.e4m3fn_decode(c) for c in q]) * float(s)
        # dequantisation error: half an E4M3 quantum of v * inv, with slack
        # 2^-20 for the fp32 roundings of inv, s and the product
        vin = np.abs(v) * (448.0 / a)
        bound = np.where(vin >= 2 ** -6, 2.0 ** -4 * np.abs(v), 2.0 ** -10 * float(s)) * (1 + 2.0 ** -20)
        assert np.all(np.abs(dec - v) <= bound + 1e-300)
        # sign kept, including zero
        assert np.all((q >> 7) == np.signbit(v).astype(np.uint8))
        # monotone: ordering of values is kept (weakly) by the codes
        order = np.argsort(v, kind="stable")
        dq = np.array([oracle.e4m3fn_decode(c) for c in q])[order]
        assert np.all(np.diff(dq) >= 0)


def test_quant_block_special_cases():
    z = workloads.bf16_bits_from_f32(np.zeros(128, np.float32))
    z[3] = 0x8000  # -0
    q, s = oracle.quant_block(z)
    assert float(s) == np.float32(2.0 ** -64) / np.float32(448.0)
    assert q[3] == 0x80 and np.all(np.delete(q, 3) == 0)
    one = np.zeros(128, np.float32)
    one[77] = -3.0
    q, s = oracle.quant_block(workloads.bf16_bits_from_f32(one))
    assert q[77] == 0xFE and np.all(np.delete(q, 77) == 0)
    assert float(s) == np.float32(3.0) / np.float32(448.0)
    # amax 224 -> inv 2 exactly, scale 0.5 exactly
    b = np.zeros(128, np.float32)
    b[0], b[1], b[2], b[3] = 224.0, 1.0, 0.001, -0.0029296875
    q, s = oracle.quant_block(workloads.bf16_bits_from_f32(b))
    assert float(s) == 0.5
    assert q[0] == 0x7E and q[1] == 0x40
    # 0.001 in bf16 is 0.00099945068..., times 2 -> 1.0*2^-9 nearest -> 0x01
    assert q[2] == 0x01
    # -0.0029296875 * 2 = -3 * 2^-9 -> 0x83
    assert q[3] == 0x83
    # bf16 subnormal inputs: a = 2^-64 and every code is a signed zero
    sub = workloads.random_rows(4, 1, 128, "subnormal")[0]
    q, s = oracle.quant_block(sub)
    assert np.all(q & 0x7F == 0)


# ----------------------------------------------------------------------------
# layout / offsets / slots
# ----------------------------------------------------------------------------

def _valid_independent(idx, E):
    """First valid occurrence of each in-range id per row, via np.unique."""
    T, K = idx.shape
    v = np.zeros((T, K), np.uint8)
    for t in range(T):
        row = idx[t]
        ok = np.nonzero((row >= 0) & (row < E))[0]
        if ok.size:
            _, first = np.unique(row[ok], return_index=True)
            v[t, ok[first]] = 1
    return v


def test_layout_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "layout_worked_example.json")))
    idx = np.array(g["topk_idx"], np.int64)
    lay = oracle.layout(idx, g["E"], g["P"])
    assert lay["num_tokens_per_expert"].tolist() == g["num_tokens_per_expert"]
    assert lay["num_tokens_per_partition"].tolist() == g["num_tokens_per_partition"]
    assert lay["is_token_in_partition"].tolist() == g["is_token_in_partition"]
    assert lay["num_invalid"] == g["num_invalid"]
    off = oracle.expert_offsets(lay["num_tokens_per_expert"])
    assert off.tolist() == g["expert_offset"]
    slot, src, ovf = oracle.slots(idx, lay["valid"], off, 15)
    assert slot.tolist() == g["slot"] and ovf == 0
    assert src[:off[-1]].tolist() == g["src_token"]
    c6 = g["capacity_6"]
    slot6, src6, ovf6 = oracle.slots(idx, lay["valid"], off, 6)
    assert slot6.tolist() == c6["slot"] and src6.tolist() == c6["src_token"] and ovf6 == c6["overflow"]
    cb = g["combine"]
    y = np.array([[r, -r] for r in range(9)], np.float32)
    out = oracle.combine(workloads.bf16_bits_from_f32(y), slot, np.array(cb["weights"], np.float32))
    assert np.array_equal(_f32(out), np.array(cb["out"], np.float32))
    al = g["aligned_2"]
    off2 = oracle.expert_offsets(lay["num_tokens_per_expert"], 2)
    assert off2.tolist() == al["expert_offset"]
    slot2, src2, ovf2 = oracle.slots(idx, lay["valid"], off2, int(off2[-1]))
    assert slot2.tolist() == al["slot"] and ovf2 == 0
    assert sorted(set(range(int(off2[-1]))) - set(slot2[slot2 >= 0].tolist())) == al["padding_rows"]
    st = g["static_cap_2"]
    slot_s, ovf_s = oracle.slots_static(idx, lay["valid"], g["E"], 2)
    assert slot_s.tolist() == st["slot"] and ovf_s == st["overflow"]
    bw = g["backward"]
    yb = workloads.bf16_bits_from_f32(y)
    gx = oracle.dispatch_backward(yb, slot)
    assert np.array_equal(_f32(gx), np.array(bw["dispatch_backward"], np.float32))
    go = workloads.bf16_bits_from_f32(np.tile(np.array([[1.0, 2.0]], np.float32), (g["T"], 1)))
    gy, gw = oracle.combine_backward(go, yb, slot, np.array(cb["weights"], np.float32), 9)
    assert np.array_equal(_f32(gy), np.array(bw["grad_y"], np.float32))
    assert np.array_equal(gw, np.array(bw["grad_w"], np.float32))
    c8 = g["combine_fp8"]
    q = np.repeat(np.array([int(c, 16) for c in c8["row_codes"]], np.uint8)[:, None], 256, axis=1)
    sc = np.tile(np.array(c8["scales"], np.float32), (9, 1))
    for wts, key in ((np.array(cb["weights"], np.float32), "out_weighted"), (None, "out_unit")):
        o = _f32(oracle.combine_fp8(q, sc, slot, wts))
        assert np.array_equal(o, np.repeat(np.array(c8[key], np.float32), 128, axis=1)), key



def test_ep_worked_example():
    """The expert-parallel flow on the hand-worked example in
    golden/ep_worked_example.json: destinations, packed rows and their
    metadata, each destination's receive rows, pre-reduced rows and the
    origin's sums, every value given there."""
    g = json.load(open(os.path.join(GOLDEN, "ep_worked_example.json")))
    idx = np.array(g["topk_idx"], np.int64)
    w = np.array(g["topk_weights"], np.float32)
    E, P, H = g["E"], g["P"], g["H"]
    x = workloads.bf16_bits_from_f32(np.arange(g["T"] * H, dtype=np.float32).reshape(g["T"], H))
    y_parts = [workloads.bf16_bits_from_f32(np.array([[10 * p + u + 1, -(10 * p + u + 1)] for u in range(n)],
                                                     np.float32).reshape(n, H))
               for p, n in enumerate(g["expert_outputs"]["rows_per_destination"])]
    r = oracle.ep_one_source(idx, w, x, E, P, False, y_parts=y_parts)
    assert r["part_idx"].tolist() == g["part_idx"]
    assert r["pack"]["num_tokens_per_expert"].tolist() == g["pack_rows_per_destination"]
    assert r["pack"]["slot"].tolist() == g["pack_slot"]
    rows = sum(g["pack_rows_per_destination"])
    assert r["local_idx"][:rows].tolist() == g["local_idx"]
    assert np.array_equal(r["local_w"][:rows], np.array(g["local_w"], np.float32))
    for p, d in enumerate(r["dest"]):
        assert d["unpack"]["slot"].tolist() == g["unpack_slot"][p], p
        assert d["unpack"]["rows"] == g["expert_outputs"]["rows_per_destination"][p], p
    assert np.array_equal(_f32(r["partials"]), np.array(g["partials"], np.float32))
    assert np.array_equal(_f32(r["out"]), np.array(g["out"], np.float32))


CASES = [
    dict(T=1, E=1, K=1, P=1), dict(T=7, E=8, K=3, P=2), dict(T=64, E=16, K=4, P=4),
    dict(T=65, E=32, K=8, P=8), dict(T=300, E=64, K=6, P=8), dict(T=513, E=256, K=8, P=16),
    dict(T=200, E=1024, K=16, P=64), dict(T=50, E=5, K=5, P=5),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("mode", ["clean", "masked", "dirty"])
def test_layout_and_slots_against_independent_definitions(case, mode):
    T, E, K, P = case["T"], case["E"], case["K"], case["P"]
    kw = dict(clean={}, masked=dict(mask_frac=0.2),
              dirty=dict(distinct=False, mask_frac=0.1, invalid_frac=0.1, dup_frac=0.2))[mode]
    idx, w = workloads.random_case(1000 + T, T, E, K, **kw)
    lay = oracle.layout(idx, E, P)
    valid = _valid_independent(idx, E)
    assert np.array_equal(lay["valid"], valid)
    masked = int((idx < 0).sum())
    ninv = T * K - masked - int(valid.sum())
    assert lay["num_invalid"] == ninv
    cnt = np.bincount(idx[valid == 1], minlength=E)
    assert np.array_equal(lay["num_tokens_per_expert"], cnt)
    assert cnt.sum() == T * K - masked - ninv
    epp = E // P
    part = np.zeros((T, P), np.uint8)
    for t in range(T):
        for e in np.unique(idx[t][valid[t] == 1]):
            part[t, e // epp] = 1
    assert np.array_equal(lay["is_token_in_partition"], part)
    pc = lay["num_tokens_per_partition"]
    assert np.array_equal(pc, part.sum(axis=0))
    assert np.all(pc <= T)
    for p in range(P):
        assert pc[p] >= cnt[p * epp:(p + 1) * epp].max(initial=0)
    off = oracle.expert_offsets(cnt)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
    N = int(off[-1])
    for cap in (T * K, N, max(N - 7, 0), N // 2, 0):
        slot, src, ovf = oracle.slots(idx, lay["valid"], off, cap)
        # textbook stable sort of the flattened pairs by expert id; invalid
        # pairs sort last
        key = np.where(valid.reshape(-1) == 1, idx.reshape(-1), np.int64(1) << 62)
        order = np.argsort(key, kind="stable")
        rank = np.empty(order.size, np.int64)
        rank[order] = np.arange(order.size)
        exp = np.where((valid.reshape(-1) == 1) & (rank < cap), rank, -1).reshape(T, K)
        assert np.array_equal(slot, exp)
        assert ovf == int(N > cap)
        rows = min(N, cap)
        tok = np.repeat(np.arange(T), K)
        assert np.array_equal(src[:rows], tok[order[:rows]])
        if cap >= N:
            # bijection onto [0, N), each row inside its expert's range,
            # source tokens strictly increasing within an expert
            got = np.sort(slot[slot >= 0])
            assert np.array_equal(got, np.arange(N))
            for e in range(E):
                seg = src[off[e]:off[e + 1]]
                assert np.all(np.diff(seg) > 0)
                es = slot[(idx == e) & (valid == 1)]
                assert np.all((es >= off[e]) & (es < off[e + 1]))


def test_layout_rejects_bad_dims():
    idx = np.zeros((4, 2), np.int64)
    with pytest.raises(ValueError):
        oracle.layout(idx, 6, 4)


def test_empty_input():
    idx = np.zeros((0, 4), np.int64)
    lay = oracle.layout(idx, 8, 2)
    assert lay["num_tokens_per_expert"].sum() == 0 and lay["num_tokens_per_partition"].sum() == 0
    off = oracle.expert_offsets(lay["num_tokens_per_expert"])
    slot, src, ovf = oracle.slots(idx, lay["valid"], off, 0)
    assert slot.size == 0 and ovf == 0


# ----------------------------------------------------------------------------
# dispatch / combine
# ----------------------------------------------------------------------------

def _pipeline(idx, w, x, E, P, use_fp8, cap=None):
    return oracle.run_all(idx, w, x, E, P, use_fp8, capacity=cap)


@pytest.mark.parametrize("use_fp8", [False, True])
def test_dispatch_rows_are_the_source_rows(use_fp8):
    T, H, E, K, P = 97, 384, 32, 4, 4
    idx, w = workloads.random_case(7, T, E, K, mask_frac=0.1)
    x = workloads.random_rows(8, T, H, "wide")
    r = _pipeline(idx, w, x, E, P, use_fp8)
    recv = r["recv_x"]
    src = r["src_token"]
    if not use_fp8:
        assert np.array_equal(recv, x[src])
    else:
        for row in range(r["rows"]):
            t = src[row]
            for b in range(H // 128):
                q, s = oracle.quant_block(x[t, b * 128:(b + 1) * 128])
                assert np.array_equal(recv[row, b * 128:(b + 1) * 128], q)
                assert r["recv_scales"][row, b] == s


def test_dispatch_capacity_drops_rows():
    T, H, E, K, P = 40, 128, 8, 3, 2
    idx, w = workloads.random_case(17, T, E, K)
    x = workloads.random_rows(18, T, H, "normal")
    full = _pipeline(idx, w, x, E, P, False)
    part = _pipeline(idx, w, x, E, P, False, cap=50)
    assert part["overflow"] == 1 and part["rows"] == 50
    assert np.array_equal(part["recv_x"], full["recv_x"][:50])


@pytest.mark.parametrize("name", ["tiny", "skewed"])
def test_bf16_round_trip_is_exact_identity(name):
    """Identity experts and weights summing to 1: combine(dispatch(x)) == x
    bit for bit (fp32 error ~K*2^-24 is far below half a BF16 ulp)."""
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    r = _pipeline(idx, w, x, wl.E, wl.P, False)
    out = oracle.combine(r["recv_x"], r["slot"], w)
    live = (r["slot"] >= 0).any(axis=1)
    wsum = w.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(wsum[live] - 1) <= wl.K * 2.0 ** -24)
    assert np.array_equal(out[live], x[live])
    assert np.all(out[~live] == 0)


def test_fp8_round_trip_within_fp8_error():
    wl = workloads.config("decode")
    idx, w, x = workloads.make(wl)
    r = _pipeline(idx, w, x, wl.E, wl.P, True)
    nb = wl.H // 128
    dq = np.empty((r["rows"], wl.H), np.float32)
    lut = np.array([oracle.e4m3fn_decode(c) if (c & 0x7F) != 0x7F else 0.0 for c in range(256)], np.float32)
    for b in range(nb):
        dq[:, b * 128:(b + 1) * 128] = lut[r["recv_x"][:, b * 128:(b + 1) * 128]] * r["recv_scales"][:, b:b + 1]
    y = workloads.bf16_bits_from_f32(dq)
    out = _f32(oracle.combine(y, r["slot"], w)).astype(np.float64)
    xf = _f32(x).astype(np.float64)
    s_tok = np.repeat(r["recv_scales"][np.maximum(r["slot"][:, 0], 0)], 128, axis=1)
    bound = 2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * s_tok + 2.0 ** -7 * np.abs(xf) + 1e-30
    assert np.all(np.abs(out - xf) <= bound)


def test_adjoint_exact_on_small_integers():
    """<dispatch(x), y> == <x, combine_{w=1}(y)> exactly when all values are
    small integers (every product and sum is exact in fp32, bf16 and fp64)."""
    rng = np.random.default_rng(4)
    for T, E, K, P, H in [(33, 8, 3, 2, 16), (130, 64, 6, 8, 24), (64, 16, 16, 4, 8)]:
        idx, _ = workloads.random_case(T, T, E, K, mask_frac=0.15, distinct=K <= E)
        w = np.ones((T, K), np.float32)
        x = workloads.bf16_bits_from_f32(rng.integers(-3, 4, (T, H)).astype(np.float32))
        r = _pipeline(idx, w, x, E, P, False)
        y = workloads.bf16_bits_from_f32(rng.integers(-3, 4, (r["rows"], H)).astype(np.float32))
        lhs = (_f32(r["recv_x"]).astype(np.float64) * _f32(y)).sum()
        cy = oracle.combine(y, r["slot"], w)
        rhs = (_f32(x).astype(np.float64) * _f32(cy)).sum()
        assert lhs == rhs


def test_combine_is_gather_for_k1():
    T, H, E = 50, 64, 10
    idx, _ = workloads.random_case(3, T, E, 1, mask_frac=0.2)
    w = np.ones((T, 1), np.float32)
    r = _pipeline(idx, w, None, E, 2, False)
    y = workloads.random_rows(5, r["rows"], H, "bits")
    out = oracle.combine(y, r["slot"], w)
    s = r["slot"][:, 0]
    ref = torch.from_numpy(y.view(np.int16)).index_select(0, torch.from_numpy(np.maximum(s, 0).astype(np.int64))).numpy().view(np.uint16)
    assert np.array_equal(out[s >= 0], ref[s >= 0])
    # masked token -> +0 row (fma(w, y, +0) never runs)
    assert np.all(out[s < 0] == 0)


def test_combine_within_one_ulp_of_exact_sum():
    T, H, E, K = 80, 256, 32, 8
    idx, w = workloads.random_case(12, T, E, K, mask_frac=0.1)
    r = _pipeline(idx, w, None, E, 4, False)
    y = workloads.random_rows(13, r["rows"], H, "wide")
    out = _f32(oracle.combine(y, r["slot"], w)).astype(np.float64)
    yf = _f32(y).astype(np.float64)
    exact = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            s = r["slot"][t, k]
            if s >= 0:
                exact[t] += float(w[t, k]) * yf[s]
    # 1 bf16 ulp of the exact value (8 significant bits), plus the fp32
    # accumulation error bound K * 2^-24 * sum|w y|
    mag = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            s = r["slot"][t, k]
            if s >= 0:
                mag[t] += abs(float(w[t, k])) * np.abs(yf[s])
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-38))) - 7)
    assert np.all(np.abs(out - exact) <= ulp + K * 2.0 ** -24 * mag + 1e-38)


def test_combine_pow2_weights_exact():
    T, H, E, K = 40, 32, 16, 4
    idx, w = workloads.random_case(14, T, E, K, weights="pow2")
    r = _pipeline(idx, w, None, E, 4, False)
    rng = np.random.default_rng(15)
    y = workloads.bf16_bits_from_f32(rng.integers(-8, 9, (r["rows"], H)).astype(np.float32))
    out = _f32(oracle.combine(y, r["slot"], w)).astype(np.float64)
    yf = _f32(y).astype(np.float64)
    exact = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            exact[t] += float(w[t, k]) * yf[r["slot"][t, k]]
    # every partial sum is a short dyadic number, so the fp32 fma chain is
    # exact and the only rounding is the final one to bf16 (torch's RNE)
    assert np.all(np.abs(exact) < 2 ** 10)
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(out, ref.astype(np.float64))


# ----------------------------------------------------------------------------
# the five workloads: invariants at full size
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "decode", "v3", "skewed", "large"])
def test_workload_invariants(name):
    wl = workloads.config(name)
    idx, w, _ = workloads.make(wl, with_x=False)
    lay = oracle.layout(idx, wl.E, wl.P)
    masked = int((idx < 0).sum())
    assert lay["num_invalid"] == 0
    assert lay["num_tokens_per_expert"].sum() == wl.T * wl.K - masked
    assert masked == int(np.floor(wl.mask_frac * wl.T * wl.K))
    assert np.array_equal(lay["num_tokens_per_expert"], np.bincount(idx[idx >= 0], minlength=wl.E))
    if name == "v3":
        # group-limited gating: at most 4 of the 8 groups (= partitions)
        assert lay["is_token_in_partition"].sum(axis=1).max() <= 4
    if name == "skewed":
        c = lay["num_tokens_per_expert"]
        assert c.max() > 20 * max(c.min(), 1)


# ----------------------------------------------------------------------------
# backward calls
# ----------------------------------------------------------------------------

def _small_int_bf16(rng, shape, lo=-3, hi=4):
    return workloads.bf16_bits_from_f32(rng.integers(lo, hi, shape).astype(np.float32))


@pytest.mark.parametrize("T,E,K,P,H", [(33, 8, 3, 2, 16), (130, 64, 6, 8, 24), (64, 16, 16, 4, 8)])
def test_dispatch_backward_is_the_adjoint_of_dispatch(T, E, K, P, H):
    """<dispatch(x), g> == <x, dispatch_backward(g)> exactly on small integers
    (the backward of dispatch is combine with unit weights)."""
    rng = np.random.default_rng(T + K)
    idx, _ = workloads.random_case(T, T, E, K, mask_frac=0.15, distinct=K <= E,
                                   invalid_frac=0.05)
    w = np.ones((T, K), np.float32)
    x = _small_int_bf16(rng, (T, H))
    r = oracle.run_all(idx, w, x, E, P, False)
    g = _small_int_bf16(rng, (r["rows"], H))
    lhs = (_f32(r["recv_x"]).astype(np.float64) * _f32(g)).sum()
    gx = oracle.dispatch_backward(g, r["slot"])
    rhs = (_f32(x).astype(np.float64) * _f32(gx)).sum()
    assert lhs == rhs
    # a token none of whose pairs was dispatched gets a +0 gradient
    dead = (r["slot"] < 0).all(axis=1)
    assert np.all(gx[dead] == 0)


@pytest.mark.parametrize("T,E,K,P,H", [(40, 8, 3, 2, 16), (96, 32, 8, 4, 32)])
def test_combine_backward_grad_y_is_the_adjoint_of_combine(T, E, K, P, H):
    """<combine_w(y), g> == <y, grad_y> exactly (small integers, weights in
    {1/2, 1, 2}); rows no pair maps to keep their previous contents."""
    rng = np.random.default_rng(7 * T + K)
    idx, _ = workloads.random_case(T + 1, T, E, K, mask_frac=0.2)
    w = np.array([0.5, 1.0, 2.0], np.float32)[rng.integers(0, 3, (T, K))]
    r = oracle.run_all(idx, w, None, E, P, False, capacity=T * K)
    rows = T * K
    y = _small_int_bf16(rng, (rows, H))
    g = _small_int_bf16(rng, (T, H))
    out = oracle.combine(y, r["slot"], w)
    gy, gw = oracle.combine_backward(g, y, r["slot"], w, rows, fill=0x7777)
    used = np.zeros(rows, bool)
    used[r["slot"][r["slot"] >= 0]] = True
    assert np.all(gy[~used] == 0x7777)
    gy_f = np.where(used[:, None], _f32(gy).astype(np.float64), 0.0)
    lhs = (_f32(out).astype(np.float64) * _f32(g)).sum()
    rhs = (_f32(y).astype(np.float64) * gy_f).sum()
    assert lhs == rhs
    assert np.all(gw[r["slot"] < 0] == 0)


def test_combine_backward_grad_w_matches_finite_differences():
    """combine is linear in w: <combine(y, w + e_tk), g> - <combine(y, w), g>
    equals grad_w[t, k] exactly when every value is a small integer."""
    rng = np.random.default_rng(3)
    T, E, K, P, H = 24, 16, 4, 4, 16
    idx, _ = workloads.random_case(5, T, E, K, mask_frac=0.1)
    w = rng.integers(1, 3, (T, K)).astype(np.float32)
    r = oracle.run_all(idx, w, None, E, P, False)
    y = _small_int_bf16(rng, (r["rows"], H))
    g = _small_int_bf16(rng, (T, H))
    _, gw = oracle.combine_backward(g, y, r["slot"], w, r["rows"])
    base = (_f32(oracle.combine(y, r["slot"], w)).astype(np.float64) * _f32(g)).sum()
    for t in range(T):
        for k in range(K):
            w2 = w.copy()
            w2[t, k] += 1.0
            bumped = (_f32(oracle.combine(y, r["slot"], w2)).astype(np.float64) * _f32(g)).sum()
            assert gw[t, k] == bumped - base, (t, k)


def test_combine_backward_grad_y_single_rounding():
    """grad_y is one fp32 product rounded once to BF16 (checked against
    torch's multiply and BF16 rounding on wide-range values)."""
    T, E, K, P, H = 50, 8, 2, 2, 128
    idx, _ = workloads.random_case(9, T, E, K)
    w = workloads.random_case(9, T, E, K, weights="dirichlet")[1]
    r = oracle.run_all(idx, w, None, E, P, False)
    g = workloads.random_rows(10, T, H, "wide")
    gy, _ = oracle.combine_backward(g, None, r["slot"], w, r["rows"])
    gt = torch.from_numpy(_f32(g))
    for t in range(T):
        for k in range(K):
            s = r["slot"][t, k]
            ref = (gt[t] * torch.tensor(float(w[t, k]), dtype=torch.float32)).to(torch.bfloat16)
            assert np.array_equal(gy[s], ref.view(torch.int16).numpy().view(np.uint16))


# ----------------------------------------------------------------------------
# low-latency (static-capacity) layout
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,K,cap", [(128, 256, 8, 16), (200, 16, 4, 64), (64, 8, 3, 5), (1, 4, 2, 1)])
@pytest.mark.parametrize("mode", ["clean", "dirty"])
def test_static_slots_against_stable_sort(T, E, K, cap, mode):
    """slot = e*cap + rank, rank = position of the pair among expert e's pairs
    in a textbook stable sort by expert id; pairs ranked >= cap are dropped."""
    kw = {} if mode == "clean" else dict(distinct=False, mask_frac=0.1, invalid_frac=0.05, dup_frac=0.1)
    idx, _ = workloads.random_case(T + cap, T, E, K, **kw)
    valid = _valid_independent(idx, E)
    slot, ovf = oracle.slots_static(idx, valid, E, cap)
    key = np.where(valid.reshape(-1) == 1, idx.reshape(-1), np.int64(1) << 62)
    order = np.argsort(key, kind="stable")
    pos = np.empty(order.size, np.int64)
    pos[order] = np.arange(order.size)
    cnt = np.bincount(idx[valid == 1], minlength=E)
    first = np.concatenate([[0], np.cumsum(cnt)])[:E]
    flat_idx = idx.reshape(-1)
    exp = np.full(T * K, -1, np.int64)
    ok = valid.reshape(-1) == 1
    rank = pos[ok] - first[flat_idx[ok]]
    exp[np.nonzero(ok)[0]] = np.where(rank < cap, flat_idx[ok] * cap + rank, -1)
    assert np.array_equal(slot.reshape(-1), exp)
    assert ovf == int((cnt > cap).any())
    # rows are distinct and inside the owning expert's block
    s = slot[slot >= 0]
    assert np.unique(s).size == s.size
    assert np.all(s // cap == idx[slot >= 0])


# ----------------------------------------------------------------------------
# combine of FP8 rows (the dequantising option of the backward of dispatch)
# ----------------------------------------------------------------------------

def _finite_codes(rng, shape):
    q = rng.integers(0, 256, shape, dtype=np.uint32).astype(np.uint8)
    nan = (q & 0x7F) == 0x7F
    q[nan] ^= 0x01                       # 0x7F / 0xFF (NaN) -> 0x7E / 0xFE (+-448)
    return q


def test_combine_fp8_single_pair_matches_torch_dequant():
    """K=1, unit weight: out = bf16( +0 + decode(q) * scale ), with torch's own
    float8_e4m3fn decoder, fp32 multiply and bfloat16 rounding (the sum starts
    from +0, so a -0 product gives +0)."""
    rng = np.random.default_rng(31)
    T, H = 64, 256
    q = _finite_codes(rng, (T, H))
    sc = (rng.standard_normal((T, H // 128)).astype(np.float32) *
          np.ldexp(np.float32(1), rng.integers(-20, 21, (T, H // 128))).astype(np.float32))
    slot = rng.permutation(T).astype(np.int32).reshape(T, 1)
    out = oracle.combine_fp8(q, sc, slot, None)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).float()
    s_full = torch.from_numpy(np.repeat(sc, 128, axis=1))
    want = ((dec * s_full)[torch.from_numpy(slot[:, 0].astype(np.int64))] + 0.0).to(torch.bfloat16)
    assert np.array_equal(out, want.view(torch.int16).numpy().view(np.uint16))
    # weighted form with w = 1 is the unit form
    assert np.array_equal(oracle.combine_fp8(q, sc, slot, np.ones((T, 1), np.float32)), out)


def test_combine_fp8_pow2_scales_and_weights_exact():
    """Power-of-two scales and weights keep every product and partial sum a
    short dyadic number: the fp32 chain is exact and only the final rounding
    (torch's bf16 RNE of the exact sum) remains."""
    T, H, E, K = 48, 256, 16, 4
    idx, w = workloads.random_case(32, T, E, K, weights="pow2", mask_frac=0.1)
    r = _pipeline(idx, w, None, E, 4, False)
    rng = np.random.default_rng(33)
    rows = r["rows"]
    q = _finite_codes(rng, (rows, H))
    q[(q & 0x78) > 0x50] &= 0x87         # keep magnitudes < 2^4 so sums stay short
    sc = np.ldexp(np.float32(1), rng.integers(-6, 3, (rows, H // 128))).astype(np.float32)
    out = _f32(oracle.combine_fp8(q, sc, r["slot"], w)).astype(np.float64)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    v = dec * np.repeat(sc.astype(np.float64), 128, axis=1)
    exact = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            s = r["slot"][t, k]
            if s >= 0:
                exact[t] += float(w[t, k]) * v[s]
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(out, ref.astype(np.float64))
    # a token whose every pair is masked gets +0
    dead = np.all(r["slot"] < 0, axis=1)
    assert np.all(oracle.combine_fp8(q, sc, r["slot"], w)[dead] == 0)


def test_combine_fp8_round_trip_within_fp8_error():
    """dispatch (FP8) then the FP8 combine with unit weights: each token's K
    identical rows sum to K * x within the FP8 error bound."""
    wl = workloads.config("decode")
    idx, w, x = workloads.make(wl)
    r = _pipeline(idx, w, x, wl.E, wl.P, True)
    out = _f32(oracle.combine_fp8(r["recv_x"], r["recv_scales"], r["slot"], None)).astype(np.float64)
    xf = _f32(x).astype(np.float64)
    kk = (r["slot"] >= 0).sum(axis=1, keepdims=True).astype(np.float64)
    s_tok = np.repeat(r["recv_scales"][np.maximum(r["slot"][:, 0], 0)], 128, axis=1)
    bound = kk * (2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * s_tok) + 2.0 ** -8 * kk * np.abs(xf) + 1e-30
    assert np.all(np.abs(out - kk * xf) <= bound)


# ----------------------------------------------------------------------------
# GEMM-facing layouts: aligned expert blocks, pre-quantised FP8 input
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("A", [1, 4, 64, 128])
def test_aligned_offsets_closed_form(A):
    rng = np.random.default_rng(A)
    cnt = rng.integers(0, 300, 97).astype(np.int32)
    cnt[::7] = 0
    off = oracle.expert_offsets(cnt, A)
    block = -(-cnt.astype(np.int64) // A) * A          # smallest multiple of A >= count
    assert off[0] == 0 and np.array_equal(np.diff(off), block)
    assert np.all(off % A == 0)
    if A == 1:
        assert np.array_equal(off[1:], np.cumsum(cnt))


@pytest.mark.parametrize("A,use_fp8", [(16, False), (128, True)])
def test_aligned_dispatch_places_rows_and_zero_padding(A, use_fp8):
    T, H, E, K = 300, 256, 24, 4
    idx, w = workloads.random_case(55 + A, T, E, K, mask_frac=0.05)
    x = workloads.random_rows(56, T, H, "wide" if use_fp8 else "normal")
    r = oracle.run_all(idx, w, x, E, 4, use_fp8, align=A)
    off, cnt = r["expert_offset"], r["num_tokens_per_expert"]
    assert r["overflow"] == 0 and r["rows"] == off[-1] and r["N"] == cnt.sum()
    # rows of expert e: [off[e], off[e] + cnt[e]), ascending source token
    dense = oracle.run_all(idx, w, x, E, 4, use_fp8)
    doff = dense["expert_offset"]
    for t in range(T):
        for k in range(K):
            s, sd = r["slot"][t, k], dense["slot"][t, k]
            assert (s < 0) == (sd < 0)
            if s >= 0:
                e = idx[t, k]
                assert s - off[e] == sd - doff[e]            # same rank within the expert
                assert np.array_equal(r["recv_x"][s], dense["recv_x"][sd])
    pad = np.ones(r["rows"], bool)
    for e in range(E):
        pad[off[e]:off[e] + cnt[e]] = False
    assert np.all(r["recv_x"][pad] == 0)
    if use_fp8:
        assert np.all(r["recv_scales"][pad] == 0)
    assert np.all(r["src_token"][pad] == -1)


def test_fp8_input_dispatch_copies_codes_and_scales():
    T, H, E, K = 200, 512, 16, 4
    idx, w = workloads.random_case(61, T, E, K, mask_frac=0.1)
    rng = np.random.default_rng(62)
    xq = rng.integers(0, 256, (T, H), dtype=np.uint32).astype(np.uint8)
    xs = rng.standard_normal((T, H // 128)).astype(np.float32)
    r = oracle.run_all(idx, w, None, E, 4, True)
    recv, sc = oracle.dispatch_fp8_input(xq, xs, r["slot"], r["rows"])
    src = r["src_token"]
    assert np.all(src >= 0)
    assert np.array_equal(recv, xq[src]) and np.array_equal(sc.view(np.uint32), xs[src].view(np.uint32))
    # passing dispatch's own per-token quantisation through reproduces the quantising dispatch
    x = workloads.random_rows(63, T, H, "wide")
    q = np.empty((T, H), np.uint8)
    s = np.empty((T, H // 128), np.float32)
    for t in range(T):
        for b in range(H // 128):
            q[t, b * 128:(b + 1) * 128], s[t, b] = oracle.quant_block(x[t, b * 128:(b + 1) * 128])
    r2 = oracle.run_all(idx, w, x, E, 4, True)
    recv2, sc2 = oracle.dispatch_fp8_input(q, s, r2["slot"], r2["rows"])
    assert np.array_equal(recv2, r2["recv_x"]) and np.array_equal(sc2, r2["recv_scales"])


# ----------------------------------------------------------------------------
# the oracle's own memory safety: every entry point under ASan + UBSan
# ----------------------------------------------------------------------------

def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-I", os.path.join(root, "oracle"),
           os.path.join(root, "tests", "oracle_sanitize_driver.c"),
           os.path.join(root, "oracle", "oracle.c"), "-lm", "-o", str(exe)]
    built = subprocess.run(cmd, capture_output=True, text=True)
    if built.returncode != 0 and "sanitize" in built.stderr:
        pytest.skip("sanitizer runtime not available: " + built.stderr[-200:])
    assert built.returncode == 0, built.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr[-3000:]
    assert "oracle sanitizer run: ok" in run.stdout


# ----------------------------------------------------------------------------
# brute force on tiny cases: an independent pure-Python reading of the steps
# ----------------------------------------------------------------------------

def _brute_layout_slots(idx, E, P, cap):
    """Layout and slots enumerated the slow way: rows of expert 0 first, in
    token order, then expert 1, ..."""
    T, K = idx.shape
    epp = E // P
    valid = np.zeros((T, K), np.uint8)
    cnt = [0] * E
    mask = np.zeros((T, P), np.uint8)
    ninv = 0
    for t in range(T):
        seen = set()
        for k in range(K):
            e = int(idx[t, k])
            if e < 0:
                continue
            if e >= E or e in seen:
                ninv += 1
                continue
            seen.add(e)
            valid[t, k] = 1
            cnt[e] += 1
            mask[t, e // epp] = 1
    order = [(t, k) for e in range(E) for t in range(T) for k in range(K)
             if valid[t, k] and int(idx[t, k]) == e]
    slot = np.full((T, K), -1, np.int32)
    ovf = 0
    for r, (t, k) in enumerate(order):
        if r < cap:
            slot[t, k] = r
        else:
            ovf = 1
    return dict(num_tokens_per_expert=np.array(cnt, np.int32), is_token_in_partition=mask,
                num_tokens_per_partition=mask.sum(axis=0).astype(np.int32), num_invalid=ninv,
                slot=slot, overflow=ovf)


def _rn_f32(q):
    """Round an exact rational to the nearest fp32, ties to even."""
    from fractions import Fraction
    if q == 0:
        return 0.0
    s = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                        # below the normal range: quantum 2^-149
    m = a / Fraction(2) ** (e - 23)
    n = int(m)
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * float(np.float32(n * 2.0 ** (e - 23)))


def test_brute_force_tiny_cases_1000_seeds():
    rng = np.random.default_rng(2024)
    for seed in range(1000):
        T, E, K = int(rng.integers(0, 9)), int(rng.choice([1, 2, 4, 8])), int(rng.integers(1, 4))
        P = int(rng.choice([p for p in (1, 2, 4) if E % p == 0]))
        idx = rng.integers(-2, E + 2, (T, K)).astype(np.int64)
        cap = int(rng.integers(0, T * K + 1)) if seed % 3 == 0 else T * K
        ref = _brute_layout_slots(idx, E, P, cap)
        r = oracle.run_all(idx, np.ones((T, K), np.float32), None, E, P, False, capacity=cap)
        for key in ("num_tokens_per_expert", "num_tokens_per_partition", "is_token_in_partition",
                    "slot"):
            assert np.array_equal(r[key], ref[key]), (seed, key)
        assert r["num_invalid"] == ref["num_invalid"] and r["overflow"] == ref["overflow"], seed


def test_brute_force_tiny_dispatch_and_combine():
    """FP8 quantisation by nearest-value search and combine by exact rational
    arithmetic with one rounding per fma, on 200 tiny random cases."""
    from fractions import Fraction
    rng = np.random.default_rng(77)
    H = 128
    for seed in range(200):
        T, E, K = int(rng.integers(1, 9)), int(rng.choice([2, 4, 8])), int(rng.integers(1, 4))
        idx = rng.integers(-1, E, (T, K)).astype(np.int64)
        w = rng.random((T, K)).astype(np.float32)
        x = workloads.random_rows(seed, T, H, ["normal", "wide", "bits", "subnormal"][seed % 4])
        r = oracle.run_all(idx, w, x, E, 1, True)
        ref = _brute_layout_slots(idx, E, 1, T * K)
        assert np.array_equal(r["slot"], ref["slot"])
        xf = _f32(x)
        for t in range(T):
            a = np.float32(max(np.float32(np.abs(xf[t]).max()), np.float32(2.0 ** -64)))
            inv = np.float32(448.0) / a
            s = a / np.float32(448.0)
            v = (xf[t] * inv).astype(np.float32)
            codes = _nearest_brute(v)
            for k in range(K):
                if ref["slot"][t, k] >= 0:
                    assert np.array_equal(r["recv_x"][ref["slot"][t, k]], codes), (seed, t, k)
                    assert r["recv_scales"][ref["slot"][t, k], 0] == s
        # combine of random BF16 rows with exact fma emulation
        y = workloads.random_rows(seed + 5000, max(r["rows"], 1), H)
        yf = _f32(y)
        out = _f32(oracle.combine(y, r["slot"], w))
        for t in range(T):
            for j in range(0, H, 17):
                acc = 0.0
                for k in range(K):
                    s_ = ref["slot"][t, k]
                    if s_ >= 0:
                        acc = _rn_f32(Fraction(float(w[t, k])) * Fraction(float(yf[s_, j])) + Fraction(acc))
                want = torch.tensor([acc], dtype=torch.float32).to(torch.bfloat16).float().item()
                assert out[t, j] == want or (out[t, j] == 0 and want == 0), (seed, t, j)


# ----------------------------------------------------------------------------
# exact-arithmetic pins of the backward reductions: the fp32 chain in
# ascending k (one rounding per operation) and grad_w's single final rounding
# ----------------------------------------------------------------------------

def _decode_e4m3_exact(q):
    """Exact values of E4M3FN codes, by torch's own decoder (fp32 is exact
    for every finite code)."""
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double().numpy()


def _bf16_of(values_f64):
    """torch's BF16 rounding (RNE) of fp32 values, as bit patterns."""
    t = torch.from_numpy(np.asarray(values_f64, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _wide_rows(rng, rows, H):
    """BF16 rows whose values span many binades within and across rows, so
    that the order of an fp32 sum changes its rounding."""
    v = rng.standard_normal((rows, H)).astype(np.float32)
    v *= np.ldexp(np.float32(1.0), rng.integers(-12, 13, (rows, H))).astype(np.float32)
    return workloads.bf16_bits_from_f32(v)


def _cancelling_pattern(slot):
    """Per token, the roles of its dispatched pairs in ascending k: the first
    is small, the next two are a large value and its exact negative, the rest
    small.  Summed left to right the first small term is absorbed by the large
    one and the cancellation leaves the later ones; summed in any other order
    different small terms survive, which stays visible after BF16 rounding."""
    roles = {}
    for t in range(slot.shape[0]):
        ks = [k for k in range(slot.shape[1]) if slot[t, k] >= 0]
        for i, k in enumerate(ks):
            roles[(t, k)] = ("big+" if i == 1 else "big-" if i == 2 else "small") if len(ks) >= 3 else "small"
    return roles


def test_dispatch_backward_exact_fp32_chain_in_k_order():
    """grad_x[t][j] = bf16( ((0 + g_k0) + g_k1) + ... ) over the dispatched k
    in ascending order, each addition one fp32 rounding of the exact rational
    sum (stakiran "DeepEP 要約" section 3: the backward of dispatch is combine,
    whose accumulation runs over k ascending).  The rows hold a small term, a
    large value and its negative, so a reversed or reassociated sum gives a
    different BF16 result."""
    from fractions import Fraction
    rng = np.random.default_rng(505)
    H = 128
    differs = 0
    for case in range(12):
        T, E, K = int(rng.integers(3, 7)), 8, int(rng.integers(3, 6))
        idx = rng.integers(-1, E, (T, K)).astype(np.int64)
        idx[0] = np.arange(K) % E                            # one token with K pairs
        r = oracle.run_all(idx, np.ones((T, K), np.float32), None, E, 2, False)
        rows = max(r["rows"], 1)
        gv = rng.standard_normal((rows, H)).astype(np.float32)
        for (t, k), role in _cancelling_pattern(r["slot"]).items():
            if role == "big+":
                big = rng.integers(128, 256, H).astype(np.float32) * np.ldexp(
                    np.float32(1), rng.integers(20, 28, H)).astype(np.float32)
                big *= np.where(rng.integers(0, 2, H) == 1, np.float32(-1), np.float32(1))
                gv[r["slot"][t, k]] = big
                k2 = [kk for kk in range(K) if r["slot"][t, kk] >= 0][2]
                gv[r["slot"][t, k2]] = -big
        g = workloads.bf16_bits_from_f32(gv)
        gf = _f32(g)
        got = oracle.dispatch_backward(g, r["slot"])
        want = np.zeros((T, H))
        rev = np.zeros((T, H))
        for t in range(T):
            ks = [k for k in range(K) if r["slot"][t, k] >= 0]
            for j in range(H):
                acc = 0.0
                for k in ks:
                    acc = _rn_f32(Fraction(acc) + Fraction(float(gf[r["slot"][t, k], j])))
                want[t, j] = acc
                acc = 0.0
                for k in reversed(ks):
                    acc = _rn_f32(Fraction(acc) + Fraction(float(gf[r["slot"][t, k], j])))
                rev[t, j] = acc
        assert np.array_equal(got, _bf16_of(want)), case
        differs += int((_bf16_of(rev) != _bf16_of(want)).sum())
    assert differs > 500        # the data tell the two orders apart after rounding


@pytest.mark.parametrize("weighted", [False, True])
def test_combine_fp8_exact_fp32_chain_in_k_order(weighted):
    """FP8 combine: v = fp32(decode(q) * scale) (one rounding), then
    acc = fp32(w * v + acc) per dispatched k in ascending order (one rounding
    per fused multiply-add; w = 1 gives fp32(v + acc)), then BF16 RNE
    (stakiran section 3: the backward of dispatch is combine; aikraft.ru
    "Технические детали и требования": FP8 rows).  Scales are not powers of
    two, weights are arbitrary fp32 (equal on the cancelling pair), and each
    token's rows hold a small term, a large row and its negative: the order,
    the fusion and the scale product all show in the BF16 result."""
    from fractions import Fraction
    rng = np.random.default_rng(606 + weighted)
    H = 128
    differs = 0
    for case in range(10):
        T, E, K = int(rng.integers(3, 7)), 8, int(rng.integers(3, 6))
        idx = rng.integers(-1, E, (T, K)).astype(np.int64)
        idx[0] = np.arange(K) % E
        w = (rng.random((T, K)) * 2.0 - 0.5).astype(np.float32)
        r = oracle.run_all(idx, w, None, E, 2, False)
        rows = max(r["rows"], 1)
        q = _finite_codes(rng, (rows, H))
        sc = (rng.random((rows, 1)) + 0.5).astype(np.float32) * \
            np.ldexp(np.float32(1), rng.integers(-8, 0, (rows, 1))).astype(np.float32)
        for (t, k), role in _cancelling_pattern(r["slot"]).items():
            if role == "big+":
                k2 = [kk for kk in range(K) if r["slot"][t, kk] >= 0][2]
                s1, s2 = r["slot"][t, k], r["slot"][t, k2]
                q[s1] = (rng.integers(0x70, 0x7F, H) | (rng.integers(0, 2, H) << 7)).astype(np.uint8)
                q[s2] = q[s1] ^ np.uint8(0x80)
                sc[s1] = sc[s2] = np.float32(rng.random() + 0.5) * np.float32(2.0 ** 20)
                w[t, k2] = w[t, k]
        dec = _decode_e4m3_exact(q)
        got = oracle.combine_fp8(q, sc, r["slot"], w if weighted else None)
        want = np.zeros((T, H))
        rev = np.zeros((T, H))
        for t in range(T):
            ks = [k for k in range(K) if r["slot"][t, k] >= 0]
            for j in range(H):
                terms = []
                for k in ks:
                    s = r["slot"][t, k]
                    v = _rn_f32(Fraction(float(dec[s, j])) * Fraction(float(sc[s, 0])))
                    terms.append((Fraction(float(w[t, k])) if weighted else Fraction(1), Fraction(v)))
                acc = 0.0
                for wk, v in terms:
                    acc = _rn_f32(wk * v + Fraction(acc))
                want[t, j] = acc
                acc = 0.0
                for wk, v in reversed(terms):
                    acc = _rn_f32(wk * v + Fraction(acc))
                rev[t, j] = acc
        assert np.array_equal(got, _bf16_of(want)), case
        differs += int((_bf16_of(rev) != _bf16_of(want)).sum())
    assert differs > 500


def _exact_dot_rounded_once(g_f32, y_f32):
    """The exact dot product of two fp32 vectors (Fraction), rounded once to
    fp32, ties to even."""
    from fractions import Fraction
    s = Fraction(0)
    for a, b in zip(g_f32.tolist(), y_f32.tolist()):
        s += Fraction(a) * Fraction(b)
    return _rn_f32(s)


def test_combine_backward_grad_w_is_the_exact_dot_rounded_once():
    """grad_w[t,k] = <grad_out[t], y[slot]>: the exact sum of the H exact
    products, rounded once to fp32 (linearity of combine in w, stakiran
    section 3).  Values are BF16 with exponents in [-4, 4], so every partial
    sum needs at most 40 bits: a double accumulation is exact and the result
    must equal the rounded exact sum, while an fp32 accumulation loses bits
    on almost every dot product."""
    rng = np.random.default_rng(707)
    T, E, K, H = 12, 8, 4, 256
    idx, w = workloads.random_case(70, T, E, K, mask_frac=0.1)
    r = oracle.run_all(idx, w, None, E, 2, False)

    def rows(n):
        m = rng.integers(128, 256, (n, H)).astype(np.float32) / np.float32(128)   # 8-bit significand
        e = np.ldexp(np.float32(1), rng.integers(-4, 5, (n, H))).astype(np.float32)
        sgn = np.where(rng.integers(0, 2, (n, H)) == 1, np.float32(-1), np.float32(1))
        return workloads.bf16_bits_from_f32(m * e * sgn)
    y = rows(r["rows"])
    g = rows(T)
    _, gw = oracle.combine_backward(g, y, r["slot"], w, r["rows"])
    gf, yf = _f32(g), _f32(y)
    f32_chain_differs = 0
    for t in range(T):
        for k in range(K):
            s = r["slot"][t, k]
            if s < 0:
                assert gw[t, k] == 0.0
                continue
            want = _exact_dot_rounded_once(gf[t], yf[s])
            assert gw[t, k] == np.float32(want), (t, k, gw[t, k], want)
            acc = np.float32(0)
            for a, b in zip(gf[t], yf[s]):
                acc = np.float32(acc + np.float32(a * b))
            f32_chain_differs += int(acc != np.float32(want))
    assert f32_chain_differs > 10


def test_combine_backward_grad_w_wide_range_within_double_bound():
    """On wide-range values the double accumulation is no longer exact, but
    its error is at most (H-1) * 2^-53 * sum|g*y| before the final rounding:
    grad_w stays within half an fp32 ulp of the exact sum plus that, a bound
    some 2^29 times tighter than an fp32 accumulation allows."""
    from fractions import Fraction
    rng = np.random.default_rng(808)
    T, E, K, H = 10, 8, 3, 512
    idx, w = workloads.random_case(80, T, E, K)
    r = oracle.run_all(idx, w, None, E, 2, False)
    y = _wide_rows(rng, r["rows"], H)
    g = _wide_rows(rng, T, H)
    _, gw = oracle.combine_backward(g, y, r["slot"], w, r["rows"])
    gf, yf = _f32(g).astype(np.float64), _f32(y).astype(np.float64)
    for t in range(T):
        for k in range(K):
            s = r["slot"][t, k]
            exact = sum((Fraction(a) * Fraction(b) for a, b in zip(gf[t].tolist(), yf[s].tolist())),
                        Fraction(0))
            mag = float(np.abs(gf[t] * yf[s]).sum())
            rn = _rn_f32(exact)
            ulp = float(np.spacing(np.float32(abs(rn)))) if rn != 0 else 2.0 ** -149
            bound = 0.5 * ulp + (H - 1) * 2.0 ** -53 * mag
            assert abs(Fraction(float(gw[t, k])) - exact) <= Fraction(bound), (t, k)


# ----------------------------------------------------------------------------
# expert parallelism over ranks, one rank's share: destination routing, the
# packed rows' metadata, and the flow composed from the pinned functions
# ----------------------------------------------------------------------------

def _brute_rank_routing(idx, E, P):
    """Distinct partitions of each token's dispatched experts, ascending."""
    T, K = idx.shape
    epp = E // P
    valid = _valid_independent(idx, E)
    out = np.full((T, min(K, P)), -1, np.int64)
    for t in range(T):
        parts = sorted({int(idx[t, k]) // epp for k in range(K) if valid[t, k]})
        out[t, :len(parts)] = parts
    return out


EP_SHAPES = [(50, 16, 4, 4), (200, 64, 6, 8), (64, 256, 8, 8), (33, 8, 16, 2), (40, 64, 3, 64), (7, 4, 2, 1)]


def _ep_case(T, E, K, mode, seed):
    kw = {} if mode == "clean" else dict(distinct=False, mask_frac=0.15, invalid_frac=0.05, dup_frac=0.1)
    return workloads.random_case(seed, T, E, K, **kw)


@pytest.mark.parametrize("mode", ["clean", "dirty"])
@pytest.mark.parametrize("T,E,K,P", EP_SHAPES)
def test_rank_routing_against_brute_force(T, E, K, P, mode):
    """part_idx = the ascending distinct destination ranks of each token
    (devtrends.ru "Как это выглядит в коде": is_token_in_rank), checked
    against a set construction and against the layout's own mask."""
    idx, _ = _ep_case(T, E, K, mode, T + E + K + P)
    part = oracle.rank_routing(idx, E, P)
    assert np.array_equal(part, _brute_rank_routing(idx, E, P))
    mask = oracle.layout(idx, E, P)["is_token_in_partition"]
    for t in range(T):
        assert list(part[t][part[t] >= 0]) == list(np.nonzero(mask[t])[0])


@pytest.mark.parametrize("mode", ["clean", "dirty"])
@pytest.mark.parametrize("T,E,K,P", EP_SHAPES)
def test_pack_metadata_against_brute_force(T, E, K, P, mode):
    """Each packed row carries the token's K ids as local ids of its
    destination (-1 for experts elsewhere, masked, out of range or repeated)
    and the matching weights (0 elsewhere); across a token's rows the local
    ids map back to exactly its dispatched experts."""
    idx, w = _ep_case(T, E, K, mode, 3 * T + E + K + P)
    epp = E // P
    part = _brute_rank_routing(idx, E, P)
    Kp = part.shape[1]
    pk = oracle.run_all(part, np.ones((T, Kp), np.float32), None, P, P, False)
    li, lw = oracle.pack_metadata(idx, w, part, pk["slot"], pk["rows"], E, P)
    valid = _valid_independent(idx, E)
    used = np.zeros(pk["rows"], bool)
    for t in range(T):
        got = []
        for j in range(Kp):
            p, r = int(part[t, j]), int(pk["slot"][t, j])
            if p < 0:
                assert r < 0
                continue
            used[r] = True
            for k in range(K):
                e = int(idx[t, k])
                local = bool(valid[t, k]) and e // epp == p
                assert li[r, k] == (e - p * epp if local else -1), (t, j, k)
                assert lw[r, k] == (w[t, k] if local else 0.0), (t, j, k)
                if li[r, k] >= 0:
                    got.append(p * epp + int(li[r, k]))
        assert sorted(got) == sorted(int(idx[t, k]) for k in range(K) if valid[t, k])
    assert np.all(li[~used] == -7) and np.all(lw[~used] == -7.0)
    # destination blocks are contiguous and in rank order, tokens ascending inside
    off = pk["expert_offset"]
    for p in range(P):
        toks = [t for t in range(T) if p in part[t]]
        rows_p = [int(pk["slot"][t, list(part[t]).index(p)]) for t in toks]
        assert rows_p == list(range(int(off[p]), int(off[p + 1])))


@pytest.mark.parametrize("use_fp8", [False, True])
@pytest.mark.parametrize("T,E,K,P", [(60, 16, 4, 4), (130, 64, 6, 8), (33, 32, 8, 2)])
def test_ep_receive_side_reproduces_the_single_level_dispatch(T, E, K, P, use_fp8):
    """One source rank: after the pack, the identity exchange and the unpack,
    destination p holds exactly the rows (and scales) that the single-level
    dispatch puts in the blocks of p's experts, with the same per-expert
    counts (the pages' dispatch over ranks delivers each token's rows to the
    experts it chose)."""
    H = 256
    idx, w = _ep_case(T, E, K, "dirty", 5 * T + E)
    x = workloads.random_rows(T + 11, T, H, "wide")
    epp = E // P
    single = oracle.run_all(idx, w, x, E, P, use_fp8)
    ep_r = oracle.ep_one_source(idx, w, x, E, P, use_fp8)
    for p in range(P):
        u = ep_r["dest"][p]["unpack"]
        a, b = int(single["expert_offset"][p * epp]), int(single["expert_offset"][(p + 1) * epp])
        assert np.array_equal(u["num_tokens_per_expert"], single["num_tokens_per_expert"][p * epp:(p + 1) * epp])
        assert u["rows"] == b - a
        assert np.array_equal(u["recv_x"][:u["rows"]], single["recv_x"][a:b])
        if use_fp8:
            assert np.array_equal(u["recv_scales"][:u["rows"]].view(np.uint32),
                                  single["recv_scales"][a:b].view(np.uint32))


def test_ep_two_level_combine_is_combine_for_one_rank():
    """With P = 1 the expert rank pre-reduces every pair of the token and the
    origin adds one returned row to +0: the result is the single-level
    combine, bit for bit, on wide-range data."""
    T, E, K, H = 90, 32, 6, 256
    idx, w = _ep_case(T, E, K, "dirty", 17)
    x = workloads.random_rows(18, T, H, "normal")
    single = oracle.run_all(idx, w, x, E, 1, False)
    y = workloads.random_rows(19, max(single["rows"], 1), H, "wide")[:single["rows"]]
    ep_r = oracle.ep_one_source(idx, w, x, E, 1, False, y_parts=[y])
    assert np.array_equal(ep_r["out"], oracle.combine(y, single["slot"], w))


@pytest.mark.parametrize("T,E,K,P", [(64, 32, 6, 4), (40, 64, 8, 8)])
def test_ep_two_level_combine_exact_on_small_integers(T, E, K, P):
    """Expert outputs in {-3..3} and weights in {1/2, 1, 2} keep every
    product, partial row and sum exact (|sum| <= 48 in steps of 1/2 needs at
    most 7 significant bits, within BF16's 8): the origin's sum in rank order
    of the per-rank partial rows equals the single-level combine, which equals
    the exact sum (each expert's output row is the same whichever path sends
    it)."""
    H = 128
    rng = np.random.default_rng(T + K)
    idx, _ = workloads.random_case(T, T, E, K, mask_frac=0.1)
    w = np.array([0.5, 1.0, 2.0], np.float32)[rng.integers(0, 3, (T, K))]
    x = workloads.random_rows(T + 1, T, H, "normal")
    epp = E // P
    single = oracle.run_all(idx, w, x, E, P, False)
    y = _small_int_bf16(rng, (max(single["rows"], 1), H))[:single["rows"]]
    off = single["expert_offset"]
    y_parts = [y[int(off[p * epp]):int(off[(p + 1) * epp])] for p in range(P)]
    ep_r = oracle.ep_one_source(idx, w, x, E, P, False, y_parts=y_parts)
    want = oracle.combine(y, single["slot"], w)
    assert np.array_equal(ep_r["out"], want)
    exact = np.zeros((T, H))
    yf = _f32(y).astype(np.float64)
    for t in range(T):
        for k in range(K):
            s = single["slot"][t, k]
            if s >= 0:
                exact[t] += float(w[t, k]) * yf[s]
    assert np.array_equal(_f32(want).astype(np.float64), exact)
