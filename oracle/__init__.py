"""CPU oracle for MoE dispatch / combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never do; the two share no code.

This wrapper only marshals numpy arrays into ``liboracle.so`` (built from
``oracle.c`` with gcc, ``-O2 -ffp-contract=off``); the arithmetic is in C.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        L.oracle_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_e4m3fn_rne_sat.argtypes = [ctypes.c_float]
        L.oracle_e4m3fn_rne_sat.restype = ctypes.c_uint8
        L.oracle_e4m3fn_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_to_f32.restype = ctypes.c_float
        L.oracle_e4m3fn_encode_array.argtypes = [P, P, ctypes.c_int64]
        L.oracle_e4m3fn_encode_array.restype = None
        L.oracle_quant_block.argtypes = [P, P, P]
        L.oracle_quant_block.restype = None
        L.oracle_layout.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_layout.restype = i32
        L.oracle_expert_offsets.argtypes = [P, i32, P]
        L.oracle_expert_offsets.restype = None
        L.oracle_expert_offsets_aligned.argtypes = [P, i32, i32, P]
        L.oracle_expert_offsets_aligned.restype = None
        L.oracle_dispatch_fp8_input.argtypes = [P, P, i32, i32, i32, P, P, P]
        L.oracle_dispatch_fp8_input.restype = None
        L.oracle_slots.argtypes = [P, P, i32, i32, P, i32, i32, P, P, P]
        L.oracle_slots.restype = None
        L.oracle_slots_static.argtypes = [P, P, i32, i32, i32, i32, P, P]
        L.oracle_slots_static.restype = None
        L.oracle_dispatch.argtypes = [P, i32, i32, i32, P, i32, P, P]
        L.oracle_dispatch.restype = None
        L.oracle_combine.argtypes = [P, i32, i32, i32, P, P, P]
        L.oracle_combine.restype = None
        L.oracle_combine_fp8.argtypes = [P, P, i32, i32, i32, P, P, P]
        L.oracle_combine_fp8.restype = None
        L.oracle_dispatch_backward.argtypes = [P, i32, i32, i32, P, P]
        L.oracle_dispatch_backward.restype = None
        L.oracle_combine_backward.argtypes = [P, P, i32, i32, i32, P, P, P, P]
        L.oracle_combine_backward.restype = None
        L.oracle_rank_routing.argtypes = [P, i32, i32, i32, i32, P]
        L.oracle_rank_routing.restype = None
        L.oracle_pack_metadata.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P]
        L.oracle_pack_metadata.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# -- codec -------------------------------------------------------------------

def bf16_rne(f: float) -> int:
    return int(lib().oracle_bf16_rne(float(f)))


def e4m3fn(v: float) -> int:
    return int(lib().oracle_e4m3fn_rne_sat(float(v)))


def e4m3fn_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    q = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3fn_encode_array(_p(v), _p(q), v.size)
    return q


def e4m3fn_decode(q: int) -> float:
    return float(lib().oracle_e4m3fn_to_f32(int(q)))


def quant_block(x128_bits: np.ndarray):
    x = _c(x128_bits, np.uint16)
    assert x.size == 128
    q = np.empty(128, dtype=np.uint8)
    s = np.empty(1, dtype=np.float32)
    lib().oracle_quant_block(_p(x), _p(q), _p(s))
    return q, np.float32(s[0])


# -- the path ----------------------------------------------------------------

def layout(topk_idx: np.ndarray, E: int, P: int):
    """Returns dict(num_tokens_per_expert, num_tokens_per_partition,
    is_token_in_partition [T,P] uint8, num_invalid int, valid [T,K] uint8)."""
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    cnt = np.empty(E, np.int32)
    pc = np.empty(P, np.int32)
    mask = np.empty((T, P), np.uint8)
    ninv = np.empty(1, np.int32)
    valid = np.empty((T, K), np.uint8)
    rc = lib().oracle_layout(_p(idx), T, K, E, P, _p(cnt), _p(pc), _p(mask), _p(ninv), _p(valid))
    if rc != 0:
        raise ValueError("oracle_layout: invalid dimensions")
    return dict(num_tokens_per_expert=cnt, num_tokens_per_partition=pc,
                is_token_in_partition=mask, num_invalid=int(ninv[0]), valid=valid)


def expert_offsets(cnt: np.ndarray, align: int = 1) -> np.ndarray:
    """Exclusive prefix sum of the counts; align > 1 rounds each expert's block
    up to a multiple of align (GEMM-aligned layout)."""
    cnt = _c(cnt, np.int32)
    off = np.empty(cnt.size + 1, np.int32)
    if align == 1:
        lib().oracle_expert_offsets(_p(cnt), cnt.size, _p(off))
    else:
        lib().oracle_expert_offsets_aligned(_p(cnt), cnt.size, align, _p(off))
    return off


def slots(topk_idx: np.ndarray, valid: np.ndarray, off: np.ndarray, capacity: int):
    """Returns (slot [T,K] int32, src_token [capacity] int32 (-1 where unset), overflow int)."""
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    valid = _c(valid, np.uint8)
    off = _c(off, np.int32)
    E = off.size - 1
    slot = np.empty((T, K), np.int32)
    src = np.full(max(capacity, 1), -1, np.int32)
    ovf = np.zeros(1, np.int32)
    lib().oracle_slots(_p(idx), _p(valid), T, K, _p(off), E, capacity, _p(slot), _p(src), _p(ovf))
    return slot, src[:capacity], int(ovf[0])


def slots_static(topk_idx: np.ndarray, valid: np.ndarray, E: int, cap: int):
    """Low-latency layout: returns (slot [T,K] int32, overflow int)."""
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    valid = _c(valid, np.uint8)
    slot = np.empty((T, K), np.int32)
    ovf = np.zeros(1, np.int32)
    lib().oracle_slots_static(_p(idx), _p(valid), T, K, E, cap, _p(slot), _p(ovf))
    return slot, int(ovf[0])


def run_low_latency(topk_idx, topk_weights, x_bits, E, P, use_fp8, cap):
    """The low-latency path on the CPU: layout counts, static-capacity slots
    and the permute into E*cap rows (unused rows stay zero)."""
    lay = layout(topk_idx, E, P)
    slot, ovf = slots_static(topk_idx, lay["valid"], E, cap)
    res = dict(lay, slot=slot, overflow=ovf, rows=E * cap)
    if x_bits is not None:
        recv, scales = dispatch(x_bits, slot, E * cap, use_fp8)
        res.update(recv_x=recv, recv_scales=scales)
    return res


def dispatch(x_bits: np.ndarray, slot: np.ndarray, rows: int, use_fp8: bool):
    """Returns (recv [rows,H] uint8|uint16, scales [rows,H/128] fp32 or None).
    Rows that no pair maps to are left zero."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    slot = _c(slot, np.int32)
    K = slot.shape[1]
    if use_fp8:
        recv = np.zeros((rows, H), np.uint8)
        scales = np.zeros((rows, H // 128), np.float32)
        lib().oracle_dispatch(_p(x), T, H, K, _p(slot), 1, _p(recv), _p(scales))
        return recv, scales
    recv = np.zeros((rows, H), np.uint16)
    lib().oracle_dispatch(_p(x), T, H, K, _p(slot), 0, _p(recv), None)
    return recv, None


def dispatch_fp8_input(xq: np.ndarray, xs: np.ndarray, slot: np.ndarray, rows: int):
    """Pre-quantised rows: returns (recv uint8 [rows,H], scales fp32 [rows,H/128]),
    rows no pair maps to left zero."""
    xq = _c(xq, np.uint8)
    xs = _c(xs, np.float32)
    slot = _c(slot, np.int32)
    T, H = xq.shape
    K = slot.shape[1]
    recv = np.zeros((rows, H), np.uint8)
    scales = np.zeros((rows, H // 128), np.float32)
    lib().oracle_dispatch_fp8_input(_p(xq), _p(xs), T, H, K, _p(slot), _p(recv), _p(scales))
    return recv, scales


def combine(y_bits: np.ndarray, slot: np.ndarray, w: np.ndarray) -> np.ndarray:
    y = _c(y_bits, np.uint16)
    slot = _c(slot, np.int32)
    w = _c(w, np.float32)
    T, K = slot.shape
    H = y.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().oracle_combine(_p(y), T, H, K, _p(slot), _p(w), _p(out))
    return out


def combine_fp8(q: np.ndarray, scales: np.ndarray, slot: np.ndarray, w) -> np.ndarray:
    """Combine of FP8 rows (codes uint8 [rows,H], scales fp32 [rows,H/128]);
    w None = unit weights.  Returns bf16 bits [T,H]."""
    q = _c(q, np.uint8)
    sc = _c(scales, np.float32)
    slot = _c(slot, np.int32)
    T, K = slot.shape
    H = q.shape[1]
    wv = None if w is None else _c(w, np.float32)
    out = np.empty((T, H), np.uint16)
    lib().oracle_combine_fp8(_p(q), _p(sc), T, H, K, _p(slot), None if wv is None else _p(wv), _p(out))
    return out


def dispatch_backward(grad_recv_bits: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """grad_x [T,H] bf16 bits from grad_recv [rows,H] bf16 bits."""
    g = _c(grad_recv_bits, np.uint16)
    slot = _c(slot, np.int32)
    T, K = slot.shape
    H = g.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().oracle_dispatch_backward(_p(g), T, H, K, _p(slot), _p(out))
    return out


def combine_backward(grad_out_bits: np.ndarray, y_bits, slot: np.ndarray, w: np.ndarray,
                     rows: int, fill: int = 0):
    """Returns (grad_y [rows,H] bf16 bits, rows nobody maps to = fill;
    grad_w [T,K] fp32 or None when y_bits is None)."""
    g = _c(grad_out_bits, np.uint16)
    slot = _c(slot, np.int32)
    w = _c(w, np.float32)
    T, K = slot.shape
    H = g.shape[1]
    grad_y = np.full((rows, H), fill, np.uint16)
    y = None if y_bits is None else _c(y_bits, np.uint16)
    grad_w = None if y is None else np.empty((T, K), np.float32)
    lib().oracle_combine_backward(_p(g), None if y is None else _p(y), T, H, K, _p(slot), _p(w),
                                  _p(grad_y), None if grad_w is None else _p(grad_w))
    return grad_y, grad_w


def rank_routing(topk_idx: np.ndarray, E: int, P: int) -> np.ndarray:
    """Destination ranks of each token: int64 [T, min(K, P)], the distinct
    partitions of its dispatched experts, ascending, then -1."""
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    Kp = min(K, P)
    out = np.empty((T, Kp), np.int64)
    lib().oracle_rank_routing(_p(idx), T, K, E, P, _p(out))
    return out


def pack_metadata(topk_idx: np.ndarray, topk_weights: np.ndarray, part_idx: np.ndarray,
                  slot_pack: np.ndarray, rows: int, E: int, P: int, fill_idx: int = -7,
                  fill_w: float = -7.0):
    """Metadata of the packed rows: (local_idx int64 [rows, K], local_w fp32
    [rows, K]); rows no pair maps to keep the fill values."""
    idx = _c(topk_idx, np.int64)
    w = _c(topk_weights, np.float32)
    part = _c(part_idx, np.int64)
    sp = _c(slot_pack, np.int32)
    T, K = idx.shape
    local_idx = np.full((rows, K), fill_idx, np.int64)
    local_w = np.full((rows, K), fill_w, np.float32)
    lib().oracle_pack_metadata(_p(idx), _p(w), _p(part), _p(sp), T, K, E, P, _p(local_idx), _p(local_w))
    return local_idx, local_w


def run_all(topk_idx, topk_weights, x_bits, E, P, use_fp8, capacity=None, y_bits=None, align=1):
    """The whole path on the CPU: layout, offsets, slots, dispatch and, when
    y_bits is given, combine.  Returns a dict of every intermediate.  With
    align > 1 the receive layout is GEMM-aligned; the default capacity is then
    the worst case T*K + E*(align-1)."""
    T, K = topk_idx.shape
    lay = layout(topk_idx, E, P)
    off = expert_offsets(lay["num_tokens_per_expert"], align)
    cap = T * K + E * (align - 1) if capacity is None else capacity
    slot, src, ovf = slots(topk_idx, lay["valid"], off, cap)
    N = int(lay["num_tokens_per_expert"].sum())        # dispatched pairs
    rows = min(int(off[-1]), cap)                      # receive rows (padding included)
    res = dict(lay, expert_offset=off, slot=slot, src_token=src[:rows], overflow=ovf, N=N, rows=rows)
    if x_bits is not None:
        recv, scales = dispatch(x_bits, slot, rows, use_fp8)
        res.update(recv_x=recv, recv_scales=scales)
    if y_bits is not None:
        res["out"] = combine(y_bits, slot, topk_weights)
    return res


def ep_one_source(topk_idx, topk_weights, x_bits, E, P, use_fp8, y_parts=None):
    """The expert-parallel flow over P ranks for one source rank's tokens,
    composed from the functions above (every exchange between ranks is the
    identity here: destination p receives the packed block p).

    Sender: rank_routing, then the packed rows are the dispatch of the
    rows along part_idx (E' = P experts, one per destination, so each token
    lands once per destination, ascending token), with their metadata.
    Receiver p: layout and dispatch of its block along the local ids (E/P
    local experts, one partition), the received rows taken as they are.
    With y_parts (list of bf16 rows per destination, in p's receive order):
    partial rows = combine with the received weights, and the origin's
    result = the unit-weight sum of the returned rows in rank order.
    Returns a dict of every intermediate."""
    T, K = topk_idx.shape
    epp = E // P
    part = rank_routing(topk_idx, E, P)
    Kp = part.shape[1]
    pk = run_all(part, np.ones((T, Kp), np.float32), x_bits, P, P, use_fp8)
    slot_pack = pk["slot"]
    rows = pk["rows"]
    local_idx, local_w = pack_metadata(topk_idx, topk_weights, part, slot_pack, rows, E, P)
    off = pk["expert_offset"]
    res = dict(part_idx=part, pack=pk, local_idx=local_idx, local_w=local_w, dest=[])
    partials = np.zeros((rows, x_bits.shape[1] if x_bits is not None else 0), np.uint16)
    for p in range(P):
        r0, r1 = int(off[p]), int(off[p + 1])
        li = np.ascontiguousarray(local_idx[r0:r1])
        lw = np.ascontiguousarray(local_w[r0:r1])
        d = dict(rows=(r0, r1))
        if x_bits is not None:
            if use_fp8:
                ru = run_all(li, lw, None, epp, 1, True)
                recv, scales = dispatch_fp8_input(pk["recv_x"][r0:r1], pk["recv_scales"][r0:r1], ru["slot"],
                                                  ru["rows"])
                ru.update(recv_x=recv, recv_scales=scales)
            else:
                ru = run_all(li, lw, pk["recv_x"][r0:r1], epp, 1, False)
            d["unpack"] = ru
            if y_parts is not None:
                d["partial"] = combine(y_parts[p], ru["slot"], lw)
                partials[r0:r1] = d["partial"]
        res["dest"].append(d)
    if y_parts is not None:
        res["partials"] = partials
        res["out"] = dispatch_backward(partials, slot_pack)
    return res
