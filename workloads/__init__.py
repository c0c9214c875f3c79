"""Seeded synthetic inputs for MoE dispatch / combine.

This module only draws inputs: routing (``topk_idx``, ``topk_weights``), token
rows ``x`` and expert-output rows ``y``.  It holds none of the dispatch /
combine arithmetic, so both the CPU oracle and the HIP path can be fed from it
without sharing any of the method's code.

Everything is drawn with numpy's PCG64 generator from a ``SeedSequence`` of
``(seed, substream)``; each quantity has its own substream so that changing one
draw never shifts another.  BF16 values are produced by drawing fp32 and
rounding to bfloat16 with torch's CPU conversion (round to nearest even); they
are returned as raw ``uint16`` bit patterns.

Workloads (the shapes follow the DeepEP pages; routing details that the pages
leave open are this module's stated choices):

* ``tiny``   T=128  H=256  E=16  K=2 P=4,  BF16 dispatch.  Softmax of N(0,1)
  logits, top-2, weights renormalised to sum 1.
* ``decode`` T=128  H=7168 E=256 K=8 P=8,  FP8 dispatch.  Same routing as
  ``tiny`` with top-8 (the decode batch of 128 tokens quoted for the
  low-latency kernels on devtrends.ru, "Производительность на практике").
* ``v3``     T=8192 H=7168 E=256 K=8 P=8,  FP8 dispatch.  The V3 benchmark
  shape (8K tokens, hidden 7168, top-8, FP8 dispatch / BF16 combine; GeekNews
  page, "Kết quả đo hiệu năng").  DeepSeek-V3 style group-limited gating: sigmoid
  scores, 8 groups of 32 experts scored by their maximum, top-4 groups kept,
  top-8 experts among those 128, chosen scores renormalised.  The 8 logical
  partitions coincide with the 8 groups.
* ``skewed`` T=4096 H=4096 E=64  K=6 P=8,  BF16 dispatch.  Expert popularity
  p(e) ~ (rank(e)+1)^-1.2 with rank from a seeded permutation; 6 distinct
  experts per token drawn sequentially without replacement (Plackett-Luce, via
  Gumbel top-k); exactly floor(0.05*T*K) entries set to -1; weights softmax of
  N(0,1) logits over the 6 chosen, masked ones zeroed, the rest renormalised.
* ``large``  T=16384 H=7168 E=256 K=8 P=16, FP8 dispatch.  8 distinct experts
  uniformly at random per token; weights Dirichlet(1) (normalised -ln u).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "config", "make", "expert_outputs", "random_case",
    "random_rows", "bf16_bits_from_f32", "f32_from_bf16_bits",
]

# substream ids
_S_X, _S_ROUTE, _S_WEIGHT, _S_MASK, _S_Y, _S_PERM = range(6)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    K: int
    P: int
    use_fp8: bool
    seed: int
    routing: str
    mask_frac: float = 0.0


CONFIGS = {
    "tiny": Workload("tiny", 128, 256, 16, 2, 4, False, 1, "softmax"),
    "decode": Workload("decode", 128, 7168, 256, 8, 8, True, 2, "softmax"),
    "v3": Workload("v3", 8192, 7168, 256, 8, 8, True, 3, "group_limited"),
    "skewed": Workload("skewed", 4096, 4096, 64, 6, 8, False, 4, "zipf", 0.05),
    "large": Workload("large", 16384, 7168, 256, 8, 16, True, 5, "uniform_dirichlet"),
}


def config(name: str) -> Workload:
    return CONFIGS[name]


def _rng(seed: int, sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(sub)])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), using torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 1024) -> np.ndarray:
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = bf16_bits_from_f32(rng.standard_normal((r1 - r0, cols), dtype=np.float32))
    return out


def _topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    # descending by score, ties broken toward the lower expert id
    return np.argsort(-scores, axis=1, kind="stable")[:, :k]


def _route_softmax(w: Workload):
    rng = _rng(w.seed, _S_ROUTE)
    logits = rng.standard_normal((w.T, w.E))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    probs = z / z.sum(axis=1, keepdims=True)
    idx = _topk_desc(probs, w.K)
    sel = np.take_along_axis(probs, idx, axis=1)
    weights = sel / sel.sum(axis=1, keepdims=True)
    return idx.astype(np.int64), weights.astype(np.float32)


def _route_group_limited(w: Workload, n_groups: int = 8, topk_groups: int = 4):
    rng = _rng(w.seed, _S_ROUTE)
    logits = rng.standard_normal((w.T, w.E))
    scores = 1.0 / (1.0 + np.exp(-logits))
    gsize = w.E // n_groups
    gscore = scores.reshape(w.T, n_groups, gsize).max(axis=2)
    keep = _topk_desc(gscore, topk_groups)
    gmask = np.zeros((w.T, n_groups), dtype=bool)
    np.put_along_axis(gmask, keep, True, axis=1)
    masked = np.where(np.repeat(gmask, gsize, axis=1), scores, -np.inf)
    idx = _topk_desc(masked, w.K)
    sel = np.take_along_axis(scores, idx, axis=1)
    weights = sel / sel.sum(axis=1, keepdims=True)
    return idx.astype(np.int64), weights.astype(np.float32)


def _route_zipf(w: Workload, s: float = 1.2):
    prng = _rng(w.seed, _S_PERM)
    perm = prng.permutation(w.E)
    rank = np.empty(w.E, dtype=np.int64)
    rank[perm] = np.arange(w.E)
    logp = -s * np.log(rank + 1.0)
    rng = _rng(w.seed, _S_ROUTE)
    gumbel = -np.log(-np.log(rng.random((w.T, w.E))))
    idx = _topk_desc(logp[None, :] + gumbel, w.K).astype(np.int64)
    mrng = _rng(w.seed, _S_MASK)
    n_mask = int(np.floor(w.mask_frac * w.T * w.K))
    flat = mrng.choice(w.T * w.K, size=n_mask, replace=False)
    idx.reshape(-1)[flat] = -1
    wrng = _rng(w.seed, _S_WEIGHT)
    lg = wrng.standard_normal((w.T, w.K))
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    z[idx < 0] = 0.0
    tot = z.sum(axis=1, keepdims=True)
    weights = np.divide(z, tot, out=np.zeros_like(z), where=tot > 0)
    return idx, weights.astype(np.float32)


def _route_uniform_dirichlet(w: Workload):
    rng = _rng(w.seed, _S_ROUTE)
    keys = rng.random((w.T, w.E))
    idx = np.argsort(keys, axis=1, kind="stable")[:, :w.K].astype(np.int64)
    wrng = _rng(w.seed, _S_WEIGHT)
    g = -np.log(1.0 - wrng.random((w.T, w.K)))
    weights = g / g.sum(axis=1, keepdims=True)
    return idx, weights.astype(np.float32)


_ROUTERS = {
    "softmax": _route_softmax,
    "group_limited": _route_group_limited,
    "zipf": _route_zipf,
    "uniform_dirichlet": _route_uniform_dirichlet,
}


def make(w: Workload | str, with_x: bool = True):
    """Return ``(topk_idx int64 [T,K], topk_weights fp32 [T,K], x uint16 [T,H] or None)``."""
    if isinstance(w, str):
        w = CONFIGS[w]
    idx, weights = _ROUTERS[w.routing](w)
    x = _normal_bf16(_rng(w.seed, _S_X), (w.T, w.H)) if with_x else None
    return np.ascontiguousarray(idx), np.ascontiguousarray(weights), x


def expert_outputs(w: Workload | str, rows: int, seed_offset: int = 0) -> np.ndarray:
    """Synthetic expert-output rows ``y`` (bf16 bits, [rows, H]), N(0,1)."""
    if isinstance(w, str):
        w = CONFIGS[w]
    return _normal_bf16(_rng(w.seed + 1000003 * seed_offset, _S_Y), (rows, w.H))


def random_rows(seed: int, rows: int, H: int, kind: str = "normal") -> np.ndarray:
    """BF16 rows of a chosen value mix (bits, [rows, H]).

    kinds: ``normal`` N(0,1); ``wide`` N(0,1) scaled by 2^U{-30..30} per
    128-channel block; ``bits`` uniformly random finite bf16 bit patterns;
    ``zeros`` all +0 / -0; ``subnormal`` bf16 subnormals mixed with zeros;
    ``ties`` values whose scaled fp8 image lands on rounding ties.
    """
    rng = _rng(seed, _S_X)
    if kind == "normal":
        return _normal_bf16(rng, (rows, H))
    if kind == "wide":
        v = rng.standard_normal((rows, H // 128, 128), dtype=np.float32)
        sc = np.ldexp(np.float32(1.0), rng.integers(-30, 31, (rows, H // 128, 1))).astype(np.float32)
        return bf16_bits_from_f32((v * sc).reshape(rows, H))
    if kind == "bits":
        b = rng.integers(0, 1 << 16, (rows, H), dtype=np.uint32).astype(np.uint16)
        exp_all_ones = (b & 0x7F80) == 0x7F80
        b[exp_all_ones] &= np.uint16(0xBFFF)  # clear top exponent bit -> finite
        return b
    if kind == "zeros":
        return (rng.integers(0, 2, (rows, H), dtype=np.uint32).astype(np.uint16) << 15).astype(np.uint16)
    if kind == "subnormal":
        mant = rng.integers(0, 128, (rows, H), dtype=np.uint32).astype(np.uint16)
        sign = (rng.integers(0, 2, (rows, H), dtype=np.uint32).astype(np.uint16) << 15).astype(np.uint16)
        return (mant | sign).astype(np.uint16)
    if kind == "ties":
        # amax fixed to 448 in every block (so the block scale is exactly 1),
        # remaining values are E4M3 midpoints, which are exact in bf16 for the
        # upper binades.
        mids = np.array([m for m in (
            [(2 * j + 1) * 2.0 ** -10 for j in range(8)] +
            [(1 + (2 * j + 1) / 16) * 2.0 ** e for e in range(-6, 8) for j in range(8)])], dtype=np.float32)
        v = rng.choice(mids, size=(rows, H)).astype(np.float32)
        v *= np.where(rng.integers(0, 2, (rows, H)) == 1, np.float32(-1), np.float32(1))
        v.reshape(rows, H // 128, 128)[:, :, 0] = 448.0
        return bf16_bits_from_f32(v)
    raise ValueError(kind)


def random_case(seed: int, T: int, E: int, K: int, *, distinct: bool = True,
                mask_frac: float = 0.0, invalid_frac: float = 0.0, dup_frac: float = 0.0,
                weights: str = "dirichlet") -> tuple[np.ndarray, np.ndarray]:
    """Random routing for edge-case tests.

    ``distinct`` draws K distinct experts per token (needs K <= E), else K
    independent draws (duplicates possible).  ``mask_frac`` of the entries are
    set to a negative id (-1 or another negative value), ``invalid_frac`` to an
    id >= E, ``dup_frac`` to a copy of an earlier entry of the same row.
    """
    rng = _rng(seed, _S_ROUTE)
    if distinct and K <= E:
        idx = np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :K].astype(np.int64)
    else:
        idx = rng.integers(0, E, (T, K)).astype(np.int64)
    flat = idx.reshape(-1)
    n = flat.size
    u = rng.random(n)
    if dup_frac > 0 and K > 1:
        kk = np.arange(n) % K
        pick = (u < dup_frac) & (kk > 0)
        src = np.arange(n) - 1 - (rng.integers(0, 1 << 30, n) % np.maximum(kk, 1))
        flat[pick] = flat[src[pick]]
    u2 = rng.random(n)
    inv = u2 < invalid_frac
    flat[inv] = E + rng.integers(0, 3 * E + 7, int(inv.sum()))
    u3 = rng.random(n)
    msk = u3 < mask_frac
    negs = np.array([-1, -1, -1, -2, -7, -(1 << 40)], dtype=np.int64)
    flat[msk] = negs[rng.integers(0, negs.size, int(msk.sum()))]
    wr = _rng(seed, _S_WEIGHT)
    if weights == "dirichlet":
        g = -np.log(1.0 - wr.random((T, K)))
        w = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    elif weights == "ones":
        w = np.ones((T, K), dtype=np.float32)
    elif weights == "pow2":
        w = np.ldexp(np.float32(1.0), wr.integers(-3, 2, (T, K))).astype(np.float32)
    else:
        raise ValueError(weights)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)
