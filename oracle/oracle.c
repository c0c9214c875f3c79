/*
 * CPU oracle for MoE dispatch / combine -- TEST INFRASTRUCTURE ONLY.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Plain definitions, single thread, no blocking or reordering.  The pages
 * (four web summaries of DeepEP) state the interface and the problem but not
 * the kernels' internals; each function names the passage it follows and the
 * reading taken where the pages are silent.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------
 * BF16.  bfloat16 is the upper half of an IEEE binary32.  Widening is a shift;
 * narrowing rounds to nearest, ties to even, on the 16 dropped bits.  Inputs
 * are finite by contract (the combine operands are finite BF16 rows and
 * finite fp32 weights).
 * ------------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;          /* parity of the kept part     */
    uint32_t r = u + 0x7FFFu + lsb;         /* > half rounds up, == half to even */
    return (uint16_t)(r >> 16);
}

/* ---------------------------------------------------------------------------
 * FP8.  The pages say only "FP8 dispatch" (aikraft.ru, "Технические детали и
 * требования").  Reading taken: OCP E4M3FN -- 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN, largest finite 448.
 * Values: subnormals m * 2^-9 (m = 1..7); normals (1 + m/8) * 2^(e-7) for
 * e = 1..15, m = 0..7, except (15, 7).  Rounding to nearest, ties to even,
 * saturating to +-448 (never NaN) and keeping the sign of zero.
 * ------------------------------------------------------------------------ */
float oracle_e4m3fn_to_f32(uint8_t q)
{
    int sign = q >> 7;
    int e = (q >> 3) & 0xF;
    int m = q & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(sign ? -v : v);
}

uint8_t oracle_e4m3fn_rne_sat(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;                 /* satfinite: +-448            */
    if (a == 0.0)
        return sign;
    /* a = f * 2^ex with f in [0.5, 1): the binade [2^(ex-1), 2^ex) has a
     * spacing of 2^(ex-1-3) between E4M3 values; below 2^-6 the spacing stays
     * at the subnormal quantum 2^-9. */
    int ex;
    frexp(a, &ex);
    int lead = ex - 1;                      /* a in [2^lead, 2^(lead+1))  */
    if (lead < -6)
        lead = -6;
    double quantum = ldexp(1.0, lead - 3);
    /* a / quantum is exact (power-of-two scaling of a double holding an
     * fp32); nearbyint rounds it to the nearest integer, ties to even, in the
     * default rounding mode. */
    double n = nearbyint(a / quantum);
    double r = n * quantum;                 /* the rounded magnitude, exact */
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6))                 /* subnormal: r = n * 2^-9    */
        return sign | (uint8_t)n;
    int rex;
    double rf = frexp(r, &rex);             /* r = rf * 2^rex, rf in [0.5,1) */
    int ebits = (rex - 1) + 7;              /* biased exponent            */
    int mbits = (int)((rf * 2.0 - 1.0) * 8.0);  /* exact: 3 fraction bits  */
    return sign | (uint8_t)((ebits << 3) | mbits);
}

void oracle_e4m3fn_encode_array(const float* v, uint8_t* q, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = oracle_e4m3fn_rne_sat(v[i]);
}

/* One 128-channel block: amax -> scale s = amax / 448, codes of x * (448 /
 * amax).  The scale convention (per token, per 128 channels, fp32, amax/448)
 * is a stated choice; the pages give only "FP8 dispatch".  Readings: the
 * division is done once per block as inv = 448 / a (correctly rounded fp32)
 * and each value is multiplied by inv (one rounded fp32 product); a =
 * max(amax, 2^-64) keeps inv finite for all-zero blocks. */
void oracle_quant_block(const uint16_t* x128, uint8_t* q128, float* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i) {
        float m = fabsf(oracle_bf16_to_f32(x128[i]));
        if (m > amax)
            amax = m;
    }
    float a = amax > ldexpf(1.0f, -64) ? amax : ldexpf(1.0f, -64);
    float inv = 448.0f / a;
    float s = a / 448.0f;
    for (int i = 0; i < 128; ++i) {
        float p = oracle_bf16_to_f32(x128[i]) * inv;
        q128[i] = oracle_e4m3fn_rne_sat(p);
    }
    *scale = s;
}

/* ---------------------------------------------------------------------------
 * Layout: get_dispatch_layout turns topk_idx into per-destination counts that
 * dispatch consumes (stakiran summary, section 3, training/prefill forward
 * flow; devtrends.ru, "Как это выглядит в коде", the num_tokens_per_rank
 * argument), and per-expert counts are what the grouped GEMM needs (GeekNews,
 * usage section).
 * Readings: destination partitions are contiguous blocks of E/P experts; a
 * negative id is masked; an id >= E, or an id already seen earlier in the same
 * row, is invalid and counted in num_invalid; num_tokens_per_expert counts
 * (token, k) pairs; num_tokens_per_partition counts distinct tokens with at
 * least one valid pair in the partition (a token goes to a rank once).
 * ------------------------------------------------------------------------ */
int oracle_layout(const int64_t* topk_idx, int T, int K, int E, int P,
                  int32_t* num_tokens_per_expert, int32_t* num_tokens_per_partition,
                  uint8_t* is_token_in_partition, int32_t* num_invalid,
                  uint8_t* valid)
{
    if (T < 0 || K < 1 || E < 1 || P < 1 || E % P != 0)
        return -1;
    int epp = E / P;
    for (int e = 0; e < E; ++e)
        num_tokens_per_expert[e] = 0;
    for (int p = 0; p < P; ++p)
        num_tokens_per_partition[p] = 0;
    int32_t ninv = 0;
    uint8_t* seen = (uint8_t*)calloc((size_t)E, 1);
    for (int t = 0; t < T; ++t) {
        for (int p = 0; p < P; ++p)
            is_token_in_partition[(size_t)t * P + p] = 0;
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            uint8_t ok = 0;
            if (e < 0) {
                ok = 0;                               /* masked          */
            } else if (e >= E || seen[e]) {
                ok = 0;                               /* invalid         */
                ninv++;
            } else {
                ok = 1;
                seen[e] = 1;
                num_tokens_per_expert[e]++;
                is_token_in_partition[(size_t)t * P + e / epp] = 1;
            }
            valid[(size_t)t * K + k] = ok;
        }
        for (int k = 0; k < K; ++k) {                 /* reset row marks */
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e >= 0 && e < E)
                seen[e] = 0;
        }
        for (int p = 0; p < P; ++p)
            num_tokens_per_partition[p] += is_token_in_partition[(size_t)t * P + p];
    }
    free(seen);
    *num_invalid = ninv;
    return 0;
}

/* The receive buffer is expert-contiguous (experts in ascending id, no
 * padding), so expert e's rows start at the exclusive prefix sum of the
 * counts of experts 0..e-1. */
void oracle_expert_offsets(const int32_t* num_tokens_per_expert, int E, int32_t* off)
{
    off[0] = 0;
    for (int e = 0; e < E; ++e)
        off[e + 1] = off[e] + num_tokens_per_expert[e];
}

/* GEMM-aligned variant: each expert's block of rows is its count rounded up
 * to a multiple of A, so every block starts on a multiple of A (the grouped
 * GEMM's row tile).  The rows of a block past its count are padding. */
void oracle_expert_offsets_aligned(const int32_t* num_tokens_per_expert, int E, int A, int32_t* off)
{
    off[0] = 0;
    for (int e = 0; e < E; ++e) {
        int32_t c = num_tokens_per_expert[e];
        off[e + 1] = off[e] + ((c + A - 1) / A) * A;
    }
}

/* Every valid (token, k) pair gets one receive row.  Reading: rows of one
 * expert are ordered by ascending source token (a stable counting sort of the
 * pairs by expert id), which makes the assignment deterministic.  A pair whose
 * row index reaches the caller's capacity is dropped and flagged. */
void oracle_slots(const int64_t* topk_idx, const uint8_t* valid, int T, int K,
                  const int32_t* off, int E, int capacity,
                  int32_t* slot, int32_t* src_token, int32_t* overflow)
{
    int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e)
        cur[e] = off[e];
    *overflow = 0;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            if (!valid[i]) {
                slot[i] = -1;
                continue;
            }
            int e = (int)topk_idx[i];
            int32_t s = cur[e]++;
            if (s < capacity) {
                slot[i] = s;
                src_token[s] = t;
            } else {
                slot[i] = -1;
                *overflow = 1;
            }
        }
    }
    free(cur);
}

/* Low-latency layout: each expert has a fixed block of cap rows, filled in
 * ascending token order. */
void oracle_slots_static(const int64_t* topk_idx, const uint8_t* valid, int T, int K, int E,
                         int cap, int32_t* slot, int32_t* overflow)
{
    int32_t* cur = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
    *overflow = 0;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            if (!valid[i]) {
                slot[i] = -1;
                continue;
            }
            int e = (int)topk_idx[i];
            int32_t r = cur[e]++;
            if (r < cap) {
                slot[i] = (int32_t)e * cap + r;
            } else {
                slot[i] = -1;
                *overflow = 1;
            }
        }
    }
    free(cur);
}

/* dispatch routes each token row to every expert it selected; BF16 and FP8
 * payloads are both supported (GeekNews usage section: "supports BF16 and FP8
 * input"; FP8 dispatch / BF16 combine in the V3 benchmark setup).  In FP8 mode
 * a token is quantised once and its codes and scales are written to each of
 * its rows. */
void oracle_dispatch(const uint16_t* x, int T, int H, int K, const int32_t* slot,
                     int use_fp8, void* recv, float* scales)
{
    int nb = H / 128;
    uint8_t* q = NULL;
    float* s = NULL;
    if (use_fp8) {
        q = (uint8_t*)malloc((size_t)H);
        s = (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    }
    for (int t = 0; t < T; ++t) {
        const uint16_t* row = x + (size_t)t * H;
        if (use_fp8)
            for (int b = 0; b < nb; ++b)
                oracle_quant_block(row + (size_t)b * 128, q + (size_t)b * 128, s + b);
        for (int k = 0; k < K; ++k) {
            int32_t r = slot[(size_t)t * K + k];
            if (r < 0)
                continue;
            if (use_fp8) {
                memcpy((uint8_t*)recv + (size_t)r * H, q, (size_t)H);
                memcpy(scales + (size_t)r * nb, s, sizeof(float) * (size_t)nb);
            } else {
                memcpy((uint16_t*)recv + (size_t)r * H, row, sizeof(uint16_t) * (size_t)H);
            }
        }
    }
    free(q);
    free(s);
}

/* combine reduces the expert outputs back to each token (GeekNews usage
 * section; stakiran summary, section 3).  Reading: the weights are applied
 * here, accumulation is fp32 with one fused multiply-add per valid k in
 * ascending k, starting from +0.0f, and the sum is rounded once to BF16.  A
 * token with no valid pair gets a row of +0. */
void oracle_combine(const uint16_t* y, int T, int H, int K, const int32_t* slot,
                    const float* w, uint16_t* out)
{
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < H; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = slot[(size_t)t * K + k];
                if (r < 0)
                    continue;
                acc = fmaf(w[(size_t)t * K + k], oracle_bf16_to_f32(y[(size_t)r * H + j]), acc);
            }
            out[(size_t)t * H + j] = oracle_bf16_rne(acc);
        }
    }
}

/* Dispatch of rows that arrive already quantised (E4M3FN codes xq [T,H] with
 * fp32 block scales xs [T,H/128]): no arithmetic, each token's codes and
 * scales are copied to each of its receive rows. */
void oracle_dispatch_fp8_input(const uint8_t* xq, const float* xs, int T, int H, int K,
                               const int32_t* slot, uint8_t* recv, float* scales)
{
    int nb = H / 128;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int32_t r = slot[(size_t)t * K + k];
            if (r < 0)
                continue;
            memcpy(recv + (size_t)r * H, xq + (size_t)t * H, (size_t)H);
            memcpy(scales + (size_t)r * nb, xs + (size_t)t * nb, sizeof(float) * (size_t)nb);
        }
    }
}

/* Combine of FP8 rows (the dequantising option of the backward of dispatch,
 * and of combine): each received element is first widened to its value,
 * v = decode(q) * scale of its 128-channel block (one fp32 multiply), then
 * reduced as in oracle_combine.  w == NULL means unit weights, for which
 * fmaf(1, v, acc) is the plain sum acc + v. */
void oracle_combine_fp8(const uint8_t* q, const float* scales, int T, int H, int K,
                        const int32_t* slot, const float* w, uint16_t* out)
{
    const int nb = H / 128;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < H; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = slot[(size_t)t * K + k];
                if (r < 0)
                    continue;
                float v = oracle_e4m3fn_to_f32(q[(size_t)r * H + j]) * scales[(size_t)r * nb + j / 128];
                float wk = w ? w[(size_t)t * K + k] : 1.0f;
                acc = fmaf(wk, v, acc);
            }
            out[(size_t)t * H + j] = oracle_bf16_rne(acc);
        }
    }
}

/* Backward of dispatch (straight-through for the FP8 cast): each token's
 * gradient is the sum of the gradients of its received rows.  The sum is the
 * combine definition with unit weights: fp32, k ascending, from +0.0f, then
 * one rounding to BF16. */
void oracle_dispatch_backward(const uint16_t* grad_recv, int T, int H, int K,
                              const int32_t* slot, uint16_t* grad_x)
{
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < H; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = slot[(size_t)t * K + k];
                if (r < 0)
                    continue;
                acc = acc + oracle_bf16_to_f32(grad_recv[(size_t)r * H + j]);
            }
            grad_x[(size_t)t * H + j] = oracle_bf16_rne(acc);
        }
    }
}

/* Backward of combine.  out[t] = sum_k w[t,k] * y[slot[t,k]] is linear in y
 * and in w: d out / d y[slot[t,k]] = w[t,k] (so grad_y is grad_out scaled by
 * the weight and sent back along the pair), and d out / d w[t,k] =
 * y[slot[t,k]] (so grad_w is a dot product over the hidden dimension).  The
 * dot product is taken in double and rounded once to fp32. */
void oracle_combine_backward(const uint16_t* grad_out, const uint16_t* y, int T, int H, int K,
                             const int32_t* slot, const float* w, uint16_t* grad_y,
                             float* grad_w)
{
    for (int t = 0; t < T; ++t) {
        const uint16_t* g = grad_out + (size_t)t * H;
        for (int k = 0; k < K; ++k) {
            int32_t r = slot[(size_t)t * K + k];
            if (r < 0) {
                if (y)
                    grad_w[(size_t)t * K + k] = 0.0f;
                continue;
            }
            float wk = w[(size_t)t * K + k];
            for (int j = 0; j < H; ++j)
                grad_y[(size_t)r * H + j] = oracle_bf16_rne(wk * oracle_bf16_to_f32(g[j]));
            if (y) {
                double dot = 0.0;
                for (int j = 0; j < H; ++j)
                    dot += (double)oracle_bf16_to_f32(g[j]) *
                           (double)oracle_bf16_to_f32(y[(size_t)r * H + j]);
                grad_w[(size_t)t * K + k] = (float)dot;
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Expert parallelism over P ranks, one rank's share.  With partitions as real
 * ranks, a token goes to each rank that hosts one of its dispatched experts,
 * once (devtrends.ru, "Как это выглядит в коде": is_token_in_rank and
 * num_tokens_per_rank; stakiran summary section 3: dispatch, expert GEMM,
 * combine).  Readings: the sender packs its rows partition-major, ascending
 * token within each destination; each packed row carries the token's K
 * expert ids as local ids of the destination (e - p*E/P, or -1 for experts
 * elsewhere, masked or invalid) and its K weights (0 where the id is -1); the
 * origin sums the returned per-rank rows in rank order.
 * ------------------------------------------------------------------------ */

/* part_idx [T][Kp], Kp = min(K, P): the distinct partitions of the token's
 * dispatched experts (the validity rules of oracle_layout), ascending, then
 * -1. */
void oracle_rank_routing(const int64_t* topk_idx, int T, int K, int E, int P, int64_t* part_idx)
{
    const int epp = E / P;
    const int Kp = K < P ? K : P;
    uint8_t* hit = (uint8_t*)malloc((size_t)P);
    uint8_t* seen = (uint8_t*)calloc((size_t)E, 1);
    for (int t = 0; t < T; ++t) {
        for (int p = 0; p < P; ++p)
            hit[p] = 0;
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e < 0 || e >= E || seen[e])
                continue;
            seen[e] = 1;
            hit[e / epp] = 1;
        }
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e >= 0 && e < E)
                seen[e] = 0;
        }
        int j = 0;
        for (int p = 0; p < P; ++p)
            if (hit[p])
                part_idx[(size_t)t * Kp + j++] = p;
        for (; j < Kp; ++j)
            part_idx[(size_t)t * Kp + j] = -1;
    }
    free(seen);
    free(hit);
}

/* Metadata of the packed rows: row r = slot_pack[t][j] carries token t to
 * partition p = part_idx[t][j].  local_idx[r][k] = e - p*E/P when the token's
 * k-th id e is dispatched (oracle_layout's rules) and lies in p, else -1;
 * local_w[r][k] = topk_weights[t][k] there, else 0.  Rows no pair maps to are
 * not written. */
void oracle_pack_metadata(const int64_t* topk_idx, const float* topk_weights, const int64_t* part_idx,
                          const int32_t* slot_pack, int T, int K, int E, int P,
                          int64_t* local_idx, float* local_w)
{
    const int epp = E / P;
    const int Kp = K < P ? K : P;
    uint8_t* seen = (uint8_t*)calloc((size_t)E, 1);
    uint8_t* ok = (uint8_t*)malloc((size_t)K);
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            ok[k] = 0;
            if (e >= 0 && e < E && !seen[e]) {
                seen[e] = 1;
                ok[k] = 1;
            }
        }
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e >= 0 && e < E)
                seen[e] = 0;
        }
        for (int j = 0; j < Kp; ++j) {
            int64_t p = part_idx[(size_t)t * Kp + j];
            int32_t r = slot_pack[(size_t)t * Kp + j];
            if (p < 0 || r < 0)
                continue;
            for (int k = 0; k < K; ++k) {
                int64_t e = topk_idx[(size_t)t * K + k];
                int local = ok[k] && e / epp == p;
                local_idx[(size_t)r * K + k] = local ? e - p * epp : -1;
                local_w[(size_t)r * K + k] = local ? topk_weights[(size_t)t * K + k] : 0.0f;
            }
        }
    }
    free(ok);
    free(seen);
}
