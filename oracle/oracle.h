/*
 * CPU oracle for MoE dispatch / combine -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load or call this library.  The GPU library never does, and
 * shares no code with it.
 *
 * It is the plain, slow definition of what the hot path computes, written from
 * the DeepEP pages:
 *   - the call flow get_dispatch_layout -> dispatch(x, topk_idx, topk_weights)
 *     -> expert GEMM -> combine(y, handle), and "backward of dispatch is
 *     combine and vice versa" (stakiran github-trend-summarizer, DeepEP 要約,
 *     section 3 "使うときの流れ");
 *   - the handle carries the routing metadata combine needs, and
 *     handle.num_recv_tokens_per_expert_list gives per-expert counts for the
 *     GEMM (GeekNews, "Mẫu sử dụng cho huấn luyện, prefill và decoding");
 *   - FP8 dispatch with BF16 combine (aikraft.ru, "Технические детали и
 *     требования"; GeekNews, "Kết quả đo hiệu năng");
 *   - reuse of routing metadata through a cached handle (GeekNews, same usage
 *     section).
 * Where the pages leave a step open (receive layout, id validity rules, FP8
 * variant and scale convention, combine summation order) the readings are the
 * ones stated beside each function below.
 *
 * Every function is single-threaded plain loops.  Build with -O2
 * -ffp-contract=off so that every fp32 operation is the single IEEE operation
 * the source names (fmaf is an explicit fused multiply-add).
 */
#ifndef MOE_EP_ORACLE_H
#define MOE_EP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Codec helpers (exported so that tests can pin them one value at a time). */
uint16_t oracle_bf16_rne(float f);         /* fp32 -> bf16, round to nearest even   */
float    oracle_bf16_to_f32(uint16_t b);   /* exact widening                         */
uint8_t  oracle_e4m3fn_rne_sat(float v);   /* fp32 -> OCP E4M3FN, RNE, satfinite     */
float    oracle_e4m3fn_to_f32(uint8_t q);  /* exact decode (0x7F/0xFF -> NaN)        */
void     oracle_e4m3fn_encode_array(const float* v, uint8_t* q, int64_t n);

/* Quantise one block of 128 BF16 values: q[128] codes and the scale s. */
void oracle_quant_block(const uint16_t* x128, uint8_t* q128, float* scale);

/* Step 1, layout.  valid[T*K] receives 1 for a pair that takes part in
 * dispatch, 0 for masked (id < 0), out-of-range (id >= E) or repeated ids.
 * Returns 0, or -1 on invalid dimensions. */
int oracle_layout(const int64_t* topk_idx, int T, int K, int E, int P,
                  int32_t* num_tokens_per_expert, int32_t* num_tokens_per_partition,
                  uint8_t* is_token_in_partition, int32_t* num_invalid,
                  uint8_t* valid);

/* Exclusive prefix sum of per-expert counts: off[0] = 0, off[E] = N. */
void oracle_expert_offsets(const int32_t* num_tokens_per_expert, int E, int32_t* off);

/* GEMM-aligned offsets: off[e+1] = off[e] + (count rounded up to a multiple
 * of A); rows [off[e] + count[e], off[e+1]) are padding. */
void oracle_expert_offsets_aligned(const int32_t* num_tokens_per_expert, int E, int A, int32_t* off);

/* Step 2, slots.  slot[T*K] (-1 when not dispatched), src_token[capacity]
 * (entries at and beyond min(N, capacity) are left untouched), *overflow = 1
 * when a pair's slot would be >= capacity. */
void oracle_slots(const int64_t* topk_idx, const uint8_t* valid, int T, int K,
                  const int32_t* off, int E, int capacity,
                  int32_t* slot, int32_t* src_token, int32_t* overflow);

/* Static-capacity receive layout of the low-latency dispatch (devtrends.ru,
 * "Как это выглядит в коде": low_latency_dispatch(hidden_states, topk_idx,
 * num_max_tokens, num_experts)): expert e owns rows [e*cap, (e+1)*cap), and a
 * dispatched pair takes row e*cap + (number of earlier tokens that chose e).
 * A pair whose rank reaches cap is dropped (slot -1) and *overflow = 1. */
void oracle_slots_static(const int64_t* topk_idx, const uint8_t* valid, int T, int K, int E,
                         int cap, int32_t* slot, int32_t* overflow);

/* Step 3, permute (BF16: bit copy of the row) or quantise-then-permute (FP8).
 * recv has capacity rows of H elements (uint16 bf16 or uint8 e4m3fn);
 * scales has capacity rows of H/128 fp32 (FP8 mode only). */
void oracle_dispatch(const uint16_t* x, int T, int H, int K, const int32_t* slot,
                     int use_fp8, void* recv, float* scales);

/* Combine: out[t, j] = bf16_rne( fmaf chain over k ascending of
 * w[t,k] * y[slot[t,k], j], starting from +0.0f, skipping slot < 0 ). */
void oracle_combine(const uint16_t* y, int T, int H, int K, const int32_t* slot,
                    const float* w, uint16_t* out);

/* Dispatch of pre-quantised rows: recv[slot[t,k]] = xq[t] (H codes) and
 * scales[slot[t,k]] = xs[t] (H/128 fp32). */
void oracle_dispatch_fp8_input(const uint8_t* xq, const float* xs, int T, int H, int K,
                               const int32_t* slot, uint8_t* recv, float* scales);

/* Combine of FP8 rows q [rows, H] with fp32 block scales [rows, H/128]:
 *   v = e4m3fn_to_f32(q) * scale   (one fp32 multiply)
 *   out[t, j] = bf16_rne( fmaf chain over k ascending of w[t,k] * v, from +0.0f )
 * w == NULL: unit weights (the dequantising backward of dispatch). */
void oracle_combine_fp8(const uint8_t* q, const float* scales, int T, int H, int K,
                        const int32_t* slot, const float* w, uint16_t* out);

/* Backward of dispatch: the backward of dispatch is combine (stakiran summary,
 * section 3).  With the FP8 cast taken as straight-through, grad_x[t] =
 * bf16_rne( fp32 sum over dispatched k ascending of grad_recv[slot[t,k]],
 * from +0.0f ); a token with no dispatched pair gets +0. */
void oracle_dispatch_backward(const uint16_t* grad_recv, int T, int H, int K,
                              const int32_t* slot, uint16_t* grad_x);

/* Backward of combine: the backward of combine is dispatch (stakiran summary,
 * section 3), here of grad_out scaled by each pair's weight:
 *   grad_y[slot[t,k]][j] = bf16_rne( w[t,k] * grad_out[t][j] )  (one fp32 product)
 *   grad_w[t,k] = (float) sum_j grad_out[t][j] * y[slot[t,k]][j]  (sum in double)
 * Rows of grad_y that no pair maps to are left untouched; grad_w is 0 for
 * pairs that were not dispatched.  y == NULL skips grad_w. */
void oracle_combine_backward(const uint16_t* grad_out, const uint16_t* y, int T, int H, int K,
                             const int32_t* slot, const float* w, uint16_t* grad_y,
                             float* grad_w);

/* Expert parallelism over P ranks, one rank's share (partitions as ranks).
 * Destination ranks of each token: part_idx [T][min(K,P)], the distinct
 * partitions of its dispatched experts, ascending, then -1. */
void oracle_rank_routing(const int64_t* topk_idx, int T, int K, int E, int P, int64_t* part_idx);

/* Metadata of the packed rows: for row r = slot_pack[t][j] (destination
 * p = part_idx[t][j]), local_idx[r][k] = e - p*E/P for the token's dispatched
 * experts in p, else -1; local_w[r][k] = topk_weights[t][k] there, else 0. */
void oracle_pack_metadata(const int64_t* topk_idx, const float* topk_weights, const int64_t* part_idx,
                          const int32_t* slot_pack, int T, int K, int E, int P,
                          int64_t* local_idx, float* local_w);

#ifdef __cplusplus
}
#endif
#endif
