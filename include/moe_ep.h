/*
 * moe_ep -- MoE expert-parallel dispatch and combine for one rank's share of
 * the work, on one AMD Instinct MI355X (gfx950).
 *
 * The calls follow the interface the DeepEP pages describe: the forward flow
 * get_dispatch_layout -> dispatch(x, topk_idx, topk_weights) -> expert GEMM ->
 * combine(y, handle), with backward being the other call (stakiran
 * github-trend-summarizer, "DeepEP 要約", section 3 "使うときの流れ"); the
 * handle carries the routing metadata combine needs, per-expert received
 * counts feed the grouped GEMM, and a cached handle lets a caller skip the
 * layout step when routing has not changed (GeekNews, "Mẫu sử dụng cho huấn
 * luyện, prefill và decoding").  Destination partitions stand for the EP ranks
 * of the pages; here they are logical groups of experts within one GPU's HBM.
 *
 * Conventions
 *  - Every call returns EP_OK (0) or a negative EP_E* code; ep_last_error()
 *    then holds a message (thread-local).  Arguments are validated before any
 *    HIP call, so an invalid argument never touches the device.
 *  - Every device buffer and stream belongs to the caller.  The library never
 *    allocates device memory and never creates streams or events.
 *  - Every call enqueues its kernels on `stream` and returns without waiting,
 *    except ep_handle_recv_counts, which synchronises `stream`.
 *  - Layouts are row-major.  topk_idx is int64 [T, K]; a negative id means
 *    "masked", an id >= E or an id repeated earlier in the same row is
 *    "invalid": both are skipped everywhere, invalid ones are counted.
 *  - Partition p owns experts [p*E/P, (p+1)*E/P).
 *  - The receive buffer is expert-contiguous: one row per dispatched (t, k)
 *    pair, experts in ascending id, and within one expert ascending source
 *    token, with no padding.  Row order is therefore deterministic.
 *  - FP8 is OCP E4M3FN (max 448).  Each token is quantised once, per block of
 *    128 channels: a = max(amax, 2^-64), codes = RNE_satfinite(x * (448 / a)),
 *    scale = a / 448 (fp32, dequantise as code * scale).
 *  - combine accumulates in fp32 with one fused multiply-add per dispatched k
 *    in ascending k from +0.0f, then rounds to BF16 (nearest even).
 *  - x, y, the gradients and the weights are finite.  NaN and infinities are
 *    outside the contract: the codes, scales and sums they touch are then
 *    unspecified (no call traps or faults on them).
 *  - Limits: 1 <= K <= 16, 1 <= E <= 1024, 1 <= P <= 64, E % P == 0,
 *    0 <= T, T*K < 2^31, 1 <= H <= 32768, H % 8 == 0 (H % 128 == 0 for FP8).
 *    x, recv_x, y and out must be 16-byte aligned, topk_idx 8-byte, the other
 *    device arrays 4-byte; the workspace 256-byte aligned.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_OK          0
#define EP_EINVAL     (-1)   /* invalid argument (nothing was enqueued)         */
#define EP_EHIP       (-2)   /* a HIP runtime call failed                        */
#define EP_ECAPACITY  (-3)   /* dispatch dropped pairs: capacity_rows < N         */
#define EP_EIDS       (-4)   /* topk_idx held out-of-range or repeated ids        */

#define EP_MAX_TOPK        16
#define EP_MAX_EXPERTS     1024
#define EP_MAX_PARTITIONS  64
#define EP_MAX_HIDDEN      32768

#define EP_MAX_LL_TOKENS   256     /* tokens per ep_low_latency_dispatch call     */
#define EP_NOALLOC_SCRATCH_BYTES 81920   /* per-GPU array of the allocation-free
                                            low-latency dispatch: the handle
                                            arrays of T=256, K=16, E=1024, P=64
                                            take 78592 bytes                  */
#define EP_MAX_ALIGNMENT   1024    /* expert_alignment of an aligned layout        */

#define EP_HANDLE_MAGIC    0x31485045u   /* "EPH1" */

/*
 * Routing metadata of one dispatch, filled by ep_get_dispatch_layout and
 * completed by ep_dispatch.  A host-side plain struct owned by the caller; the
 * device arrays it points to live inside the caller's workspace and stay valid
 * while that workspace is neither freed nor reused by another layout call.
 * Treat the fields as read-only.
 * Calls that take a handle refuse, with EP_EINVAL, one the layout call did
 * not fill (magic), one below the stage the call needs, and one whose
 * dimensions are outside the limits above.
 */
typedef struct ep_handle {
    uint32_t magic;            /* EP_HANDLE_MAGIC once the layout call filled it  */
    int32_t  stage;            /* 1: layout done, 2: dispatched                    */
    int32_t  num_tokens;       /* T */
    int32_t  num_topk;         /* K */
    int32_t  num_experts;      /* E */
    int32_t  num_partitions;   /* P */
    int32_t  hidden;           /* H (set by ep_dispatch)                           */
    int32_t  use_fp8;          /* 0: BF16 rows, 1: E4M3FN rows + fp32 scales       */
    int32_t  capacity_rows;    /* rows available in recv_x (set by ep_dispatch)    */
    int32_t  has_weights;      /* 1 when ep_dispatch copied topk_weights            */
    int32_t  num_chunks;       /* ceil(T / 256)                                    */
    int32_t  static_cap;       /* rows per expert of ep_low_latency_dispatch's
                                  static layout; 0 for the dense layout          */
    void*    ws;               /* the workspace                                    */
    size_t   ws_bytes;
    int32_t* expert_offset;    /* [E+1] first receive row of each expert; [E] = N  */
    int32_t* slot;             /* [T*K] receive row of pair (t,k), -1 if none      */
    int32_t* src_token;        /* [T*K] source token of receive row r, r < min(N, capacity);
                                  NULL for the static layout                     */
    float*   weights;          /* [T*K] copy of topk_weights                       */
    int32_t* status;           /* [4] overflow flag, num_invalid, N, 0             */
    int32_t* pair_code;        /* [T*K] (expert << 8 | rank in chunk), -1 if none  */
    int32_t* chunk_base;       /* [chunks*E] rows of expert e in earlier chunks    */
    int32_t* chunk_pcnt;       /* [chunks*P] */
    int32_t* chunk_inv;        /* [chunks]   */
    int32_t* chunk_cnt;        /* [chunks*E] rows of expert e in each chunk        */
    int32_t  expert_alignment; /* row tile of the expert blocks (1 or 0: dense)    */
    int32_t  scale_ld;         /* 0: row-major scales; else column-major, this
                                  leading dimension (set by ep_dispatch_ex)      */
    int32_t  fp8_input;        /* 1 when ep_dispatch_ex got pre-quantised input    */
    int32_t  dispatch_seq;     /* number of the handle's latest ep_dispatch /
                                  ep_dispatch_ex (1, 2, ...): that dispatch
                                  marks dropped pairs by writing it into the
                                  overflow word, so an earlier dispatch's mark
                                  is not mistaken for its own               */
} ep_handle_t;

/* Library version, major*10000 + minor*100 + patch.  EP_VERSION is the
 * version of this header; ep_version() that of the loaded library. */
#define EP_VERSION 10201
int ep_version(void);

/* Message describing the last error returned on this thread ("" if none). */
const char* ep_last_error(void);

/*
 * Bytes of device workspace that ep_get_dispatch_layout / ep_dispatch need for
 * T tokens, top-K, E experts and P partitions (0 on invalid dimensions).  The
 * workspace holds the handle's arrays and per-chunk tables.
 */
size_t ep_workspace_bytes(int num_tokens, int num_topk, int num_experts, int num_partitions);

/*
 * get_dispatch_layout: per-expert and per-partition token counts and the
 * token-in-partition mask (stakiran summary section 3: get_dispatch_layout
 * comes before dispatch; devtrends.ru "Как это выглядит в коде": dispatch
 * takes num_tokens_per_rank).  Also prepares the handle for ep_dispatch.
 *
 *   topk_idx                  device int64 [T*K]
 *   num_tokens_per_partition  device int32 [P]  distinct tokens with >= 1
 *                             dispatched pair in the partition
 *   num_tokens_per_expert     device int32 [E]  dispatched pairs per expert
 *   is_token_in_partition     device uint8 [T*P] 1 if the token has a
 *                             dispatched pair in the partition, else 0
 *   num_invalid               device int32 [1]  out-of-range + repeated ids
 *   ws, ws_bytes              device workspace of ep_workspace_bytes(T,K,E,P)
 *   handle                    host; overwritten
 * Errors: EP_EINVAL (bad dims, pointers, alignment, small workspace), EP_EHIP.
 */
int ep_get_dispatch_layout(const int64_t* topk_idx, int num_tokens, int num_topk,
                           int num_experts, int num_partitions,
                           int32_t* num_tokens_per_partition, int32_t* num_tokens_per_expert,
                           uint8_t* is_token_in_partition, int32_t* num_invalid,
                           void* ws, size_t ws_bytes, ep_handle_t* handle,
                           hipStream_t stream);

/*
 * dispatch: every dispatched (t, k) pair gets one receive row (the slot scan),
 * and token t's row is written to each of its rows -- as BF16, or quantised
 * once to FP8 E4M3FN with per-128-channel fp32 scales (GeekNews usage section:
 * BF16 and FP8 input; aikraft.ru "Технические детали и требования": FP8
 * dispatch, BF16 combine).  Must follow ep_get_dispatch_layout with the same
 * handle on the same stream (or after it completed).
 *
 *   x              device bf16 [T*H]
 *   topk_weights   device fp32 [T*K] or NULL; copied into the workspace for
 *                  ep_combine, so the caller may free it afterwards
 *   hidden         H
 *   use_fp8        0: recv_x is bf16 [capacity_rows*H]; 1: recv_x is
 *                  e4m3fn bytes [capacity_rows*H], recv_scales fp32
 *                  [capacity_rows*H/128]
 *   capacity_rows  rows in recv_x, at most T*K (T*K + E*(A-1) for a layout
 *                  aligned to A rows); that maximum never overflows, or pass
 *                  the exact N read back by ep_handle_recv_counts.  Pairs
 *                  whose row would be >= capacity_rows are dropped (slot -1)
 *                  and flagged.
 *   handle         in: from the layout call, or already dispatched (a
 *                  dispatch again on the same routing, e.g. with a larger
 *                  capacity after EP_ECAPACITY); out: stage 2.  Each dispatch
 *                  recomputes every slot; the overflow status that
 *                  ep_handle_recv_counts reports is the latest dispatch's.
 * Receive rows at and beyond N (the end of the last expert block) are not
 * written.
 * Errors: EP_EINVAL, EP_EHIP.  Overflow is reported by ep_handle_recv_counts.
 *
 * The call takes the handle the layout call filled, not topk_idx and the
 * dimensions again: the handle already holds the routing (as per-pair codes
 * the layout computed), the dimensions and the workspace.
 */
int ep_dispatch(const void* x, const float* topk_weights, int hidden, int use_fp8,
                void* recv_x, float* recv_scales, int capacity_rows,
                ep_handle_t* handle, hipStream_t stream);

/*
 * Low-latency dispatch for decode batches: layout, slot assignment and the
 * (quantise-and-)permute in ONE kernel launch, with no host synchronisation
 * and no memset, so it can be captured in a HIP graph (devtrends.ru "Как это
 * выглядит в коде": low_latency_dispatch(hidden_states, topk_idx,
 * num_max_tokens, num_experts); stakiran summary section 3: the decode path,
 * CUDA-graph compatible).  The receive buffer has a static per-expert
 * capacity: expert e owns rows [e*cap, (e+1)*cap), and a dispatched pair takes
 * row e*cap + (its rank among expert e's pairs in token order).  A pair whose
 * rank reaches cap is dropped (slot -1) and flagged.  Rows past an expert's
 * count are not written.
 *
 *   x, topk_idx, topk_weights   as for ep_get_dispatch_layout / ep_dispatch;
 *                               0 <= num_tokens <= EP_MAX_LL_TOKENS
 *   num_max_tokens              cap, rows per expert (E*cap < 2^31)
 *   recv_x                      bf16 or e4m3fn [E*cap*H]; recv_scales fp32
 *                               [E*cap*H/128] in FP8 mode
 *   num_tokens_per_expert ...   the layout outputs, as ep_get_dispatch_layout
 *                               (num_tokens_per_expert counts every dispatched
 *                               pair, including dropped ones)
 *   ws, ws_bytes                ep_workspace_bytes(T, K, E, P)
 *   handle                      out: a dispatched handle.  ep_combine,
 *                               ep_dispatch_cached and the backward calls use
 *                               it as any other; ep_handle_recv_counts reports
 *                               min(count, cap) rows per expert and returns
 *                               EP_ECAPACITY when a pair was dropped.
 * Errors: EP_EINVAL, EP_EHIP.
 */
int ep_low_latency_dispatch(const void* x, const int64_t* topk_idx, const float* topk_weights,
                            int num_tokens, int hidden, int num_topk, int num_experts,
                            int num_partitions, int use_fp8, int num_max_tokens,
                            void* recv_x, float* recv_scales,
                            int32_t* num_tokens_per_partition, int32_t* num_tokens_per_expert,
                            uint8_t* is_token_in_partition, int32_t* num_invalid,
                            void* ws, size_t ws_bytes, ep_handle_t* handle, hipStream_t stream);

/*
 * Allocation-free low-latency dispatch, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The same launch and results as
 * ep_low_latency_dispatch, but the handle's arrays (slots, weight copy,
 * expert offsets, status) live in a library-owned device array of
 * EP_NOALLOC_SCRATCH_BYTES on each GPU instead of a caller workspace.  The
 * call allocates nothing; the array is set up on the first call on each
 * device (a symbol lookup) and stays until the process ends.
 *
 * Arguments as for ep_low_latency_dispatch, without ws / ws_bytes; the
 * current device must be the device of `stream` (else EP_EINVAL).  Every call on one GPU uses
 * that GPU's one array, which keeps the latest call's contents: the handle
 * stays valid (for ep_combine, ep_dispatch_cached, the backward calls,
 * ep_handle_recv_counts) until the next call of this entry point on the same
 * GPU, and calls that overlap on one GPU (several streams or host threads)
 * race.  A captured graph replays into the same array.
 * Errors: EP_EINVAL (as ep_low_latency_dispatch; dimensions whose arrays do
 * not fit the scratch, which the stated limits never produce), EP_EHIP.
 */
int ep_low_latency_dispatch_noalloc(const void* x, const int64_t* topk_idx,
                                    const float* topk_weights, int num_tokens, int hidden,
                                    int num_topk, int num_experts, int num_partitions,
                                    int use_fp8, int num_max_tokens, void* recv_x,
                                    float* recv_scales, int32_t* num_tokens_per_partition,
                                    int32_t* num_tokens_per_expert,
                                    uint8_t* is_token_in_partition, int32_t* num_invalid,
                                    ep_handle_t* handle, hipStream_t stream);

/*
 * GEMM-facing layout options (GeekNews, "Những thay đổi chính của bản phát
 * hành V2": a new GEMM layout; usage section: per-expert counts feed the
 * grouped GEMM; aikraft.ru "Технические детали и требования": FP8 input).
 *
 * ep_get_dispatch_layout_aligned: as ep_get_dispatch_layout, with each
 * expert's block of receive rows rounded up to a multiple of
 * expert_alignment (1 <= A <= EP_MAX_ALIGNMENT), so every block starts on a
 * multiple of A.  Rows [off[e] + count[e], off[e+1]) of a block are padding,
 * written as zero codes / zero BF16 values and zero scales by every dispatch
 * through the handle.  The counts ep_handle_recv_counts reports are the block
 * sizes (padding included); num_tokens_per_expert keeps the real counts.  The
 * handle keeps no source-token table (src_token NULL) when A > 1.  A dispatch
 * without drops needs capacity_rows >= T*K + E*(A-1) in the worst case.
 *
 * ep_dispatch_ex: ep_dispatch with two more options.
 *   x_scales  NULL: x is BF16 as for ep_dispatch.  Non-NULL (needs use_fp8):
 *             x holds E4M3FN codes [T*H] and x_scales fp32 [T*H/128] their
 *             block scales; codes and scales are copied, not re-quantised.
 *   scale_ld  0: recv_scales row-major [capacity_rows][H/128].  Otherwise
 *             (FP8 only; >= capacity_rows, a multiple of 4) column-major:
 *             the scale of receive row r, block b is recv_scales[b*scale_ld + r].
 * ep_dispatch_cached_ex: the cached dispatch of such a handle; x_scales must
 * be given exactly when the handle was dispatched from FP8 input.
 * Errors: EP_EINVAL, EP_EHIP.
 */
int ep_get_dispatch_layout_aligned(const int64_t* topk_idx, int num_tokens, int num_topk,
                                   int num_experts, int num_partitions, int expert_alignment,
                                   int32_t* num_tokens_per_partition,
                                   int32_t* num_tokens_per_expert,
                                   uint8_t* is_token_in_partition, int32_t* num_invalid,
                                   void* ws, size_t ws_bytes, ep_handle_t* handle,
                                   hipStream_t stream);
int ep_dispatch_ex(const void* x, const float* x_scales, const float* topk_weights, int hidden,
                   int use_fp8, int scale_ld, void* recv_x, float* recv_scales, int capacity_rows,
                   ep_handle_t* handle, hipStream_t stream);
int ep_dispatch_cached_ex(const void* x, const float* x_scales, const ep_handle_t* handle,
                          void* recv_x, float* recv_scales, hipStream_t stream);

/*
 * Cached dispatch: re-sends new token rows along the routing of an earlier
 * dispatch, skipping the layout and the slot scan (GeekNews usage section:
 * routing metadata reused through cached_handle when gating is unchanged).
 * Output is bit-identical to a fresh ep_dispatch of the same x.
 *   x, recv_x, recv_scales as in ep_dispatch (same H, use_fp8, capacity).
 * Errors: EP_EINVAL (handle not dispatched), EP_EHIP.
 */
int ep_dispatch_cached(const void* x, const ep_handle_t* handle,
                       void* recv_x, float* recv_scales, hipStream_t stream);

/*
 * combine: out[t] = bf16_rne( sum over dispatched k, ascending, of
 * w[t,k] * y[slot[t,k]] ) with fp32 fused multiply-adds from +0.0f; a token
 * with no dispatched pair gets a +0 row (GeekNews usage section: combine
 * reduces expert outputs back to their origin; stakiran section 3).
 *
 *   y             device bf16 [rows*H], rows in the receive order of dispatch;
 *                 non-NULL whenever capacity_rows > 0, even if no pair was
 *                 dispatched (the host does not know N without a sync)
 *   handle        a dispatched handle
 *   topk_weights  device fp32 [T*K], or NULL to use the copy dispatch took
 *   out           device bf16 [T*H]
 * Errors: EP_EINVAL (no weights available, bad pointers), EP_EHIP.
 */
int ep_combine(const void* y, const ep_handle_t* handle, const float* topk_weights,
               void* out, hipStream_t stream);

/*
 * Backward of dispatch: the backward of dispatch is combine (stakiran summary,
 * section 3 "使うときの流れ"; GeekNews usage section).  With the FP8 cast taken
 * as straight-through, grad_x[t] = bf16_rne( fp32 sum over dispatched k,
 * ascending, of grad_recv[slot[t,k]], from +0.0f ); a token with no
 * dispatched pair gets +0.  Uses the handle of the forward dispatch.
 *   grad_recv  device bf16 [capacity_rows*H], in the receive order
 *   grad_x     device bf16 [T*H]
 * Errors: EP_EINVAL (handle not dispatched, bad pointers), EP_EHIP.
 */
int ep_dispatch_backward(const void* grad_recv, const ep_handle_t* handle, void* grad_x,
                         hipStream_t stream);

/*
 * Combine and backward of dispatch on FP8 rows: the dequantising option of
 * the backward of dispatch (stakiran summary, section 3: the backward of
 * dispatch is combine), for rows that arrive as E4M3FN codes with the same
 * per-128-channel fp32 scales dispatch produces (aikraft.ru "Технические
 * детали и требования": FP8 traffic).  Each gathered element is widened to
 * decode(q) * scale (one fp32 multiply) and then reduced as in ep_combine
 * (weighted) or ep_dispatch_backward (unit weights).
 *   y / grad_recv          device e4m3fn [capacity_rows*H], receive order
 *   y_scales / grad_scales device fp32, laid out as the handle's dispatch
 *                          wrote recv_scales: row-major [capacity_rows][H/128],
 *                          or column-major [H/128][scale_ld] when
 *                          ep_dispatch_ex was given scale_ld
 *   topk_weights           as for ep_combine
 *   out / grad_x           device bf16 [T*H]
 * Needs hidden % 128 == 0.  Errors: EP_EINVAL, EP_EHIP.
 */
int ep_combine_fp8(const void* y, const float* y_scales, const ep_handle_t* handle,
                   const float* topk_weights, void* out, hipStream_t stream);
int ep_dispatch_backward_fp8(const void* grad_recv, const float* grad_scales,
                             const ep_handle_t* handle, void* grad_x, hipStream_t stream);

/*
 * Backward of combine: the backward of combine is dispatch (same passages),
 * of grad_out scaled by each pair's weight, plus the weight gradient:
 *   grad_y[slot[t,k]] = bf16_rne(w[t,k] * grad_out[t])   (one fp32 product)
 *   grad_w[t,k]       = <grad_out[t], y[slot[t,k]]>       (fp32; 0 for pairs
 *                       not dispatched)
 *   grad_out      device bf16 [T*H]
 *   y             device bf16 [capacity_rows*H], the forward's expert outputs;
 *                 NULL when grad_w is NULL
 *   topk_weights  device fp32 [T*K], or NULL to use the copy dispatch took
 *   grad_y        device bf16 [capacity_rows*H]; rows no pair maps to are
 *                 not written
 *   grad_w        device fp32 [T*K] or NULL.  Each dot product is reduced in
 *                 a fixed order (per-lane fma chains over the hidden
 *                 dimension, a 64-lane tree, then 8 wave partials added in
 *                 wave order), so results are deterministic; against the
 *                 exact sum the error is at most gamma_d * sum_j |grad_out*y|,
 *                 gamma_d = d*2^-24/(1 - d*2^-24), d = 8*ceil(ceil(H/512)/8)
 *                 + 13 (29 for H = 7168).
 * Errors: EP_EINVAL, EP_EHIP.
 */
int ep_combine_backward(const void* grad_out, const void* y, const ep_handle_t* handle,
                        const float* topk_weights, void* grad_y, float* grad_w,
                        hipStream_t stream);

/*
 * Expert parallelism over P ranks, one rank's share.  With partitions as real
 * ranks a token goes once to each rank that hosts one of its dispatched
 * experts (devtrends.ru, "Как это выглядит в коде": is_token_in_rank and
 * num_tokens_per_rank; stakiran summary section 3: dispatch, expert GEMM,
 * combine).  The exchange between ranks is not part of this library; the
 * calls below and the single-rank calls give every step on either side of it:
 *
 *  sender   ep_rank_routing(topk_idx -> part_idx), then
 *           ep_get_dispatch_layout(part_idx, T, Kp, P, P, ...) + ep_dispatch:
 *           the packed rows, destination-major, ascending token within a
 *           destination, each token quantised once; that layout's
 *           num_tokens_per_expert[p] is the row count for destination p;
 *           ep_pack_metadata: each packed row's local expert ids and weights
 *  receiver ep_get_dispatch_layout(local_idx of the received rows, R, K, E/P,
 *           1, ...) + ep_dispatch_ex with the received codes and scales as
 *           FP8 input: the expert-contiguous layout of the local experts, in
 *           receive order (source rank, then token)
 *  expert   ep_combine(y, that handle, received local_w, partial): one BF16
 *           row per received row, its local experts pre-reduced
 *  origin   ep_dispatch_backward(returned partial rows in the packed order,
 *           the pack's handle, out): each token's rows summed in rank order
 *           (fp32 from +0, then BF16)
 * Kp = min(K, P).
 *
 * ep_rank_routing: part_idx int64 [T*Kp], the distinct partitions of each
 * token's in-range expert ids, ascending, then -1.  Errors: EP_EINVAL, EP_EHIP.
 */
int ep_rank_routing(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts,
                    int num_partitions, int64_t* part_idx, hipStream_t stream);

/*
 * ep_pack_metadata: for the packed rows of pack_handle (a dense layout of
 * part_idx over P "experts", dispatched), packed row r = slot[t][j] carries
 * token t to p = part_idx[t][j]; local_idx[r*K + k] = e - p*E/P when the
 * token's k-th id e is dispatched (in range, first occurrence in its row)
 * and lies in p, else -1; local_w[r*K + k] = topk_weights[t*K + k] there,
 * else 0.  local_idx int64 and local_w fp32 hold capacity_rows*K entries;
 * rows no pair maps to are not written.  Errors: EP_EINVAL, EP_EHIP.
 */
int ep_pack_metadata(const int64_t* topk_idx, const float* topk_weights, int num_topk,
                     int num_experts, const int64_t* part_idx, const ep_handle_t* pack_handle,
                     int64_t* local_idx, float* local_w, hipStream_t stream);

/*
 * Per-expert received counts to the host, for the grouped GEMM (GeekNews
 * usage section: handle.num_recv_tokens_per_expert_list).  Synchronises
 * `stream`.  host_counts: int32 [E] or NULL; host_num_recv: int32 [1] or NULL
 * receives N.  Returns EP_ECAPACITY if dispatch dropped pairs, else EP_EIDS if
 * topk_idx held invalid ids (the counts are valid in both cases), else EP_OK.
 */
int ep_handle_recv_counts(const ep_handle_t* handle, int32_t* host_counts,
                          int32_t* host_num_recv, hipStream_t stream);

/*
 * Asynchronous form of ep_handle_recv_counts, so the host can wait for the
 * counts while later work (combine, the next layout) is already queued.
 * Enqueues one device-to-host copy of the handle's expert offsets and status
 * words into host_buf and returns without waiting.
 *   host_buf  int32 [E + 5], caller-owned host memory; page-locked memory
 *             (hipHostMalloc, torch pin_memory) keeps the copy asynchronous
 * Once the stream has passed this point (the caller waits on an event
 * recorded after it, or on the stream), ep_recv_counts_decode gives the same
 * results and return code as ep_handle_recv_counts.
 * The counts are final once the layout has run.  For a dense layout
 * (ep_get_dispatch_layout, or alignment 1) the copy may therefore be taken
 * right after the layout call, e.g. on a second stream that waits for it, so
 * that it overlaps dispatch: ep_recv_counts_decode then detects dropped pairs
 * from N > capacity_rows of the dispatched handle.  (On MI355X with ROCm 7
 * the cross-stream wait costs more than the small copy it hides, so the
 * same-stream copy after dispatch is the faster default.)  For aligned and
 * low-latency layouts the drop flag is written by dispatch: copy after it.
 * Errors: EP_EINVAL, EP_EHIP.
 */
int ep_handle_recv_counts_async(const ep_handle_t* handle, int32_t* host_buf, hipStream_t stream);

/*
 * Decodes a buffer filled by ep_handle_recv_counts_async (host only, no HIP
 * call).  host_counts: int32 [E] or NULL; host_num_recv: int32 [1] or NULL.
 * Returns EP_OK, EP_ECAPACITY or EP_EIDS as ep_handle_recv_counts does.
 */
int ep_recv_counts_decode(const ep_handle_t* handle, const int32_t* host_buf,
                          int32_t* host_counts, int32_t* host_num_recv);

/*
 * The device E4M3FN encoder that dispatch uses, applied elementwise:
 * out[i] = RNE_satfinite_e4m3fn(in[i]) (sign of zero kept).  For testing the
 * codec on its own.  in: device fp32 [n]; out: device uint8 [n].
 */
int ep_e4m3fn_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_EP_H */
