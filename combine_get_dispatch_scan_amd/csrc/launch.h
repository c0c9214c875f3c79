// Host-side launchers of the moe_ep kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_ep {

// EP_DEBUG=1 in the environment: every launch prints its kernel, grid, block
// and dynamic LDS to stderr (read once per process).
void debug_launch(const char* kernel, dim3 grid, dim3 block, size_t lds);

// get_dispatch_layout: per-chunk count kernel + one-workgroup scan kernel.
hipError_t launch_layout(const int64_t* topk_idx, int T, int K, int E, int P, int align,
                         uint8_t* is_token_in_partition, int32_t* pair_code,
                         int32_t* chunk_cnt, int32_t* chunk_base, int32_t* chunk_pcnt,
                         int32_t* chunk_inv, int32_t* expert_offset,
                         int32_t* num_tokens_per_expert, int32_t* num_tokens_per_partition,
                         int32_t* num_invalid, int32_t* status, hipStream_t stream);

struct DispatchLaunch {
    const void* x;
    const float* x_scales;    // non-null: x holds E4M3FN codes with these block scales
    int T, H, K, E;
    int use_fp8;
    bool fresh;               // compute slots from pair codes (else reuse slot[])
    int seq;                  // the handle's dispatch number, written on overflow
    int capacity;
    int align;                // GEMM row tile of the expert blocks (1: dense)
    int scale_ld;             // 0: row-major scales, else column-major leading dimension
    const int32_t* pair_code;
    const int32_t* chunk_base;
    const int32_t* chunk_cnt;
    const int32_t* expert_offset;
    const float* w_in;
    float* w_copy;
    int32_t* slot;
    int32_t* src_token;
    int32_t* status;
    void* recv;
    float* scales;
};

hipError_t launch_dispatch(const DispatchLaunch& L, hipStream_t stream);

// Low-latency dispatch: T <= 256 tokens, static per-expert capacity `cap`.
constexpr int kLowLatencyMaxTokens = 256;

struct LowLatencyLaunch {
    const void* x;
    const int64_t* topk_idx;
    const float* w_in;
    int T, H, K, E, P, cap;
    int use_fp8;
    void* recv;
    float* scales;
    int32_t* slot;
    float* w_copy;
    int32_t* status;
    int32_t* expert_offset;
    int32_t* num_tokens_per_expert;
    int32_t* num_tokens_per_partition;
    uint8_t* is_token_in_partition;
    int32_t* num_invalid;
};

hipError_t launch_low_latency_dispatch(const LowLatencyLaunch& L, hipStream_t stream);

// combine; w == nullptr means unit weights (the backward of dispatch).
hipError_t launch_combine(const void* y, int T, int H, int K, const int32_t* slot,
                          const float* w, void* out, hipStream_t stream);

// combine of FP8 rows with fp32 block scales (w == nullptr: unit weights);
// scale_ld 0: row-major scales, else column-major with that leading dimension.
hipError_t launch_combine_fp8(const void* y, const float* scales, int scale_ld, int T, int H, int K,
                              const int32_t* slot, const float* w, void* out, hipStream_t stream);

// backward of combine: grad_y rows (and grad_w when y != nullptr).
hipError_t launch_combine_backward(const void* grad_out, const void* y, int T, int H, int K,
                                   const int32_t* slot, const float* w, void* grad_y,
                                   float* grad_w, hipStream_t stream);

hipError_t launch_e4m3fn_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

// expert parallelism over ranks: destination routing and packed-row metadata
hipError_t launch_rank_routing(const int64_t* topk_idx, int T, int K, int E, int P, int64_t* part_idx,
                               hipStream_t stream);
hipError_t launch_pack_metadata(const int64_t* topk_idx, const float* topk_weights,
                                const int64_t* part_idx, const int32_t* slot_pack, int T, int K,
                                int E, int P, int64_t* local_idx, float* local_w, hipStream_t stream);

}  // namespace moe_ep
