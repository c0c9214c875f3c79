// dispatch on gfx950: slot assignment fused with the (quantise-and-)permute.
//
// dispatch routes every token row to each expert it selected; the payload is
// BF16 or FP8 (GeekNews usage section: BF16 and FP8 input; aikraft.ru
// "Технические детали и требования": FP8 dispatch, BF16 combine).  Rows land
// in an expert-contiguous receive buffer, one per dispatched (token, k) pair.
//
// Work item = (token, segment of the row), one wave each.  Lanes 0..K-1 turn
// the pair codes left by the layout step into receive rows
//     slot = expert_offset[e] + chunk_base[chunk][e] + rank_in_chunk
// and broadcast them to the wave (readlane -> SGPRs); the row itself is then
// handled by fp8_rows / bf16_rows (dispatch_rows.h).
#include "device.h"
#include "dispatch_rows.h"
#include "launch.h"

namespace moe_ep {

struct DispatchArgs {
    const uint16_t* x;
    int T, H, K, E;
    int nseg, iters_per_seg, iters;
    int capacity;
    const int32_t* pair_code;
    const int32_t* chunk_base;
    const int32_t* expert_offset;
    const float* w_in;
    float* w_copy;
    int32_t* slot;
    int32_t* src_token;
    int32_t* status;
    void* recv;
    float* scales;
};

template <int KMAX, bool FRESH>
__device__ __forceinline__ int pair_slot(const DispatchArgs& a, int t, int seg)
{
    const int lane = lane_id();
    int s = -1;
    if (lane < a.K) {
        const size_t i = (size_t)t * a.K + lane;
        if (FRESH) {
            int code = a.pair_code[i];
            bool ovf = false;
            if (code >= 0) {
                int e = code >> 8;
                s = a.expert_offset[e] + a.chunk_base[(size_t)(t / kChunk) * a.E + e] + (code & 0xFF);
                if (s >= a.capacity) {
                    s = -1;
                    ovf = true;
                }
            }
            if (seg == 0) {
                a.slot[i] = s;
                if (s >= 0)
                    a.src_token[s] = t;
                if (a.w_in)
                    a.w_copy[i] = a.w_in[i];
                if (ovf)
                    a.status[0] = 1;
            }
        } else {
            s = a.slot[i];
        }
    }
    return s;
}

template <int KMAX, bool FRESH>
__global__ __launch_bounds__(kDispatchWaves * kWave) void dispatch_fp8_kernel(DispatchArgs a)
{
    const int wi = blockIdx.x * kDispatchWaves + threadIdx.x / kWave;
    const int t = wi / a.nseg;
    const int seg = wi % a.nseg;
    if (t >= a.T)
        return;
    const int s_own = pair_slot<KMAX, FRESH>(a, t, seg);
    int sk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        sk[k] = k < a.K ? readlane(s_own, k) : -1;
    const int i_begin = seg * a.iters_per_seg;
    const int i_end = min(a.iters, i_begin + a.iters_per_seg);
    fp8_rows<KMAX>(a.x + (size_t)t * a.H, sk, a.H, i_begin, i_end,
                   static_cast<uint8_t*>(a.recv), a.scales);
}

template <int KMAX, bool FRESH>
__global__ __launch_bounds__(kDispatchWaves * kWave) void dispatch_bf16_kernel(DispatchArgs a)
{
    const int wi = blockIdx.x * kDispatchWaves + threadIdx.x / kWave;
    const int t = wi / a.nseg;
    const int seg = wi % a.nseg;
    if (t >= a.T)
        return;
    const int s_own = pair_slot<KMAX, FRESH>(a, t, seg);
    int sk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        sk[k] = k < a.K ? readlane(s_own, k) : -1;
    const int i_begin = seg * a.iters_per_seg;
    const int i_end = min(a.iters, i_begin + a.iters_per_seg);
    bf16_rows<KMAX>(a.x + (size_t)t * a.H, sk, a.H, i_begin, i_end,
                    static_cast<uint16_t*>(a.recv));
}

hipError_t launch_dispatch(const DispatchLaunch& L, hipStream_t stream)
{
    if (L.T == 0)
        return hipSuccess;
    DispatchArgs a;
    a.x = static_cast<const uint16_t*>(L.x);
    a.T = L.T;
    a.H = L.H;
    a.K = L.K;
    a.E = L.E;
    a.capacity = L.capacity;
    a.pair_code = L.pair_code;
    a.chunk_base = L.chunk_base;
    a.expert_offset = L.expert_offset;
    a.w_in = L.w_in;
    a.w_copy = L.w_copy;
    a.slot = L.slot;
    a.src_token = L.src_token;
    a.status = L.status;
    a.recv = L.recv;
    a.scales = L.scales;
    const int ch = L.use_fp8 ? kFp8ChPerIter : kBf16ChPerIter;
    a.iters = (L.H + ch - 1) / ch;
    if (a.iters < 1)
        a.iters = 1;
    const RowSplit rs = split_rows(L.T, a.iters, EP_DISPATCH_MIN_ITEMS, EP_DISPATCH_MAX_ITERS);
    a.nseg = rs.nseg;
    a.iters_per_seg = rs.iters_per_seg;
    const long long items = (long long)L.T * a.nseg;
    dim3 grid((unsigned)((items + kDispatchWaves - 1) / kDispatchWaves));
    dim3 block(kDispatchWaves * kWave);

#define EP_DISPATCH(KERNEL, KM, FRESH) \
    hipLaunchKernelGGL((KERNEL<KM, FRESH>), grid, block, 0, stream, a)
#define EP_DISPATCH_K(KERNEL, FRESH)                 \
    do {                                             \
        if (L.K <= 2) EP_DISPATCH(KERNEL, 2, FRESH); \
        else if (L.K <= 4) EP_DISPATCH(KERNEL, 4, FRESH); \
        else if (L.K <= 8) EP_DISPATCH(KERNEL, 8, FRESH); \
        else EP_DISPATCH(KERNEL, 16, FRESH);          \
    } while (0)

    if (L.use_fp8) {
        if (L.fresh) EP_DISPATCH_K(dispatch_fp8_kernel, true);
        else EP_DISPATCH_K(dispatch_fp8_kernel, false);
    } else {
        if (L.fresh) EP_DISPATCH_K(dispatch_bf16_kernel, true);
        else EP_DISPATCH_K(dispatch_bf16_kernel, false);
    }
#undef EP_DISPATCH_K
#undef EP_DISPATCH
    return hipGetLastError();
}

// Elementwise E4M3FN encoding with the same device converter.
__global__ __launch_bounds__(256) void e4m3fn_encode_kernel(const float* __restrict__ in,
                                                             uint8_t* __restrict__ out, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride)
        out[i] = (uint8_t)f32_to_e4m3fn(in[i]);
}

hipError_t launch_e4m3fn_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(e4m3fn_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace moe_ep
