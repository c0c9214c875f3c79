// Backward of combine on gfx950.
//
// The backward of combine is dispatch (stakiran github-trend-summarizer,
// "DeepEP 要約", section 3): combine computes out[t] = sum_k w[t,k] *
// y[slot[t,k]], which is linear in y and in w, so
//     grad_y[slot[t,k]] = bf16_rne(w[t,k] * grad_out[t])     (one fp32 product)
//     grad_w[t,k]       = <grad_out[t], y[slot[t,k]]>          (fp32 dot product)
// The first is a weight-scaled BF16 dispatch of grad_out along the forward
// routing; the second needs the forward's expert outputs y.
//
// Without grad_w a work item is one wave on a segment of the row, as in
// dispatch.  With grad_w a workgroup of 8 waves owns one token: wave w takes
// the wave steps w, w+8, w+16, ... of the row, and each dot product is reduced
// in a fixed order -- a per-lane fma chain over the lane's channels, an
// xor-shuffle tree over the 64 lanes, then the 8 waves' partial sums added in
// wave order through LDS -- so grad_w is deterministic.
#include "device.h"
#include "launch.h"

namespace moe_ep {

// 8 waves with one step in flight each measured faster than 4 waves with two
// (8192 tokens x 7168 channels, top-8, grad_w on: 418 -> 406 us in one
// process); 7, 14 and 16 waves were no better.
constexpr int kBwdWaves = 8;
constexpr int kBwdChPerIter = kWave * 8;     // 512 channels per wave step
constexpr int kBwdUnroll = 1;

struct CombineBwdArgs {
    const uint16_t* grad_out;
    const uint16_t* y;
    int T, H, K;
    int nseg, iters_per_seg, iters;
    const int32_t* slot;
    const float* w;
    uint16_t* grad_y;
    float* grad_w;
};

__device__ __forceinline__ int slot_of(const CombineBwdArgs& a, int t, int k)
{
    return a.slot[(size_t)t * a.K + k];
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m);
    return v;
}

template <int KMAX, bool WGRAD>
__global__ __launch_bounds__(kBwdWaves * kWave) void combine_backward_kernel(CombineBwdArgs a)
{
    __shared__ float lds_part[kBwdWaves][16];
    const int wave = threadIdx.x / kWave;
    const int wi = blockIdx.x * kBwdWaves + wave;
    // WGRAD: token = block, the block's waves interleave over the row's steps
    const int t = WGRAD ? (int)blockIdx.x : wi / a.nseg;
    const int seg = WGRAD ? 0 : wi % a.nseg;
    if (t >= a.T)
        return;
    const int lane = lane_id();
    int s_own = -1;
    float w_own = 0.0f;
    if (lane < a.K) {
        s_own = a.slot[(size_t)t * a.K + lane];
        w_own = a.w[(size_t)t * a.K + lane];
    }
    int sk[KMAX];
    float wk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        sk[k] = k < a.K ? readlane(s_own, k) : -1;
        wk[k] = k < a.K ? readlane_f(w_own, k) : 0.0f;
    }
    float dot[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        dot[k] = 0.0f;

    const int H = a.H;
    const uint16_t* grow = a.grad_out + (size_t)t * H;
    // steps i_begin, i_begin + stride, ... below i_end
    const int stride = WGRAD ? kBwdWaves : 1;
    const int i_begin = WGRAD ? wave : seg * a.iters_per_seg;
    const int i_end = WGRAD ? a.iters : min(a.iters, i_begin + a.iters_per_seg);

    for (int i0 = i_begin; i0 < i_end; i0 += kBwdUnroll * stride) {
        u32x4 g[kBwdUnroll];
        u32x4 yv[kBwdUnroll][KMAX];
#pragma unroll
        for (int u = 0; u < kBwdUnroll; ++u) {
            const int cb = (i0 + u * stride) * kBwdChPerIter + lane * 8;
            const bool active = (i0 + u * stride < i_end) && cb < H;
            // grad_out with plain loads, y and grad_y non-temporal.  At
            // 8192 x 7168 top-8, back to back: 382.9 against 399.5 us with a
            // non-temporal grad_out (its 117 MB can stay in the Infinity Cache,
            // as a gradient the previous layer has just written would); after a
            // 2 GiB read that empties the caches: 405.3 against 407.1 us.
            if (active)
                g[u] = load16_hint<false>(grow + cb);
            if (WGRAD) {
#pragma unroll
                for (int k = 0; k < KMAX; ++k)
                    if (sk[k] >= 0 && active)
                        yv[u][k] = load16_hint<true>(a.y + (size_t)sk[k] * H + cb);
            }
        }
#pragma unroll
        for (int u = 0; u < kBwdUnroll; ++u) {
            const int cb = (i0 + u * stride) * kBwdChPerIter + lane * 8;
            const bool active = (i0 + u * stride < i_end) && cb < H;
            if (!active)
                continue;
            float gf[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gf[2 * j] = bf16_lo(g[u][j]);
                gf[2 * j + 1] = bf16_hi(g[u][j]);
            }
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (sk[k] < 0)
                    continue;
                u32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = pack_bf16x2(wk[k] * gf[2 * j], wk[k] * gf[2 * j + 1]);
                store16_hint<true>(a.grad_y + (size_t)sk[k] * H + cb, o);
                if (WGRAD) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        dot[k] = __builtin_fmaf(gf[2 * j], bf16_lo(yv[u][k][j]), dot[k]);
                        dot[k] = __builtin_fmaf(gf[2 * j + 1], bf16_hi(yv[u][k][j]), dot[k]);
                    }
                }
            }
        }
    }
    if (WGRAD) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const float s = wave_sum(dot[k]);
            if (lane == 0)
                lds_part[wave][k] = s;
        }
        __syncthreads();
        if (threadIdx.x < a.K) {
            const int k = threadIdx.x;
            float s = lds_part[0][k];
#pragma unroll
            for (int v = 1; v < kBwdWaves; ++v)
                s += lds_part[v][k];
            a.grad_w[(size_t)t * a.K + k] = slot_of(a, t, k) >= 0 ? s : 0.0f;
        }
    }
}

hipError_t launch_combine_backward(const void* grad_out, const void* y, int T, int H, int K,
                                   const int32_t* slot, const float* w, void* grad_y,
                                   float* grad_w, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    CombineBwdArgs a;
    a.grad_out = static_cast<const uint16_t*>(grad_out);
    a.y = static_cast<const uint16_t*>(y);
    a.T = T;
    a.H = H;
    a.K = K;
    a.slot = slot;
    a.w = w;
    a.grad_y = static_cast<uint16_t*>(grad_y);
    a.grad_w = grad_w;
    a.iters = (H + kBwdChPerIter - 1) / kBwdChPerIter;
    const bool wgrad = grad_w != nullptr;
    dim3 grid;
    if (wgrad) {
        // one workgroup per token keeps each dot product's reduction order fixed
        a.nseg = 1;
        a.iters_per_seg = a.iters;
        grid = dim3((unsigned)T);
    } else {
        const RowSplit rs = split_rows(T, a.iters, 65536, 4);
        a.nseg = rs.nseg;
        a.iters_per_seg = rs.iters_per_seg;
        const long long items = (long long)T * a.nseg;
        grid = dim3((unsigned)((items + kBwdWaves - 1) / kBwdWaves));
    }
    dim3 block(kBwdWaves * kWave);
#define EP_BWD(KM)                                                                                   \
    do {                                                                                             \
        debug_launch(wgrad ? "combine_backward_kernel<wgrad>" : "combine_backward_kernel", grid, block, 0); \
        if (wgrad) hipLaunchKernelGGL((combine_backward_kernel<KM, true>), grid, block, 0, stream, a); \
        else hipLaunchKernelGGL((combine_backward_kernel<KM, false>), grid, block, 0, stream, a);      \
    } while (0)
    if (K <= 2) EP_BWD(2);
    else if (K <= 4) EP_BWD(4);
    else if (K <= 8) EP_BWD(8);
    else EP_BWD(16);
#undef EP_BWD
    return hipGetLastError();
}

}  // namespace moe_ep
