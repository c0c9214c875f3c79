// Row part of dispatch, shared by the dispatch and low-latency dispatch
// kernels: read a token's row once with 16-byte loads and write it to each of
// its receive rows with 16-byte stores -- as BF16, or quantised once to
// E4M3FN with per-128-channel fp32 scales.
//
// FP8: each lane holds 16 consecutive channels, so 8 lanes cover one
// 128-channel block.  amax is reduced over those 8 lanes, the block's inverse
// scale 448/a is one correctly rounded fp32 division, and every value is
// multiplied by it and encoded before the stores.
#pragma once

#include "device.h"

namespace moe_ep {

#ifndef EP_DISPATCH_UNROLL
#define EP_DISPATCH_UNROLL 2
#endif
#ifndef EP_DISPATCH_MIN_ITEMS
#define EP_DISPATCH_MIN_ITEMS 65536
#endif
#ifndef EP_DISPATCH_MAX_ITERS
#define EP_DISPATCH_MAX_ITERS 4
#endif
#ifndef EP_DISPATCH_WAVES
#define EP_DISPATCH_WAVES 4
#endif
// Cache hints of the row traffic.  Measured on MI355X at the V3 shape: plain
// loads of x with non-temporal stores of the received rows is fastest (~98 us
// against ~125 us with both non-temporal and ~138 us with plain stores).  A
// receive buffer that fits the 256 MB Infinity Cache is written with plain
// stores instead (the dispatch launcher decides): 36 against 39 us for the
// skewed workload's 191 MB, and its step 98 against 101 us.
#ifndef EP_DISPATCH_NT_LOAD
#define EP_DISPATCH_NT_LOAD 0
#endif
#ifndef EP_DISPATCH_NT_STORE
#define EP_DISPATCH_NT_STORE 1
#endif
#ifndef EP_DISPATCH_CACHED_RECV_BYTES
#define EP_DISPATCH_CACHED_RECV_BYTES (256ll << 20)
#endif

constexpr int kDispatchWaves = EP_DISPATCH_WAVES;   // waves per workgroup
constexpr int kFp8ChPerIter = kWave * 16;           // 1024 channels per wave step
constexpr int kBf16ChPerIter = kWave * 8;           // 512 channels per wave step
constexpr int kDispatchUnroll = EP_DISPATCH_UNROLL; // wave steps with loads in flight


// Address of receive row r's scale of block b: row-major [rows][H/128] when
// scale_ld == 0, else column-major [H/128][scale_ld] (each block's scales
// contiguous over rows, the layout a grouped GEMM reads them in).
__device__ __forceinline__ size_t scale_index(int r, int b, int nb, int scale_ld)
{
    return scale_ld ? (size_t)b * scale_ld + r : (size_t)r * nb + b;
}

// Quantise one wave step (lane: 16 channels from cb, in lo / hi) and store the
// codes and block scales to the receive rows sk[].  Called by the whole wave:
// lanes past the row end (active false) hold zeros and only join the amax
// reduction.
template <int KMAX, bool NT = EP_DISPATCH_NT_STORE>
__device__ __forceinline__ void fp8_step_store(const u32x4& lo, const u32x4& hi, int cb, bool active,
                                               const int (&sk)[KMAX], int H, int scale_ld,
                                               uint8_t* __restrict__ recv, float* __restrict__ scales)
{
    const int lane = lane_id();
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_lo(lo[j]);
        v[2 * j + 1] = bf16_hi(lo[j]);
        v[8 + 2 * j] = bf16_lo(hi[j]);
        v[8 + 2 * j + 1] = bf16_hi(hi[j]);
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        m = fmaxf(m, fabsf(v[j]));
    // 8 lanes hold one 128-channel block
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    const float amax = fmaxf(m, 0x1p-64f);
    const float inv = 448.0f / amax;
    const float scale = amax / 448.0f;
    u32x4 q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        q[j] = f32_to_e4m3fn(v[4 * j] * inv) | (f32_to_e4m3fn(v[4 * j + 1] * inv) << 8) |
               (f32_to_e4m3fn(v[4 * j + 2] * inv) << 16) | (f32_to_e4m3fn(v[4 * j + 3] * inv) << 24);
    }
    if (active) {
        const int nb = H / kQBlock;
        const int blk = cb / kQBlock;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (sk[k] >= 0) {
                store16_hint<NT>(recv + (size_t)sk[k] * H + cb, q);
                if ((lane & 7) == 0)
                    scales[scale_index(sk[k], blk, nb, scale_ld)] = scale;
            }
        }
    }
}

// Load one FP8 wave step of the row (zeros past the row end).
__device__ __forceinline__ bool fp8_step_load(const uint16_t* __restrict__ xrow, int i, int H,
                                              u32x4& lo, u32x4& hi)
{
    const int cb = i * kFp8ChPerIter + lane_id() * 16;
    if (cb < H) {
        lo = load16_hint<EP_DISPATCH_NT_LOAD>(xrow + cb);
        hi = load16_hint<EP_DISPATCH_NT_LOAD>(xrow + cb + 8);
        return true;
    }
    lo = u32x4{0u, 0u, 0u, 0u};
    hi = u32x4{0u, 0u, 0u, 0u};
    return false;
}

// x[t] row -> K receive rows over wave steps [i_begin, i_end) of 1024 channels
template <int KMAX, bool NT>
__device__ __forceinline__ void fp8_rows(const uint16_t* __restrict__ xrow, const int (&sk)[KMAX],
                                         int H, int i_begin, int i_end, int scale_ld,
                                         uint8_t* __restrict__ recv, float* __restrict__ scales)
{
    const int lane = lane_id();
    for (int i0 = i_begin; i0 < i_end; i0 += kDispatchUnroll) {
        u32x4 lo[kDispatchUnroll], hi[kDispatchUnroll];
        bool act[kDispatchUnroll];
#pragma unroll
        for (int u = 0; u < kDispatchUnroll; ++u) {
            if (i0 + u < i_end) {
                act[u] = fp8_step_load(xrow, i0 + u, H, lo[u], hi[u]);
            } else {
                act[u] = false;
                lo[u] = u32x4{0u, 0u, 0u, 0u};
                hi[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < kDispatchUnroll; ++u) {
            if (i0 + u >= i_end)
                break;
            fp8_step_store<KMAX, NT>(lo[u], hi[u], (i0 + u) * kFp8ChPerIter + lane * 16, act[u], sk,
                                     H, scale_ld, recv, scales);
        }
    }
}

// Store one BF16 wave step (lane: 8 channels from cb) to the receive rows sk[].
template <int KMAX, bool NT = EP_DISPATCH_NT_STORE>
__device__ __forceinline__ void bf16_step_store(const u32x4& d, int cb, const int (&sk)[KMAX], int H,
                                                uint16_t* __restrict__ recv)
{
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        if (sk[k] >= 0)
            store16_hint<NT>(recv + (size_t)sk[k] * H + cb, d);
}

// x[t] row -> K receive rows over wave steps [i_begin, i_end) of 512 channels
template <int KMAX, bool NT>
__device__ __forceinline__ void bf16_rows(const uint16_t* __restrict__ xrow, const int (&sk)[KMAX],
                                          int H, int i_begin, int i_end,
                                          uint16_t* __restrict__ recv)
{
    const int lane = lane_id();
    for (int i0 = i_begin; i0 < i_end; i0 += kDispatchUnroll) {
        u32x4 d[kDispatchUnroll];
#pragma unroll
        for (int u = 0; u < kDispatchUnroll; ++u) {
            const int cb = (i0 + u) * kBf16ChPerIter + lane * 8;
            if (i0 + u < i_end && cb < H)
                d[u] = load16_hint<EP_DISPATCH_NT_LOAD>(xrow + cb);
        }
#pragma unroll
        for (int u = 0; u < kDispatchUnroll; ++u) {
            const int cb = (i0 + u) * kBf16ChPerIter + lane * 8;
            if (i0 + u < i_end && cb < H)
                bf16_step_store<KMAX, NT>(d[u], cb, sk, H, recv);
        }
    }
}

// Pre-quantised input: the token's E4M3FN codes (16 per lane, 1024 channels
// per wave step) and its block scales are copied to the receive rows sk[].
template <int KMAX, bool NT>
__device__ __forceinline__ void fp8in_rows(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                           const int (&sk)[KMAX], int H, int i_begin, int i_end,
                                           int scale_ld, uint8_t* __restrict__ recv,
                                           float* __restrict__ scales)
{
    const int lane = lane_id();
    const int nb = H / kQBlock;
    for (int i0 = i_begin; i0 < i_end; i0 += kDispatchUnroll) {
        u32x4 d[kDispatchUnroll];
        float sc[kDispatchUnroll];
#pragma unroll
        for (int u = 0; u < kDispatchUnroll; ++u) {
            const int cb = (i0 + u) * kFp8ChPerIter + lane * 16;
            if (i0 + u < i_end && cb < H) {
                d[u] = load16_hint<EP_DISPATCH_NT_LOAD>(xq + cb);
                sc[u] = xs[cb / kQBlock];
            }
        }
#pragma unroll
        for (int u = 0; u < kDispatchUnroll; ++u) {
            const int cb = (i0 + u) * kFp8ChPerIter + lane * 16;
            if (i0 + u < i_end && cb < H) {
                const int blk = cb / kQBlock;
#pragma unroll
                for (int k = 0; k < KMAX; ++k) {
                    if (sk[k] >= 0) {
                        store16_hint<NT>(recv + (size_t)sk[k] * H + cb, d[u]);
                        if ((lane & 7) == 0)
                            scales[scale_index(sk[k], blk, nb, scale_ld)] = sc[u];
                    }
                }
            }
        }
    }
}

// Zero one padding row of a GEMM-aligned layout (its codes or BF16 values,
// and its scales in FP8 mode).  Called by a whole wave.
template <bool NT>
__device__ __forceinline__ void zero_row(void* __restrict__ recv, float* __restrict__ scales, int row,
                                         int H, bool fp8, int scale_ld)
{
    const int lane = lane_id();
    const size_t row_bytes = (size_t)H * (fp8 ? 1 : 2);
    uint8_t* dst = static_cast<uint8_t*>(recv) + (size_t)row * row_bytes;
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    for (size_t off = (size_t)lane * 16; off < row_bytes; off += kWave * 16)
        store16_hint<NT>(dst + off, z);
    if (fp8) {
        const int nb = H / kQBlock;
        for (int b = lane; b < nb; b += kWave)
            scales[scale_index(row, b, nb, scale_ld)] = 0.0f;
    }
}

}  // namespace moe_ep
