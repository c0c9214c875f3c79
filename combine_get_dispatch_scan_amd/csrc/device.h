// Device helpers shared by the moe_ep kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_ep {

constexpr int kWave = 64;
constexpr int kChunk = 256;        // tokens per layout workgroup (4 waves)
constexpr int kChunkWaves = kChunk / kWave;
constexpr int kQBlock = 128;       // channels per FP8 scale

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Work split of a row-streaming kernel: each token row has `iters` wave
// steps; a work item (one wave) takes `iters_per_seg` consecutive steps of
// one row (a segment; `nseg` segments per row).  Rows are split only as far
// as needed to give the launch at least `min_items` work items and no item
// more than `max_iters_per_item` steps.
struct RowSplit {
    int nseg, iters_per_seg;
};

inline RowSplit split_rows(int T, int iters, int min_items, int max_iters_per_item)
{
    int n = 1;
    if (T > 0) {
        n = (min_items + T - 1) / T;
        int need = (iters + max_iters_per_item - 1) / max_iters_per_item;
        if (n < need)
            n = need;
    }
    if (n > iters)
        n = iters;
    if (n < 1)
        n = 1;
    RowSplit r;
    r.iters_per_seg = (iters + n - 1) / n;
    r.nseg = (iters + r.iters_per_seg - 1) / r.iters_per_seg;
    return r;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int readlane(int v, int lane)
{
    return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// 16-byte accesses with an optional non-temporal hint (data touched once).
template <bool NT>
__device__ __forceinline__ u32x4 load16_hint(const void* p)
{
    if (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return *reinterpret_cast<const u32x4*>(p);
}

template <bool NT>
__device__ __forceinline__ void store16_hint(void* p, u32x4 v)
{
    if (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else
        *reinterpret_cast<u32x4*>(p) = v;
}

// Buffer-resource store with an explicit cache policy.  The descriptor covers
// `bytes` bytes from `base` (gfx9 word 3: 32-bit untyped access); `aux` holds
// the gfx950 policy bits sc0 = 1, nt = 2, sc1 = 16.  The compiler tracks these
// like any other store; offsets at or past `bytes` are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

template <int AUX>
__device__ __forceinline__ void buffer_store16(u32x4 v, __amdgpu_buffer_rsrc_t r, int byte_off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, AUX);
}

// Buffer-resource loads.  Offsets at or past the descriptor's range read
// zeros without touching memory, so a descriptor with an empty range stands
// for a row that does not exist (a masked pair), and lanes past the row end
// need no branch.
template <int AUX>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, AUX);
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Descriptor of row `row` (`row_bytes` bytes) of a row-major array, or an
// empty range when row < 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int row, int row_bytes)
{
    const bool valid = row >= 0;
    const char* p = static_cast<const char*>(base) + (valid ? (size_t)row * row_bytes : 0);
    return make_rsrc(const_cast<char*>(p), valid ? row_bytes : 0);
}

// BF16 <-> fp32.  Widening is exact; narrowing rounds to nearest, ties to
// even, on the 16 dropped bits (operands are finite by contract).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// fp32 -> OCP E4M3FN (bias 7, 3 mantissa bits, max 448, no infinities),
// round to nearest even, saturating to +-448, sign of zero kept.
//  |v| >= 448        -> 0x7E
//  |v| in [2^-6,448) -> RNE on the 20 low mantissa bits of the fp32 pattern;
//                       the fp32 exponent (bias 127) maps to bias 7 by
//                       subtracting 120 << 3 from the top 12 bits
//  |v| < 2^-6        -> subnormal code n = rint(|v| * 2^9) in 0..8 (8 is the
//                       smallest normal, whose code is also 8)
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float v)
{
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E00000u) {                     // 448.0
        code = 0x7Eu;
    } else if (a >= 0x3C800000u) {              // 2^-6
        uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);
    } else {
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | code;
}

// Two OCP E4M3FN codes (bytes 0,1 or, with HI, bytes 2,3 of w) -> their exact
// fp32 values, with gfx950's converter (v_cvt_pk_f32_fp8).  It decodes the OCP
// format exactly -- subnormals m * 2^-9, 0x7F / 0xFF as NaN: a probe compared
// all 256 codes with the formula, and a device test keeps checking the 254
// finite ones through the FP8 combine.
template <bool HI>
__device__ __forceinline__ void e4m3fn_pair_to_f32(uint32_t w, float& a, float& b)
{
    const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
    a = v[0];
    b = v[1];
}

}  // namespace moe_ep
