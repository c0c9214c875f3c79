// combine on gfx950: gather each token's expert-output rows and reduce them.
//
// combine reduces the expert outputs back to the token's origin (GeekNews
// usage section; stakiran github-trend-summarizer section 3: combine(y,
// handle)), in BF16 with fp32 accumulation (aikraft.ru "Технические детали и
// требования": BF16 combine).  Per token and channel:
//     acc = +0.0f;  for k ascending with slot >= 0: acc = fma(w[t,k], y[slot][j], acc)
//     out[t][j] = bf16_rne(acc)
//
// Work item = (token, segment of the row), one wave each.  Lanes 0..K-1 read
// the token's receive rows and weights, which are broadcast to the wave as
// scalars.  Each lane owns 8 channels per wave step; all K 16-byte gathers of
// a step (and of kCombineUnroll steps) are issued before the first fma.
#include <stdlib.h>

#include "device.h"
#include "launch.h"

namespace moe_ep {

#ifndef EP_COMBINE_UNROLL
#define EP_COMBINE_UNROLL 2
#endif
#ifndef EP_COMBINE_MIN_ITEMS
#define EP_COMBINE_MIN_ITEMS 131072
#endif
#ifndef EP_COMBINE_MAX_ITERS
#define EP_COMBINE_MAX_ITERS 2
#endif
#ifndef EP_COMBINE_WAVES
#define EP_COMBINE_WAVES 4
#endif
// Cache policy, measured on MI355X.  The gathered rows are touched once:
// non-temporal loads (plain loads: 204.6 against 170.8 us at the V3 shape).
//
// Output stores: at the V3 shape (117 MB of output) device-scope (sc1)
// buffer stores, which write through the XCD's L2, are fastest: ~173 us,
// against ~182 us with plain write-back or non-temporal stores.  The output
// writes cost far more than their share of bandwidth because they interleave
// with the 940 MB read stream at the DRAM; write-through spreads them best.
//
// Above EP_COMBINE_STREAM_OUT_BYTES of output the stores are non-temporal
// instead.  At the large workload (235 MB of output against the 256 MB
// Infinity Cache) write-through lines stay dirty in the Infinity Cache and
// are written back during the next call: the next step's dispatch took
// 282 us after a write-through combine and 218 us after a non-temporal one,
// while the combine itself went from 366 to 380 us (step 669 -> 618 us).  At
// V3 the write-through step is faster (294 us against 304 us).
#ifndef EP_COMBINE_NT_LOAD
#define EP_COMBINE_NT_LOAD 1
#endif
#ifndef EP_COMBINE_STORE_AUX
#define EP_COMBINE_STORE_AUX 16                  // sc1
#endif
#ifndef EP_COMBINE_STREAM_OUT_BYTES
#define EP_COMBINE_STREAM_OUT_BYTES (160ll << 20)
#endif
constexpr int kCombineStreamAux = 2;             // nt

constexpr int kCombineWaves = EP_COMBINE_WAVES;
constexpr int kCombineChPerIter = kWave * 8;     // 512 channels per wave step
constexpr int kCombineUnroll = EP_COMBINE_UNROLL;

struct CombineArgs {
    const uint16_t* y;
    int T, H, K;
    int nseg, iters_per_seg, iters;
    int g;                    // tokens per workgroup of the token-owner form
    const int32_t* slot;
    const float* w;
    uint16_t* out;
};

// UNIT: every weight is 1 (the backward of dispatch); fma(1, v, acc) is the
// exact sum acc + v, so no weights are read.  AUX: cache policy of the
// output stores.
template <int KMAX, bool UNIT, int AUX>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(CombineArgs a)
{
    const int wi = blockIdx.x * kCombineWaves + threadIdx.x / kWave;
    const int t = wi / a.nseg;
    const int seg = wi % a.nseg;
    if (t >= a.T)
        return;
    const int lane = lane_id();
    int s_own = -1;
    float w_own = 0.0f;
    if (lane < a.K) {
        s_own = a.slot[(size_t)t * a.K + lane];
        w_own = UNIT ? 1.0f : a.w[(size_t)t * a.K + lane];
    }
    int sk[KMAX];
    float wk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        sk[k] = k < a.K ? readlane(s_own, k) : -1;
        wk[k] = k < a.K ? readlane_f(w_own, k) : 0.0f;
    }

    const int H = a.H;
    // one descriptor per output row keeps the byte offsets small for any T
    const __amdgpu_buffer_rsrc_t orow = make_rsrc(a.out + (size_t)t * H, H * 2);
    const int i_begin = seg * a.iters_per_seg;
    const int i_end = min(a.iters, i_begin + a.iters_per_seg);

    for (int i0 = i_begin; i0 < i_end; i0 += kCombineUnroll) {
        u32x4 d[kCombineUnroll][KMAX];
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const int cb = (i0 + u) * kCombineChPerIter + lane * 8;
            const bool active = (i0 + u < i_end) && cb < H;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (sk[k] >= 0 && active)
                    d[u][k] = load16_hint<EP_COMBINE_NT_LOAD>(a.y + (size_t)sk[k] * H + cb);
        }
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const int cb = (i0 + u) * kCombineChPerIter + lane * 8;
            const bool active = (i0 + u < i_end) && cb < H;
            float acc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (sk[k] >= 0 && active) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[2 * j] = __builtin_fmaf(wk[k], bf16_lo(d[u][k][j]), acc[2 * j]);
                        acc[2 * j + 1] = __builtin_fmaf(wk[k], bf16_hi(d[u][k][j]), acc[2 * j + 1]);
                    }
                }
            }
            if (active) {
                u32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
                buffer_store16<AUX>(o, orow, cb * 2);
            }
        }
    }
}

// Token-owner form: a workgroup of kOwnerWaves waves owns `g` whole tokens.
// Wave w takes the 512-channel steps w, w + W, w + 2W, ... of the workgroup's
// g * S steps (S steps per token), one at a time.  Each step gathers its K row
// pieces, reduces them exactly as combine_kernel does (same fma order), and
// leaves its 1 KB of BF16 results in LDS; after a barrier the workgroup writes
// its g output rows as one contiguous piece.  One step at a time keeps the
// kernel near 50 VGPRs for K <= 8, so two workgroups share a CU and one
// writes while the other gathers.  Two steps at a time (93 VGPRs, one workgroup per CU) was
// 3% faster on dense routing (large workload: 359 against 371 us) but 23%
// slower on rows with few valid pairs (expert-parallel pre-reduction at the
// V3 shape: 287 against 234 us), and the launcher cannot tell them apart.
constexpr int kOwnerWaves = 16;
constexpr int kOwnerStreamAux = 18;              // nt | sc1: outputs past the Infinity Cache
constexpr int kOwnerLdsBytes = 65536;            // g * H * 2 bytes of staged output at most

template <int KMAX, bool UNIT>
__device__ __forceinline__ void owner_meta(const CombineArgs& a, int t, int (&sk)[KMAX], float (&wk)[KMAX])
{
    const int lane = lane_id();
    int s_own = -1;
    float w_own = 0.0f;
    if (lane < a.K) {
        s_own = a.slot[(size_t)t * a.K + lane];
        w_own = UNIT ? 1.0f : a.w[(size_t)t * a.K + lane];
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        sk[k] = k < a.K ? readlane(s_own, k) : -1;
        wk[k] = k < a.K ? readlane_f(w_own, k) : 0.0f;
    }
}

template <int KMAX, bool UNIT, int AUX>
__global__ __launch_bounds__(kOwnerWaves * kWave) void combine_owner_kernel(CombineArgs a)
{
    extern __shared__ u32x4 lds_out[];                  // [g][H / 8]
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int H = a.H;
    const int S = a.iters;
    const int t0 = blockIdx.x * a.g;
    const int ntok = min(a.g, a.T - t0);
    const int nsteps = ntok * S;
    for (int s = wave; s < nsteps; s += kOwnerWaves) {
        const int g = s / S;
        int sk[KMAX];
        float wk[KMAX];
        owner_meta<KMAX, UNIT>(a, t0 + g, sk, wk);
        const int cb = (s - g * S) * kCombineChPerIter + lane * 8;
        const bool act = cb < H;
        u32x4 d[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (sk[k] >= 0 && act)
                d[k] = load16_hint<EP_COMBINE_NT_LOAD>(a.y + (size_t)sk[k] * H + cb);
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (sk[k] >= 0 && act) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[2 * j] = __builtin_fmaf(wk[k], bf16_lo(d[k][j]), acc[2 * j]);
                    acc[2 * j + 1] = __builtin_fmaf(wk[k], bf16_hi(d[k][j]), acc[2 * j + 1]);
                }
            }
        }
        if (act) {
            u32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
            lds_out[(g * H + cb) / 8] = o;
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t orow = make_rsrc(a.out + (size_t)t0 * H, ntok * H * 2);
    const int n16 = ntok * H / 8;
    for (int i = threadIdx.x; i < n16; i += kOwnerWaves * kWave)
        buffer_store16<AUX>(lds_out[i], orow, i * 16);
}

// Combine of FP8 rows: every gathered element is first widened to
// decode(q) * (its block's scale), one fp32 multiply, then reduced as above.
// Each lane owns 16 channels (one 16-byte load per row) per wave step of 1024
// channels; its 8-lane group shares one 128-channel block, so one scale per
// row; the 16 BF16 results leave as two 16-byte stores.  The scales are laid
// out as dispatch wrote them: row-major [rows][H/128], or column-major
// [H/128][scale_ld] (scale_ld != 0).
struct CombineFp8Args {
    const uint8_t* y;
    const float* scales;
    int scale_ld;
    int T, H, K;
    int nseg, iters_per_seg, iters;
    const int32_t* slot;
    const float* w;
    uint16_t* out;
};

#ifndef EP_COMBINE_FP8_UNROLL
#define EP_COMBINE_FP8_UNROLL 1
#endif
#ifndef EP_COMBINE_FP8_MAX_ITERS
#define EP_COMBINE_FP8_MAX_ITERS 4
#endif
// Output stores, measured at the V3 shape on dispatch's own FP8 rows, for
// the weighted / unit-weight kernels: plain write-back 99.0 / 98.4 us,
// non-temporal 106.6 / 109.3 us, write-through (sc1) 122.7 / 122.3 us.
// Plain loads of the rows instead of non-temporal ones: 118.2 / 118.8 us.
#ifndef EP_COMBINE_FP8_STORE_AUX
#define EP_COMBINE_FP8_STORE_AUX 0
#endif
constexpr int kCombineFp8ChPerIter = kWave * 16;   // 1024 channels per wave step
constexpr int kCombineFp8Unroll = EP_COMBINE_FP8_UNROLL;

// UNIT: unit weights.  ROWBUF: unit weights on row-major scales, read through
// per-row buffer descriptors (the hot form of the backward of dispatch).
template <int KMAX, bool UNIT, bool ROWBUF>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_fp8_kernel(CombineFp8Args a)
{
    const int wi = blockIdx.x * kCombineWaves + threadIdx.x / kWave;
    const int t = wi / a.nseg;
    const int seg = wi % a.nseg;
    if (t >= a.T)
        return;
    const int lane = lane_id();
    int s_own = -1;
    float w_own = 0.0f;
    if (lane < a.K) {
        s_own = a.slot[(size_t)t * a.K + lane];
        w_own = UNIT ? 1.0f : a.w[(size_t)t * a.K + lane];
    }
    int sk[KMAX];
    float wk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        sk[k] = k < a.K ? readlane(s_own, k) : -1;
        wk[k] = k < a.K ? readlane_f(w_own, k) : 0.0f;
    }

    const int H = a.H;
    const int nb = H / kQBlock;
    const __amdgpu_buffer_rsrc_t orow = make_rsrc(a.out + (size_t)t * H, H * 2);
    const int i_begin = seg * a.iters_per_seg;
    const int i_end = min(a.iters, i_begin + a.iters_per_seg);

    if constexpr (ROWBUF) {
        // Unit weights read the rows and scales through per-row buffer
        // descriptors, with no predicated load: a masked pair's descriptors
        // have an empty range and read zeros, as do lanes past the row end
        // (whose stores the output descriptor drops), and its weight is 0, so
        // fma(0, 0, acc) leaves acc (which starts at +0 and never becomes -0).
        // The predicated form below, compiled with a constant weight, waited
        // for each gather before issuing the next: 117.5 us against 100.3 us
        // at 8192 x 7168 top-8.  With read weights the predicated form is the
        // faster one (98.5 us against 101.0 us).
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            wk[k] = sk[k] >= 0 ? 1.0f : 0.0f;
        for (int i = i_begin; i < i_end; ++i) {
            const int cb = i * kCombineFp8ChPerIter + lane * 16;
            u32x4 d[KMAX];
            float sc[KMAX];
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                d[k] = buffer_load16<EP_COMBINE_NT_LOAD ? 2 : 0>(row_rsrc(a.y, sk[k], H), cb);
                sc[k] = buffer_load_f32(row_rsrc(a.scales, sk[k], nb * 4), cb / kQBlock * 4);
            }
            float acc[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v[4];
                    e4m3fn_pair_to_f32<false>(d[k][j], v[0], v[1]);
                    e4m3fn_pair_to_f32<true>(d[k][j], v[2], v[3]);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc[4 * j + b] = __builtin_fmaf(wk[k], v[b] * sc[k], acc[4 * j + b]);
                }
            }
            u32x4 o0, o1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o0[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
                o1[j] = pack_bf16x2(acc[8 + 2 * j], acc[8 + 2 * j + 1]);
            }
            buffer_store16<EP_COMBINE_FP8_STORE_AUX>(o0, orow, cb * 2);
            buffer_store16<EP_COMBINE_FP8_STORE_AUX>(o1, orow, cb * 2 + 16);
        }
        return;
    }

    for (int i0 = i_begin; i0 < i_end; i0 += kCombineFp8Unroll) {
        u32x4 d[kCombineFp8Unroll][KMAX];
        float sc[kCombineFp8Unroll][KMAX];
#pragma unroll
        for (int u = 0; u < kCombineFp8Unroll; ++u) {
            const int cb = (i0 + u) * kCombineFp8ChPerIter + lane * 16;
            const bool active = (i0 + u < i_end) && cb < H;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (sk[k] >= 0 && active) {
                    d[u][k] = load16_hint<EP_COMBINE_NT_LOAD>(a.y + (size_t)sk[k] * H + cb);
                    sc[u][k] = a.scales[a.scale_ld ? (size_t)(cb / kQBlock) * a.scale_ld + sk[k]
                                                   : (size_t)sk[k] * nb + cb / kQBlock];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kCombineFp8Unroll; ++u) {
            const int cb = (i0 + u) * kCombineFp8ChPerIter + lane * 16;
            const bool active = (i0 + u < i_end) && cb < H;
            float acc[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (sk[k] >= 0 && active) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float v[4];
                        e4m3fn_pair_to_f32<false>(d[u][k][j], v[0], v[1]);
                        e4m3fn_pair_to_f32<true>(d[u][k][j], v[2], v[3]);
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            acc[4 * j + b] = __builtin_fmaf(wk[k], v[b] * sc[u][k], acc[4 * j + b]);
                    }
                }
            }
            if (active) {
                u32x4 o0, o1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o0[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
                    o1[j] = pack_bf16x2(acc[8 + 2 * j], acc[8 + 2 * j + 1]);
                }
                buffer_store16<EP_COMBINE_FP8_STORE_AUX>(o0, orow, cb * 2);
                buffer_store16<EP_COMBINE_FP8_STORE_AUX>(o1, orow, cb * 2 + 16);
            }
        }
    }
}

hipError_t launch_combine_fp8(const void* y, const float* scales, int scale_ld, int T, int H, int K,
                              const int32_t* slot, const float* w, void* out, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    CombineFp8Args a;
    a.y = static_cast<const uint8_t*>(y);
    a.scales = scales;
    a.scale_ld = scale_ld;
    a.T = T;
    a.H = H;
    a.K = K;
    a.slot = slot;
    a.w = w;
    a.out = static_cast<uint16_t*>(out);
    a.iters = (H + kCombineFp8ChPerIter - 1) / kCombineFp8ChPerIter;
    const RowSplit rs = split_rows(T, a.iters, EP_COMBINE_MIN_ITEMS, EP_COMBINE_FP8_MAX_ITERS);
    a.nseg = rs.nseg;
    a.iters_per_seg = rs.iters_per_seg;
    const long long items = (long long)T * a.nseg;
    dim3 grid((unsigned)((items + kCombineWaves - 1) / kCombineWaves));
    dim3 block(kCombineWaves * kWave);
    // column-major scales with unit weights take the predicated form: a
    // buffer descriptor cannot follow a strided column per row
#define EP_COMBINE8(KM)                                                                                \
    do {                                                                                               \
        debug_launch("combine_fp8_kernel", grid, block, 0);                                            \
        if (w) hipLaunchKernelGGL((combine_fp8_kernel<KM, false, false>), grid, block, 0, stream, a);  \
        else if (scale_ld) hipLaunchKernelGGL((combine_fp8_kernel<KM, true, false>), grid, block, 0, stream, a); \
        else hipLaunchKernelGGL((combine_fp8_kernel<KM, true, true>), grid, block, 0, stream, a);      \
    } while (0)
    if (K <= 2) EP_COMBINE8(2);
    else if (K <= 4) EP_COMBINE8(4);
    else if (K <= 8) EP_COMBINE8(8);
    else EP_COMBINE8(16);
#undef EP_COMBINE8
    return hipGetLastError();
}

// Which form of the BF16 combine runs: the token-owner form for outputs
// past EP_COMBINE_STREAM_OUT_BYTES, the segmented form otherwise.
// EP_COMBINE_OWNER=1 / 0 in the environment forces one form (read at every
// launch; for tests and measurements).
static bool use_owner_form(bool stream_out)
{
    const char* v = getenv("EP_COMBINE_OWNER");
    if (v && v[0] == '1')
        return true;
    if (v && v[0] == '0')
        return false;
    return stream_out;
}

hipError_t launch_combine(const void* y, int T, int H, int K, const int32_t* slot,
                          const float* w, void* out, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    CombineArgs a;
    a.y = static_cast<const uint16_t*>(y);
    a.T = T;
    a.H = H;
    a.K = K;
    a.slot = slot;
    a.w = w;
    a.out = static_cast<uint16_t*>(out);
    a.iters = (H + kCombineChPerIter - 1) / kCombineChPerIter;
    const RowSplit rs = split_rows(T, a.iters, EP_COMBINE_MIN_ITEMS, EP_COMBINE_MAX_ITERS);
    a.nseg = rs.nseg;
    a.iters_per_seg = rs.iters_per_seg;
    const long long items = (long long)T * a.nseg;
    dim3 grid((unsigned)((items + kCombineWaves - 1) / kCombineWaves));
    dim3 block(kCombineWaves * kWave);
    const bool stream_out = (long long)T * H * 2 > EP_COMBINE_STREAM_OUT_BYTES;
    if (use_owner_form(stream_out)) {
        a.g = min(4, kOwnerLdsBytes / (H * 2));        // >= 1: H <= 32768
        dim3 og((unsigned)((T + a.g - 1) / a.g));
        dim3 ob(kOwnerWaves * kWave);
        const size_t lds = (size_t)a.g * H * 2;
#define EP_OWNER_A(KM, AUX)                                                                                \
    do {                                                                                                   \
        if (w) hipLaunchKernelGGL((combine_owner_kernel<KM, false, AUX>), og, ob, lds, stream, a);         \
        else hipLaunchKernelGGL((combine_owner_kernel<KM, true, AUX>), og, ob, lds, stream, a);            \
    } while (0)
#define EP_OWNER(KM)                                                                                       \
    do {                                                                                                   \
        debug_launch(stream_out ? "combine_owner_kernel<nt>" : "combine_owner_kernel", og, ob, lds);       \
        if (stream_out) EP_OWNER_A(KM, kOwnerStreamAux);                                                   \
        else EP_OWNER_A(KM, EP_COMBINE_STORE_AUX);                                                         \
    } while (0)
        if (K <= 2) EP_OWNER(2);
        else if (K <= 4) EP_OWNER(4);
        else if (K <= 8) EP_OWNER(8);
        else EP_OWNER(16);
#undef EP_OWNER
#undef EP_OWNER_A
        return hipGetLastError();
    }
    a.g = 0;
#define EP_COMBINE_A(KM, AUX)                                                                   \
    do {                                                                                        \
        if (w) hipLaunchKernelGGL((combine_kernel<KM, false, AUX>), grid, block, 0, stream, a); \
        else hipLaunchKernelGGL((combine_kernel<KM, true, AUX>), grid, block, 0, stream, a);    \
    } while (0)
#define EP_COMBINE(KM)                                                                          \
    do {                                                                                        \
        debug_launch(stream_out ? "combine_kernel<nt>" : "combine_kernel", grid, block, 0);     \
        if (stream_out) EP_COMBINE_A(KM, kCombineStreamAux);                                    \
        else EP_COMBINE_A(KM, EP_COMBINE_STORE_AUX);                                            \
    } while (0)
    if (K <= 2) EP_COMBINE(2);
    else if (K <= 4) EP_COMBINE(4);
    else if (K <= 8) EP_COMBINE(8);
    else EP_COMBINE(16);
#undef EP_COMBINE
#undef EP_COMBINE_A
    return hipGetLastError();
}

}  // namespace moe_ep
