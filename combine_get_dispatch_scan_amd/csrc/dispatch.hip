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
// handled by fp8_rows / fp8in_rows / bf16_rows (dispatch_rows.h).
//
// GEMM-facing options (GeekNews, "Những thay đổi chính của bản phát hành
// V2": a new GEMM layout; usage section: counts per expert feed the grouped
// GEMM): expert blocks aligned to a row tile with zeroed padding rows,
// column-major block scales, and input that arrives already quantised.
#include "device.h"
#include "dispatch_rows.h"
#include "launch.h"

namespace moe_ep {

struct DispatchArgs {
    const uint16_t* x;
    const float* x_scales;    // pre-quantised input: x holds E4M3FN codes
    int T, H, K, E, B;
    int nseg, iters_per_seg, iters;
    int row_blocks;           // workgroups that move rows; the rest zero padding
    int align;                // rows per GEMM tile of an aligned layout (1: dense)
    int scale_ld;             // 0: row-major scales, else column-major leading dim
    int seq;                  // the handle's dispatch number (the overflow mark)
    int capacity;
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
                if (s >= 0 && a.src_token)
                    a.src_token[s] = t;
                if (a.w_in)
                    a.w_copy[i] = a.w_in[i];
                if (ovf)
                    a.status[0] = a.seq;
            }
        } else {
            s = a.slot[i];
        }
    }
    return s;
}

// Workgroups past row_blocks zero the padding rows of a GEMM-aligned layout:
// one wave per (expert, padding row index < align - 1).  Expert e's block is
// [expert_offset[e], expert_offset[e+1]) and its rows from expert_offset[e] +
// count(e) on are padding; count(e) is the last chunk's base plus its count.
template <bool NT>
__device__ __forceinline__ void pad_item(const DispatchArgs& a, bool fp8)
{
    const int item = (blockIdx.x - a.row_blocks) * kDispatchWaves + threadIdx.x / kWave;
    const int per = a.align - 1;
    const int e = item / per;
    if (e >= a.E)
        return;
    const size_t last = (size_t)(a.B - 1) * a.E + e;
    const int cnt = a.chunk_base[last] + a.chunk_cnt[last];
    const int row = a.expert_offset[e] + cnt + item % per;
    if (row >= a.expert_offset[e + 1] || row >= a.capacity)
        return;
    zero_row<NT>(a.recv, a.scales, row, a.H, fp8, a.scale_ld);
}

// Workgroups are handed to the 8 XCDs round-robin (hardware workgroup b runs
// on XCD b % 8).  FP8 rows remap them so that each XCD takes one contiguous
// eighth of the row work: the 32-byte scale pieces that the segments of one
// receive row write then meet in the same L2 and leave it as whole lines.
// Measured at the V3 shape: 94.5-95 us against 97.5-98 us for the plain
// order (large workload: 202 against 211 us).  The tail past the last full
// group of 8 keeps its order.
__device__ __forceinline__ int xcd_contiguous_block(int b, int row_blocks)
{
    const int per = row_blocks / 8;
    if (b >= 8 * per)
        return b;
    return (b % 8) * per + b / 8;
}

template <int KMAX>
__device__ __forceinline__ void row_slots(const DispatchArgs& a, int s_own, int (&sk)[KMAX])
{
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        sk[k] = k < a.K ? readlane(s_own, k) : -1;
}

template <int KMAX, bool FRESH, bool NTS>
__global__ __launch_bounds__(kDispatchWaves * kWave) void dispatch_fp8_kernel(DispatchArgs a)
{
    if ((int)blockIdx.x >= a.row_blocks) {
        pad_item<NTS>(a, true);
        return;
    }
    const int wi = xcd_contiguous_block(blockIdx.x, a.row_blocks) * kDispatchWaves + threadIdx.x / kWave;
    const int t = wi / a.nseg;
    const int seg = wi % a.nseg;
    if (t >= a.T)
        return;
    int sk[KMAX];
    row_slots<KMAX>(a, pair_slot<KMAX, FRESH>(a, t, seg), sk);
    const int i_begin = seg * a.iters_per_seg;
    const int i_end = min(a.iters, i_begin + a.iters_per_seg);
    fp8_rows<KMAX, NTS>(a.x + (size_t)t * a.H, sk, a.H, i_begin, i_end, a.scale_ld,
                   static_cast<uint8_t*>(a.recv), a.scales);
}

template <int KMAX, bool FRESH, bool NTS>
__global__ __launch_bounds__(kDispatchWaves * kWave) void dispatch_fp8in_kernel(DispatchArgs a)
{
    if ((int)blockIdx.x >= a.row_blocks) {
        pad_item<NTS>(a, true);
        return;
    }
    const int wi = xcd_contiguous_block(blockIdx.x, a.row_blocks) * kDispatchWaves + threadIdx.x / kWave;
    const int t = wi / a.nseg;
    const int seg = wi % a.nseg;
    if (t >= a.T)
        return;
    int sk[KMAX];
    row_slots<KMAX>(a, pair_slot<KMAX, FRESH>(a, t, seg), sk);
    const int i_begin = seg * a.iters_per_seg;
    const int i_end = min(a.iters, i_begin + a.iters_per_seg);
    fp8in_rows<KMAX, NTS>(reinterpret_cast<const uint8_t*>(a.x) + (size_t)t * a.H,
                     a.x_scales + (size_t)t * (a.H / kQBlock), sk, a.H, i_begin, i_end, a.scale_ld,
                     static_cast<uint8_t*>(a.recv), a.scales);
}

template <int KMAX, bool FRESH, bool NTS>
__global__ __launch_bounds__(kDispatchWaves * kWave) void dispatch_bf16_kernel(DispatchArgs a)
{
    if ((int)blockIdx.x >= a.row_blocks) {
        pad_item<NTS>(a, false);
        return;
    }
    const int wi = blockIdx.x * kDispatchWaves + threadIdx.x / kWave;
    const int t = wi / a.nseg;
    const int seg = wi % a.nseg;
    if (t >= a.T)
        return;
    int sk[KMAX];
    row_slots<KMAX>(a, pair_slot<KMAX, FRESH>(a, t, seg), sk);
    const int i_begin = seg * a.iters_per_seg;
    const int i_end = min(a.iters, i_begin + a.iters_per_seg);
    bf16_rows<KMAX, NTS>(a.x + (size_t)t * a.H, sk, a.H, i_begin, i_end,
                    static_cast<uint16_t*>(a.recv));
}

constexpr size_t kDispatchFp8CapLds = 32768;     // 5 workgroups per CU

hipError_t launch_dispatch(const DispatchLaunch& L, hipStream_t stream)
{
    if (L.T == 0)
        return hipSuccess;
    DispatchArgs a;
    a.x = static_cast<const uint16_t*>(L.x);
    a.x_scales = L.x_scales;
    a.T = L.T;
    a.H = L.H;
    a.K = L.K;
    a.E = L.E;
    a.B = (int)(((int64_t)L.T + kChunk - 1) / kChunk);
    a.align = L.align;
    a.scale_ld = L.scale_ld;
    a.seq = L.seq;
    a.capacity = L.capacity;
    a.pair_code = L.pair_code;
    a.chunk_base = L.chunk_base;
    a.chunk_cnt = L.chunk_cnt;
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
    a.row_blocks = (int)((items + kDispatchWaves - 1) / kDispatchWaves);
    const long long pad_items = L.align > 1 ? (long long)L.E * (L.align - 1) : 0;
    const long long pad_blocks = (pad_items + kDispatchWaves - 1) / kDispatchWaves;
    dim3 grid((unsigned)(a.row_blocks + pad_blocks));
    dim3 block(kDispatchWaves * kWave);

    // receive buffers that fit the Infinity Cache: plain stores (see the
    // cache hints in dispatch_rows.h)
    const long long recv_bytes =
        (long long)L.capacity * L.H * (L.use_fp8 ? 1 : 2) + (L.use_fp8 ? (long long)L.capacity * (L.H / kQBlock) * 4 : 0);
    const bool nt_store = EP_DISPATCH_NT_STORE && recv_bytes > EP_DISPATCH_CACHED_RECV_BYTES;
    // The quantising FP8 kernel is capped at 5 workgroups (20 waves) per CU by
    // 32 KB of dynamic LDS that it does not touch (160 KB per CU).  At the full
    // 8 workgroups its scattered row writes keep more requests in flight than
    // HBM needs; capped, it was 1-2.5% faster at 8192 and 16384 tokens of 7168
    // channels, warm and after the caches were emptied.  The BF16 copy kernel
    // was slower capped (42.5 -> 47 us cold at 4096 x 4096), so it runs uncapped.
    const size_t lds = (L.use_fp8 && !L.x_scales) ? kDispatchFp8CapLds : 0;
#define EP_DISPATCH(KERNEL, KM, FRESH)                                                  \
    do {                                                                                \
        debug_launch(nt_store ? #KERNEL "<nt>" : #KERNEL, grid, block, lds);            \
        if (nt_store) hipLaunchKernelGGL((KERNEL<KM, FRESH, true>), grid, block, lds, stream, a); \
        else hipLaunchKernelGGL((KERNEL<KM, FRESH, false>), grid, block, lds, stream, a);         \
    } while (0)
#define EP_DISPATCH_K(KERNEL, FRESH)                 \
    do {                                             \
        if (L.K <= 2) EP_DISPATCH(KERNEL, 2, FRESH); \
        else if (L.K <= 4) EP_DISPATCH(KERNEL, 4, FRESH); \
        else if (L.K <= 8) EP_DISPATCH(KERNEL, 8, FRESH); \
        else EP_DISPATCH(KERNEL, 16, FRESH);          \
    } while (0)

    if (L.use_fp8 && L.x_scales) {
        if (L.fresh) EP_DISPATCH_K(dispatch_fp8in_kernel, true);
        else EP_DISPATCH_K(dispatch_fp8in_kernel, false);
    } else if (L.use_fp8) {
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
    debug_launch("e4m3fn_encode_kernel", dim3((unsigned)blocks), dim3(256), 0);
    hipLaunchKernelGGL(e4m3fn_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace moe_ep
