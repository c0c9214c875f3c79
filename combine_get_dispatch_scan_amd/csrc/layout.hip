// get_dispatch_layout on gfx950: per-chunk counting and the chunk-column scan.
//
// The layout step turns topk_idx into the per-destination counts that
// dispatch consumes (stakiran github-trend-summarizer, "DeepEP 要約",
// section 3: get_dispatch_layout precedes dispatch; GeekNews usage section:
// per-expert counts feed the grouped GEMM).  The slot of each (token, k) pair
// is the exclusive prefix of all earlier pairs of the same expert in token
// order.  It is split as
//     slot = expert_offset[e] + chunk_base[c][e] + rank_in_chunk
// where c is the pair's 256-token chunk.  The counting step computes the rank
// and the per-chunk counts with lane bitmaps in LDS (no global atomics, so the
// result does not depend on scheduling); the scan turns the counts into
// chunk_base and expert_offset.
//
// layout_chunk_kernel counts, then the one-workgroup scan_kernel scans; a
// batch of one chunk does both in layout_single_kernel.  Two single-launch
// forms for several chunks were measured slower on MI355X at the V3 shape:
// a cooperative launch with a grid barrier (~22 us plus longer launch gaps),
// and a completion ticket whose last workgroup scans (19.9 us, against 17.7
// for the pair: each workgroup's agent-scope release fence writes its XCD's
// L2 back, which costs more than the launch it saves).
#include "device.h"
#include "launch.h"

namespace moe_ep {

// Counting step of chunk c (256 tokens, one per thread of a 256-thread
// block, one block per chunk).  LDS holds, per wave and expert, a 64-bit mask
// of the wave's tokens that chose the expert, stored wave-major ([wave][E]) so
// that the lanes of one OR, which mostly name different experts, hit
// consecutive words rather than words 32 bytes apart in the same banks.  A
// token's rank for expert e is the number of set bits before it in e's masks.  Writes the pair codes and token-in-partition
// bytes of the chunk's tokens and row c of the per-chunk count tables.
template <int KMAX>
__device__ __forceinline__ void count_chunk(
    const int64_t* __restrict__ topk_idx, int T, int K, int E, int P, int c,
    uint8_t* __restrict__ is_token_in_partition, bool wide_mask_store,
    int32_t* __restrict__ pair_code, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ chunk_pcnt, int32_t* __restrict__ chunk_inv,
    unsigned long long* lds_bits, int* lds_pcnt, int* lds_inv)
{
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int t = c * kChunk + tid;
    const int epp = E / P;

    for (int i = tid; i < E * kChunkWaves; i += kChunk)
        lds_bits[i] = 0ull;
    if (tid < 64)
        lds_pcnt[tid] = 0;
    if (tid == 0)
        *lds_inv = 0;
    __syncthreads();

    int ids[KMAX];
    unsigned long long pmask = 0ull;
    int ninv = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        ids[k] = -1;
        if (k < K && t < T) {
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e >= E) {
                ninv++;
            } else if (e >= 0) {
                bool dup = false;
#pragma unroll
                for (int j = 0; j < k; ++j)
                    dup |= (ids[j] == (int)e);
                if (dup) {
                    ninv++;
                } else {
                    ids[k] = (int)e;
                    atomicOr(&lds_bits[wave * E + (int)e], 1ull << lane);
                    pmask |= 1ull << ((int)e / epp);
                }
            }
        }
    }
    if (ninv)
        atomicAdd(lds_inv, ninv);
    for (unsigned long long m = pmask; m; m &= m - 1)
        atomicAdd(&lds_pcnt[__builtin_ctzll(m)], 1);
    __syncthreads();

    if (t < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k < K) {
                int code = -1;
                int e = ids[k];
                if (e >= 0) {
                    int r = __popcll(lds_bits[wave * E + e] & below);
                    for (int w = 0; w < wave; ++w)
                        r += __popcll(lds_bits[w * E + e]);
                    code = (e << 8) | r;
                }
                pair_code[(size_t)t * K + k] = code;
            }
        }
        uint8_t* dst = is_token_in_partition + (size_t)t * P;
        if (wide_mask_store) {
            for (int p0 = 0; p0 < P; p0 += 8) {
                unsigned long long v = 0ull;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v |= (unsigned long long)((pmask >> (p0 + j)) & 1ull) << (8 * j);
                *reinterpret_cast<unsigned long long*>(dst + p0) = v;
            }
        } else {
            for (int p = 0; p < P; ++p)
                dst[p] = (uint8_t)((pmask >> p) & 1ull);
        }
    }

    for (int e = tid; e < E; e += kChunk) {
        int n = 0;
#pragma unroll
        for (int w = 0; w < kChunkWaves; ++w)
            n += __popcll(lds_bits[w * E + e]);
        chunk_cnt[(size_t)c * E + e] = n;
    }
    if (tid < P)
        chunk_pcnt[(size_t)c * P + tid] = lds_pcnt[tid];
    if (tid == 0)
        chunk_inv[c] = *lds_inv;
}

template <int KMAX>
__global__ __launch_bounds__(kChunk) void layout_chunk_kernel(
    const int64_t* __restrict__ topk_idx, int T, int K, int E, int P,
    uint8_t* __restrict__ is_token_in_partition, bool wide_mask_store,
    int32_t* __restrict__ pair_code, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ chunk_pcnt, int32_t* __restrict__ chunk_inv)
{
    extern __shared__ unsigned long long lds_bits[];     // [kChunkWaves][E]
    __shared__ int lds_pcnt[64];
    __shared__ int lds_inv;
    count_chunk<KMAX>(topk_idx, T, K, E, P, blockIdx.x, is_token_in_partition, wide_mask_store,
                      pair_code, chunk_cnt, chunk_pcnt, chunk_inv, lds_bits, lds_pcnt, &lds_inv);
}

// Inclusive sum over the NT threads of the block; returns the thread's
// inclusive prefix and leaves the block total in *total.
template <int NT>
__device__ int block_inclusive_scan(int v, int* lds_wave, int* total)
{
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(v, d);
        if (lane >= d)
            v += o;
    }
    if (lane == kWave - 1)
        lds_wave[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int s = lane < NW ? lds_wave[lane] : 0;
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            int o = __shfl_up(s, d);
            if (lane >= d)
                s += o;
        }
        if (lane < NW)
            lds_wave[lane] = s;
    }
    __syncthreads();
    int add = wave > 0 ? lds_wave[wave - 1] : 0;
    *total = lds_wave[NW - 1];
    __syncthreads();
    return v + add;
}

constexpr int kScanThreads = 1024;
constexpr int kMaxColumnSegs = 16;

// Column sums of a [B][W] int32 matrix (W <= 1024) with the whole block:
// thread (col, seg) covers a contiguous run of rows, with at most
// kMaxColumnSegs segments per column so the carry-in sum stays short.  When
// `out` is not null it receives each column's exclusive running sum (it may
// be the input itself).  Returns the column total in lds_tot[col].  The
// matrices are in LDS or in global memory (the kernel inlines one copy per
// address space).
template <typename In, typename Out>
__device__ __forceinline__ void column_scan(const In* m, Out* out, int B, int W, int* lds_seg,
                                            int* lds_tot)
{
    const int tid = threadIdx.x;
    const int S = min(kMaxColumnSegs, kScanThreads / W);   // segments per column
    const int col = tid % W;
    const int seg = tid / W;
    const bool active = seg < S;
    const int rows_per = (B + S - 1) / S;
    const int r0 = min(B, seg * rows_per);
    const int r1 = min(B, r0 + rows_per);
    int sum = 0;
    if (active)
        for (int r = r0; r < r1; ++r)
            sum += m[(size_t)r * W + col];
    if (active)
        lds_seg[seg * W + col] = sum;
    __syncthreads();
    if (active) {
        int before = 0;
        for (int s = 0; s < seg; ++s)
            before += lds_seg[s * W + col];
        if (out) {
            int run = before;
            for (int r = r0; r < r1; ++r) {
                int v = m[(size_t)r * W + col];
                out[(size_t)r * W + col] = run;
                run += v;
            }
        }
        if (seg == S - 1)
            lds_tot[col] = before + sum;
    }
    __syncthreads();
}

// A batch of at most 256 tokens is one chunk: its counts are already the
// totals, so the workgroup that counts also scans (each thread owns up to 4
// consecutive experts) and the scan kernel's launch is saved.
template <int KMAX>
__global__ __launch_bounds__(kChunk) void layout_single_kernel(
    const int64_t* __restrict__ topk_idx, int T, int K, int E, int P, int align,
    uint8_t* __restrict__ is_token_in_partition, bool wide_mask_store,
    int32_t* __restrict__ pair_code, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ chunk_pcnt,
    int32_t* __restrict__ chunk_inv, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ num_tokens_per_expert, int32_t* __restrict__ num_tokens_per_partition,
    int32_t* __restrict__ num_invalid, int32_t* __restrict__ status)
{
    extern __shared__ unsigned long long lds_bits[];     // [kChunkWaves][E]
    __shared__ int lds_pcnt[64];
    __shared__ int lds_inv;
    __shared__ int lds_wave[kChunk / kWave];
    count_chunk<KMAX>(topk_idx, T, K, E, P, 0, is_token_in_partition, wide_mask_store,
                      pair_code, chunk_cnt, chunk_pcnt, chunk_inv, lds_bits, lds_pcnt, &lds_inv);
    // the masks and partition / invalid counts in LDS are final here
    const int tid = threadIdx.x;
    const int epT = (E + kChunk - 1) / kChunk;            // <= 4 (E <= 1024)
    int n_e[4], blk_e[4];
    int part = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * epT + j;
        n_e[j] = 0;
        blk_e[j] = 0;
        if (j < epT && e < E) {
#pragma unroll
            for (int w = 0; w < kChunkWaves; ++w)
                n_e[j] += __popcll(lds_bits[w * E + e]);
            blk_e[j] = align == 1 ? n_e[j] : (n_e[j] + align - 1) / align * align;
            part += blk_e[j];
        }
    }
    int total = 0;
    int run = block_inclusive_scan<kChunk>(part, lds_wave, &total) - part;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * epT + j;
        if (j < epT && e < E) {
            expert_offset[e] = run;
            num_tokens_per_expert[e] = n_e[j];
            chunk_base[e] = 0;
            run += blk_e[j];
        }
    }
    if (tid < P)
        num_tokens_per_partition[tid] = lds_pcnt[tid];
    if (tid == 0) {
        expert_offset[E] = total;
        num_invalid[0] = lds_inv;
        status[0] = 0;
        status[1] = lds_inv;
        status[2] = total;
        status[3] = 0;
    }
}

// Largest per-chunk table set (B * (E + P + 1) ints) staged through LDS.
constexpr int kScanLdsInts = 16384;

// One workgroup: chunk counts -> chunk_base, expert totals -> expert_offset;
// partition and invalid totals; status words for dispatch.  When the three
// per-chunk tables fit in LDS they are loaded in one pass of independent
// loads, scanned in LDS and chunk_base is written out; larger tables are
// scanned from global memory.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    int B, int E, int P, int align,
    const int32_t* __restrict__ chunk_cnt, int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ chunk_pcnt, const int32_t* __restrict__ chunk_inv,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ num_tokens_per_expert,
    int32_t* __restrict__ num_tokens_per_partition, int32_t* __restrict__ num_invalid,
    int32_t* __restrict__ status)
{
    extern __shared__ int lds_tab[];              // [B*E | B*P | B] when staged
    __shared__ int lds_seg[kScanThreads];
    __shared__ int lds_tot[kScanThreads];
    __shared__ int lds_wave[kScanThreads / kWave];
    const int tid = threadIdx.x;
    const int nE = B * E, nP = B * P;
    const bool staged = (long long)B * (E + P + 1) <= kScanLdsInts;

    int cnt;
    int ptot = 0, itot = 0;
    if (staged) {
        int* tE = lds_tab;
        int* tP = lds_tab + nE;
        int* tI = tP + nP;
#pragma unroll 4
        for (int i = tid; i < nE; i += kScanThreads)
            tE[i] = chunk_cnt[i];
        for (int i = tid; i < nP; i += kScanThreads)
            tP[i] = chunk_pcnt[i];
        for (int i = tid; i < B; i += kScanThreads)
            tI[i] = chunk_inv[i];
        __syncthreads();
        column_scan(tE, tE, B, E, lds_seg, lds_tot);
        cnt = tid < E ? lds_tot[tid] : 0;
#pragma unroll 4
        for (int i = tid; i < nE; i += kScanThreads)
            chunk_base[i] = tE[i];
        column_scan(tP, (int*)nullptr, B, P, lds_seg, lds_tot);
        ptot = tid < P ? lds_tot[tid] : 0;
        column_scan(tI, (int*)nullptr, B, 1, lds_seg, lds_tot);
        itot = lds_tot[0];
    } else {
        column_scan(chunk_cnt, chunk_base, B, E, lds_seg, lds_tot);
        cnt = tid < E ? lds_tot[tid] : 0;
        column_scan(chunk_pcnt, (int32_t*)nullptr, B, P, lds_seg, lds_tot);
        ptot = tid < P ? lds_tot[tid] : 0;
        column_scan(chunk_inv, (int32_t*)nullptr, B, 1, lds_seg, lds_tot);
        itot = lds_tot[0];
    }

    // an expert's block of receive rows: its count, rounded up to a multiple
    // of align for GEMM-aligned layouts (the rest of the block is padding)
    const int blk = align == 1 ? cnt : (cnt + align - 1) / align * align;
    int total = 0;
    int incl = block_inclusive_scan<kScanThreads>(blk, lds_wave, &total);
    if (tid < E) {
        expert_offset[tid] = incl - blk;
        num_tokens_per_expert[tid] = cnt;
    }
    if (tid < P)
        num_tokens_per_partition[tid] = ptot;
    if (tid == 0) {
        expert_offset[E] = total;
        num_invalid[0] = itot;
        status[0] = 0;
        status[1] = itot;
        status[2] = total;
        status[3] = 0;
    }
}

hipError_t launch_layout(const int64_t* topk_idx, int T, int K, int E, int P, int align,
                         uint8_t* is_token_in_partition, int32_t* pair_code,
                         int32_t* chunk_cnt, int32_t* chunk_base, int32_t* chunk_pcnt,
                         int32_t* chunk_inv, int32_t* expert_offset,
                         int32_t* num_tokens_per_expert, int32_t* num_tokens_per_partition,
                         int32_t* num_invalid, int32_t* status, hipStream_t stream)
{
    const int B = (int)(((int64_t)T + kChunk - 1) / kChunk);
    const size_t lds = (size_t)E * kChunkWaves * sizeof(unsigned long long);
    // 8 partition bytes per 64-bit store when rows start 8-byte aligned
    const bool wide = (P % 8 == 0) && ((reinterpret_cast<uintptr_t>(is_token_in_partition) & 7) == 0);
    if (B == 1) {
        dim3 grid(1), block(kChunk);
#define EP_LAYOUT1(KM)                                                                         \
        hipLaunchKernelGGL(layout_single_kernel<KM>, grid, block, lds, stream, topk_idx, T, K, \
                           E, P, align, is_token_in_partition, wide, pair_code, chunk_cnt,     \
                           chunk_base, chunk_pcnt, chunk_inv, expert_offset,                   \
                           num_tokens_per_expert, num_tokens_per_partition, num_invalid, status)
        debug_launch("layout_single_kernel", grid, block, lds);
        if (K <= 2) EP_LAYOUT1(2);
        else if (K <= 4) EP_LAYOUT1(4);
        else if (K <= 8) EP_LAYOUT1(8);
        else EP_LAYOUT1(16);
#undef EP_LAYOUT1
        return hipGetLastError();
    }
    if (B > 0) {
        dim3 grid(B), block(kChunk);
#define EP_LAYOUT(KM)                                                                   \
        hipLaunchKernelGGL(layout_chunk_kernel<KM>, grid, block, lds, stream, topk_idx, \
                           T, K, E, P, is_token_in_partition, wide, pair_code,          \
                           chunk_cnt, chunk_pcnt, chunk_inv)
        debug_launch("layout_chunk_kernel", grid, block, lds);
        if (K <= 2) EP_LAYOUT(2);
        else if (K <= 4) EP_LAYOUT(4);
        else if (K <= 8) EP_LAYOUT(8);
        else EP_LAYOUT(16);
#undef EP_LAYOUT
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    const bool staged = (long long)B * (E + P + 1) <= kScanLdsInts;
    const size_t scan_lds = staged ? (size_t)B * (E + P + 1) * sizeof(int) : 0;
    debug_launch("scan_kernel", dim3(1), dim3(kScanThreads), scan_lds);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), scan_lds, stream, B, E, P, align,
                       chunk_cnt, chunk_base, chunk_pcnt, chunk_inv, expert_offset,
                       num_tokens_per_expert, num_tokens_per_partition, num_invalid, status);
    return hipGetLastError();
}

}  // namespace moe_ep
