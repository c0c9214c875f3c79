// Low-latency dispatch on gfx950: layout, slots and the permute in one launch.
//
// The low-latency mode of the pages serves decode batches with a fixed
// per-expert receive capacity (devtrends.ru, "Как это выглядит в коде":
// low_latency_dispatch(hidden_states, topk_idx, num_max_tokens, num_experts);
// stakiran summary section 3: the decode path, CUDA-graph compatible).  With a
// static layout -- expert e owns rows [e*cap, (e+1)*cap) and a pair's row is
// e*cap + (its rank among expert e's pairs in token order) -- no global offset
// scan is needed, so the whole dispatch is one kernel with no host sync:
//
//  - every workgroup loads the (at most 256) tokens' ids, validates them and
//    ORs each token's lane bit into per-expert LDS masks; a pair's rank is the
//    popcount of the bits below it (deterministic, no global atomics);
//  - workgroup 0 then writes the per-expert / per-partition counts, the
//    status words and the exclusive scan of the received rows per expert (so
//    ep_handle_recv_counts works as for the dense layout), and moves no rows;
//  - the first wave of each token's row writes its slots, weight copy and
//    token-in-partition mask row;
//  - every wave moves one (token, wave step of the row) item with the same row
//    code as dispatch (dispatch_rows.h); its row loads are issued before the
//    routing work, so the two memory latencies overlap.
#include "device.h"
#include "dispatch_rows.h"
#include "launch.h"

namespace moe_ep {

constexpr int kLLWaves = 4;
constexpr int kLLThreads = kLLWaves * kWave;          // 256: one token per thread

struct LLArgs {
    const uint16_t* x;
    const int64_t* topk_idx;
    const float* w_in;
    int T, H, K, E, P, cap;
    int nseg;                                   // wave steps per row (one per item)
    bool wide_mask_store;
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

// Rank of token t among the tokens of expert e (bits below t in e's masks;
// the masks are wave-major, [kLLWaves][E]).
__device__ __forceinline__ int rank_of(const unsigned long long* bits, int E, int e, int t)
{
    const int w = t / kWave;
    int r = __popcll(bits[w * E + e] & ((1ull << (t % kWave)) - 1ull));
    for (int i = 0; i < w; ++i)
        r += __popcll(bits[i * E + e]);
    return r;
}

template <int KMAX, bool FP8>
__global__ __launch_bounds__(kLLThreads) void low_latency_dispatch_kernel(LLArgs a)
{
    extern __shared__ unsigned long long lds_bits[];     // [kLLWaves][E]
    __shared__ int lds_ids[kLLThreads * KMAX];           // valid expert id or -1
    __shared__ unsigned long long lds_pmask[kLLThreads]; // partitions of each token
    __shared__ int lds_pcnt[64];
    __shared__ int lds_inv;
    __shared__ int lds_ovf;
    __shared__ int lds_wave[kLLWaves];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int T = a.T, K = a.K, E = a.E, P = a.P;
    // Workgroup 0 writes the per-expert / per-partition counts and the scan;
    // every other workgroup moves rows, so that bookkeeping and row traffic
    // run side by side.
    const bool leader = blockIdx.x == 0;

    // This wave's row step does not depend on the routing: issue its loads
    // first so that their latency overlaps the routing work below.
    const int item = (blockIdx.x - 1) * kLLWaves + wave;
    const int t_row = leader ? T : item / a.nseg;
    const int seg = leader ? 0 : item % a.nseg;
    const bool has_row = t_row < T;
    const uint16_t* xrow = a.x + (size_t)(has_row ? t_row : 0) * a.H;
    u32x4 lo = u32x4{0u, 0u, 0u, 0u}, hi = u32x4{0u, 0u, 0u, 0u};
    bool act = false;
    int cb = 0;
    if (has_row) {
        if (FP8) {
            act = fp8_step_load(xrow, seg, a.H, lo, hi);
            cb = seg * kFp8ChPerIter + lane * 16;
        } else {
            cb = seg * kBf16ChPerIter + lane * 8;
            act = cb < a.H;
            if (act)
                lo = load16_hint<EP_DISPATCH_NT_LOAD>(xrow + cb);
        }
    }
    // the token's weights, for the first wave of its row (lanes < K)
    float wv = 0.0f;
    const bool first = has_row && seg == 0;
    if (first && lane < K && a.w_in)
        wv = a.w_in[(size_t)t_row * K + lane];

    // this thread's token ids
    const int t = tid;
    int64_t raw[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        raw[k] = (k < K && t < T) ? a.topk_idx[(size_t)t * K + k] : -1;

    for (int i = tid; i < E * kLLWaves; i += kLLThreads)
        lds_bits[i] = 0ull;
    if (tid < 64)
        lds_pcnt[tid] = 0;
    if (tid == 0) {
        lds_inv = 0;
        lds_ovf = 0;
    }
    __syncthreads();
    {
        const int epp = E / P;
        unsigned long long pmask = 0ull;
        int ninv = 0;
        int ids[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            ids[k] = -1;
            const int64_t e = raw[k];
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
            lds_ids[t * KMAX + k] = ids[k];
        }
        lds_pmask[t] = pmask;
        if (leader) {
            if (ninv)
                atomicAdd(&lds_inv, ninv);
            for (unsigned long long m = pmask; m; m &= m - 1)
                atomicAdd(&lds_pcnt[__builtin_ctzll(m)], 1);
        }
    }
    __syncthreads();

    if (leader) {
        // per-expert counts; received rows per expert = min(count, cap),
        // scanned into expert_offset.  Thread i owns experts [i*epT, (i+1)*epT).
        const int epT = (E + kLLThreads - 1) / kLLThreads;     // <= 4 (E <= 1024)
        int n_e[4];
        int part = 0;
        bool ovf = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid * epT + j;
            n_e[j] = 0;
            if (j < epT && e < E) {
#pragma unroll
                for (int w = 0; w < kLLWaves; ++w)
                    n_e[j] += __popcll(lds_bits[w * E + e]);
                a.num_tokens_per_expert[e] = n_e[j];
                part += min(n_e[j], a.cap);
                ovf |= n_e[j] > a.cap;
            }
        }
        // inclusive scan of the partial sums over the 256 threads
        int v = part;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            int o = __shfl_up(v, d);
            if (lane >= d)
                v += o;
        }
        const bool wave_ovf = __any(ovf);
        if (lane == kWave - 1)
            lds_wave[wave] = v;
        if (wave_ovf && lane == 0)
            lds_ovf = 1;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave; ++w)
            before += lds_wave[w];
        int run = before + v - part;
        const int total = lds_wave[0] + lds_wave[1] + lds_wave[2] + lds_wave[3];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid * epT + j;
            if (j < epT && e < E) {
                a.expert_offset[e] = run;
                run += min(n_e[j], a.cap);
            }
        }
        if (tid < P)
            a.num_tokens_per_partition[tid] = lds_pcnt[tid];
        if (tid == 0) {
            a.expert_offset[E] = total;
            a.num_invalid[0] = lds_inv;
            a.status[0] = lds_ovf;
            a.status[1] = lds_inv;
            a.status[2] = total;
            a.status[3] = 0;
        }
        return;
    }

    // row work: this wave's (token, segment) step, loaded above
    if (!has_row)
        return;
    int s_own = -1;
    if (lane < K) {
        const int e = lds_ids[t_row * KMAX + lane];
        if (e >= 0) {
            const int r = rank_of(lds_bits, E, e, t_row);
            if (r < a.cap)
                s_own = e * a.cap + r;
        }
    }
    if (first) {
        // the token's handle entries and mask row
        if (lane < K) {
            const size_t i = (size_t)t_row * K + lane;
            a.slot[i] = s_own;
            if (a.w_in)
                a.w_copy[i] = wv;
        }
        const unsigned long long pm = lds_pmask[t_row];
        uint8_t* dst = a.is_token_in_partition + (size_t)t_row * P;
        if (a.wide_mask_store) {
            const int p0 = lane * 8;
            if (p0 < P) {
                unsigned long long v = 0ull;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v |= (unsigned long long)((pm >> (p0 + j)) & 1ull) << (8 * j);
                *reinterpret_cast<unsigned long long*>(dst + p0) = v;
            }
        } else if (lane < P) {
            dst[lane] = (uint8_t)((pm >> lane) & 1ull);
        }
    }
    int sk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        sk[k] = k < K ? readlane(s_own, k) : -1;
    if (FP8)
        fp8_step_store<KMAX>(lo, hi, cb, act, sk, a.H, 0, static_cast<uint8_t*>(a.recv), a.scales);
    else if (act)
        bf16_step_store<KMAX>(lo, cb, sk, a.H, static_cast<uint16_t*>(a.recv));
}

hipError_t launch_low_latency_dispatch(const LowLatencyLaunch& L, hipStream_t stream)
{
    LLArgs a;
    a.x = static_cast<const uint16_t*>(L.x);
    a.topk_idx = L.topk_idx;
    a.w_in = L.w_in;
    a.T = L.T;
    a.H = L.H;
    a.K = L.K;
    a.E = L.E;
    a.P = L.P;
    a.cap = L.cap;
    a.wide_mask_store = (L.P % 8 == 0) &&
                        ((reinterpret_cast<uintptr_t>(L.is_token_in_partition) & 7) == 0);
    a.recv = L.recv;
    a.scales = L.scales;
    a.slot = L.slot;
    a.w_copy = L.w_copy;
    a.status = L.status;
    a.expert_offset = L.expert_offset;
    a.num_tokens_per_expert = L.num_tokens_per_expert;
    a.num_tokens_per_partition = L.num_tokens_per_partition;
    a.is_token_in_partition = L.is_token_in_partition;
    a.num_invalid = L.num_invalid;
    const int ch = L.use_fp8 ? kFp8ChPerIter : kBf16ChPerIter;
    // one wave step per item: the most waves for a small batch
    a.nseg = (L.H + ch - 1) / ch;
    const long long items = (long long)L.T * a.nseg;
    dim3 grid((unsigned)(1 + (items + kLLWaves - 1) / kLLWaves));     // + the counting workgroup
    dim3 block(kLLThreads);
    const size_t lds = (size_t)L.E * kLLWaves * sizeof(unsigned long long);
#define EP_LL(KM)                                                                                \
    do {                                                                                         \
        debug_launch("low_latency_dispatch_kernel", grid, block, lds);                            \
        if (L.use_fp8) hipLaunchKernelGGL((low_latency_dispatch_kernel<KM, true>), grid, block, lds, stream, a); \
        else hipLaunchKernelGGL((low_latency_dispatch_kernel<KM, false>), grid, block, lds, stream, a);         \
    } while (0)
    if (L.K <= 2) EP_LL(2);
    else if (L.K <= 4) EP_LL(4);
    else if (L.K <= 8) EP_LL(8);
    else EP_LL(16);
#undef EP_LL
    return hipGetLastError();
}

}  // namespace moe_ep
