// Expert parallelism over P ranks, one rank's share, on gfx950: the
// destination routing of each token and the metadata of its packed rows.
//
// With partitions as real ranks a token goes once to each rank that hosts one
// of its dispatched experts (devtrends.ru, "Как это выглядит в коде":
// is_token_in_rank, num_tokens_per_rank; stakiran summary section 3:
// dispatch, expert GEMM, combine).  The rest of the flow is the single-rank
// path run on other routing: the sender's pack is dispatch along the
// destination list (one "expert" per rank), the receiver's unpack is layout +
// dispatch along the received local ids, the expert rank's pre-reduction is
// combine with the received weights, and the origin's sum of the returned
// rows in rank order is the unit-weight combine along the pack's slots.
#include "device.h"
#include "launch.h"

namespace moe_ep {

// One thread per token: the ascending distinct partitions of its in-range
// expert ids (masked ids are negative; out-of-range ids are skipped; a
// repeated id names a partition already set), then -1 up to Kp = min(K, P).
__global__ __launch_bounds__(256) void rank_routing_kernel(const int64_t* __restrict__ topk_idx, int T,
                                                           int K, int E, int P,
                                                           int64_t* __restrict__ part_idx)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T)
        return;
    const int epp = E / P;
    const int Kp = min(K, P);
    unsigned long long m = 0ull;
    for (int k = 0; k < K; ++k) {
        const int64_t e = topk_idx[(size_t)t * K + k];
        if (e >= 0 && e < E)
            m |= 1ull << (int)(e / epp);
    }
    int64_t* out = part_idx + (size_t)t * Kp;
    int j = 0;
    for (; m; m &= m - 1)
        out[j++] = __builtin_ctzll(m);
    for (; j < Kp; ++j)
        out[j] = -1;
}

// One thread per (token, destination j): packed row r = slot_pack[t][j]
// carries token t to p = part_idx[t][j]; write its K local expert ids
// (e - p*E/P for dispatched ids in p, else -1) and weights (else 0).  A
// repeated id counts once, at its first position, as the layout counts it.
template <int KMAX>
__global__ __launch_bounds__(256) void pack_metadata_kernel(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights,
    const int64_t* __restrict__ part_idx, const int32_t* __restrict__ slot_pack, int T, int K, int E,
    int P, int64_t* __restrict__ local_idx, float* __restrict__ local_w)
{
    const int Kp = min(K, P);
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * Kp)
        return;
    const int t = i / Kp;
    const int64_t p = part_idx[i];
    const int r = slot_pack[i];
    if (p < 0 || r < 0)
        return;
    const int epp = E / P;
    int64_t ids[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        ids[k] = k < K ? topk_idx[(size_t)t * K + k] : -1;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k < K) {
            const int64_t e = ids[k];
            bool local = e >= 0 && e < E && e / epp == p;
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (j < k)
                    local = local && ids[j] != e;
            local_idx[(size_t)r * K + k] = local ? e - p * epp : -1;
            local_w[(size_t)r * K + k] = local ? topk_weights[(size_t)t * K + k] : 0.0f;
        }
    }
}

hipError_t launch_rank_routing(const int64_t* topk_idx, int T, int K, int E, int P, int64_t* part_idx,
                               hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    dim3 grid((unsigned)(((int64_t)T + 255) / 256)), block(256);
    debug_launch("rank_routing_kernel", grid, block, 0);
    hipLaunchKernelGGL(rank_routing_kernel, grid, block, 0, stream, topk_idx, T, K, E, P, part_idx);
    return hipGetLastError();
}

hipError_t launch_pack_metadata(const int64_t* topk_idx, const float* topk_weights,
                                const int64_t* part_idx, const int32_t* slot_pack, int T, int K,
                                int E, int P, int64_t* local_idx, float* local_w, hipStream_t stream)
{
    const long long n = (long long)T * min(K, P);
    if (n == 0)
        return hipSuccess;
    dim3 grid((unsigned)((n + 255) / 256)), block(256);
    debug_launch("pack_metadata_kernel", grid, block, 0);
#define EP_META(KM) hipLaunchKernelGGL((pack_metadata_kernel<KM>), grid, block, 0, stream, topk_idx, \
                                       topk_weights, part_idx, slot_pack, T, K, E, P, local_idx, local_w)
    if (K <= 2) EP_META(2);
    else if (K <= 4) EP_META(4);
    else if (K <= 8) EP_META(8);
    else EP_META(16);
#undef EP_META
    return hipGetLastError();
}

}  // namespace moe_ep
