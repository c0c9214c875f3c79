// The moe_ep C ABI: argument validation, workspace carving, handle upkeep and
// kernel launches.  Nothing here allocates device memory or synchronises,
// except ep_handle_recv_counts (a small device-to-host copy).
#include "moe_ep.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(EP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kChunk = 256;
constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
    size_t chunk_cnt, chunk_base, chunk_pcnt, chunk_inv, pair_code, expert_offset, slot,
        src_token, weights, status, total;
};

bool dims_ok(int T, int K, int E, int P)
{
    return T >= 0 && K >= 1 && K <= EP_MAX_TOPK && E >= 1 && E <= EP_MAX_EXPERTS && P >= 1 &&
           P <= EP_MAX_PARTITIONS && E % P == 0 && (int64_t)T * K < (int64_t)1 << 31;
}

int check_dims(int T, int K, int E, int P)
{
    if (dims_ok(T, K, E, P))
        return EP_OK;
    return fail(EP_EINVAL,
                "invalid dims T=%d K=%d E=%d P=%d (need T>=0, 1<=K<=%d, 1<=E<=%d, "
                "1<=P<=%d, E%%P==0, T*K<2^31)",
                T, K, E, P, EP_MAX_TOPK, EP_MAX_EXPERTS, EP_MAX_PARTITIONS);
}

WsLayout ws_layout(int T, int K, int E, int P)
{
    const size_t B = ((size_t)T + kChunk - 1) / kChunk;
    const size_t TK = (size_t)T * K;
    WsLayout L;
    size_t o = 0;
    L.chunk_cnt = o;     o += up(B * E * 4);
    L.chunk_base = o;    o += up(B * E * 4);
    L.chunk_pcnt = o;    o += up(B * P * 4);
    L.chunk_inv = o;     o += up(B * 4);
    L.pair_code = o;     o += up(TK * 4);
    // expert_offset [E+1] and status [4] are adjacent: one copy reads both
    L.expert_offset = o; o += up(((size_t)E + 1 + 4) * 4);
    L.slot = o;          o += up(TK * 4);
    L.src_token = o;     o += up(TK * 4);
    L.weights = o;       o += up(TK * 4);
    L.status = L.expert_offset + ((size_t)E + 1) * 4;
    L.total = o;
    return L;
}

int check_handle(const ep_handle_t* h, int min_stage)
{
    if (!h)
        return fail(EP_EINVAL, "handle is NULL");
    if (h->magic != EP_HANDLE_MAGIC)
        return fail(EP_EINVAL, "handle was not filled by ep_get_dispatch_layout");
    if (h->stage < min_stage)
        return fail(EP_EINVAL, "handle has not been dispatched yet (call ep_dispatch first)");
    // the layout calls fill a handle only after checking its dimensions, so
    // out-of-range ones mean a corrupted handle, whose sizes must not be used
    if (!dims_ok(h->num_tokens, h->num_topk, h->num_experts, h->num_partitions))
        return fail(EP_EINVAL, "handle dimensions out of range (T=%d K=%d E=%d P=%d): not a handle "
                    "filled by the layout call", h->num_tokens, h->num_topk, h->num_experts,
                    h->num_partitions);
    return EP_OK;
}

}  // namespace

namespace moe_ep {

void debug_launch(const char* kernel, dim3 grid, dim3 block, size_t lds)
{
    static const bool on = [] {
        const char* v = getenv("EP_DEBUG");
        return v && v[0] && v[0] != '0';
    }();
    if (on)
        fprintf(stderr, "[moe_ep] %s grid=(%u,%u,%u) block=(%u,%u,%u) lds=%zu\n", kernel, grid.x, grid.y,
                grid.z, block.x, block.y, block.z, lds);
}

}  // namespace moe_ep

extern "C" {

int ep_version(void) { return EP_VERSION; }

const char* ep_last_error(void) { return g_err.c_str(); }

size_t ep_workspace_bytes(int num_tokens, int num_topk, int num_experts, int num_partitions)
{
    if (!dims_ok(num_tokens, num_topk, num_experts, num_partitions))
        return 0;
    return ws_layout(num_tokens, num_topk, num_experts, num_partitions).total;
}

int ep_get_dispatch_layout(const int64_t* topk_idx, int T, int K, int E, int P,
                           int32_t* num_tokens_per_partition, int32_t* num_tokens_per_expert,
                           uint8_t* is_token_in_partition, int32_t* num_invalid,
                           void* ws, size_t ws_bytes, ep_handle_t* handle,
                           hipStream_t stream)
{
    return ep_get_dispatch_layout_aligned(topk_idx, T, K, E, P, 1, num_tokens_per_partition,
                                          num_tokens_per_expert, is_token_in_partition,
                                          num_invalid, ws, ws_bytes, handle, stream);
}

int ep_get_dispatch_layout_aligned(const int64_t* topk_idx, int T, int K, int E, int P,
                                   int expert_alignment, int32_t* num_tokens_per_partition,
                                   int32_t* num_tokens_per_expert,
                                   uint8_t* is_token_in_partition, int32_t* num_invalid,
                                   void* ws, size_t ws_bytes, ep_handle_t* handle,
                                   hipStream_t stream)
{
    g_err.clear();
    int rc = check_dims(T, K, E, P);
    if (rc)
        return rc;
    const int A = expert_alignment;
    if (A < 1 || A > EP_MAX_ALIGNMENT)
        return fail(EP_EINVAL, "expert_alignment=%d must be in [1, %d]", A, EP_MAX_ALIGNMENT);
    if ((int64_t)T * K + (int64_t)E * (A - 1) >= ((int64_t)1 << 31))
        return fail(EP_EINVAL, "T*K + E*(expert_alignment-1) must be < 2^31");
    if (!handle)
        return fail(EP_EINVAL, "handle is NULL");
    if (T > 0 && (!topk_idx || !aligned(topk_idx, 8)))
        return fail(EP_EINVAL, "topk_idx must be a non-NULL 8-byte aligned device pointer");
    if (T > 0 && !is_token_in_partition)
        return fail(EP_EINVAL, "is_token_in_partition is NULL");
    if (!num_tokens_per_partition || !num_tokens_per_expert || !num_invalid ||
        !aligned(num_tokens_per_partition, 4) || !aligned(num_tokens_per_expert, 4) ||
        !aligned(num_invalid, 4))
        return fail(EP_EINVAL, "count outputs must be non-NULL 4-byte aligned device pointers");
    const WsLayout L = ws_layout(T, K, E, P);
    if (!ws || !aligned(ws, kAlign))
        return fail(EP_EINVAL, "workspace must be a non-NULL 256-byte aligned device pointer");
    if (ws_bytes < L.total)
        return fail(EP_EINVAL, "workspace too small: %zu bytes given, %zu needed", ws_bytes, L.total);

    char* w = static_cast<char*>(ws);
    ep_handle_t h;
    memset(&h, 0, sizeof h);
    h.magic = EP_HANDLE_MAGIC;
    h.stage = 1;
    h.num_tokens = T;
    h.num_topk = K;
    h.num_experts = E;
    h.num_partitions = P;
    h.num_chunks = (int)(((int64_t)T + kChunk - 1) / kChunk);
    h.ws = ws;
    h.ws_bytes = ws_bytes;
    h.expert_offset = reinterpret_cast<int32_t*>(w + L.expert_offset);
    h.slot = reinterpret_cast<int32_t*>(w + L.slot);
    // the source-token table has T*K rows: kept for dense layouts only
    h.src_token = A == 1 ? reinterpret_cast<int32_t*>(w + L.src_token) : nullptr;
    h.weights = reinterpret_cast<float*>(w + L.weights);
    h.status = reinterpret_cast<int32_t*>(w + L.status);
    h.pair_code = reinterpret_cast<int32_t*>(w + L.pair_code);
    h.chunk_cnt = reinterpret_cast<int32_t*>(w + L.chunk_cnt);
    h.chunk_base = reinterpret_cast<int32_t*>(w + L.chunk_base);
    h.chunk_pcnt = reinterpret_cast<int32_t*>(w + L.chunk_pcnt);
    h.chunk_inv = reinterpret_cast<int32_t*>(w + L.chunk_inv);
    h.expert_alignment = A;

    hipError_t e = moe_ep::launch_layout(topk_idx, T, K, E, P, A, is_token_in_partition,
                                         h.pair_code, h.chunk_cnt, h.chunk_base, h.chunk_pcnt,
                                         h.chunk_inv, h.expert_offset, num_tokens_per_expert,
                                         num_tokens_per_partition, num_invalid, h.status, stream);
    if (e != hipSuccess)
        return hip_fail(e, "layout launch");
    *handle = h;
    return EP_OK;
}

// Largest receive buffer a handle can need: T*K rows, plus E*(A-1) padding
// rows for an aligned layout, or E*cap rows for a static one.
static int64_t max_rows(const ep_handle_t* h)
{
    if (h->static_cap)
        return (int64_t)h->num_experts * h->static_cap;
    const int A = h->expert_alignment > 1 ? h->expert_alignment : 1;
    return (int64_t)h->num_tokens * h->num_topk + (int64_t)h->num_experts * (A - 1);
}

static int check_rows(const ep_handle_t* h, const void* x, int H, int use_fp8, const void* recv_x,
                      const float* recv_scales, int capacity)
{
    const int T = h->num_tokens;
    if (H < 1 || H > EP_MAX_HIDDEN || H % 8 != 0)
        return fail(EP_EINVAL, "hidden=%d must be in [1, %d] and a multiple of 8", H, EP_MAX_HIDDEN);
    if (use_fp8 != 0 && use_fp8 != 1)
        return fail(EP_EINVAL, "use_fp8 must be 0 or 1");
    if (use_fp8 && H % 128 != 0)
        return fail(EP_EINVAL, "FP8 dispatch needs hidden %% 128 == 0 (hidden=%d)", H);
    const int64_t mr = max_rows(h);
    if (capacity < 0 || (int64_t)capacity > mr)
        return fail(EP_EINVAL, "capacity_rows=%d must be in [0, %lld]", capacity, (long long)mr);
    if (T > 0 && (!x || !aligned(x, 16)))
        return fail(EP_EINVAL, "x must be a non-NULL 16-byte aligned device pointer");
    if (capacity > 0 && (!recv_x || !aligned(recv_x, 16)))
        return fail(EP_EINVAL, "recv_x must be a non-NULL 16-byte aligned device pointer");
    if (use_fp8 && capacity > 0 && (!recv_scales || !aligned(recv_scales, 4)))
        return fail(EP_EINVAL, "recv_scales must be a non-NULL 4-byte aligned device pointer");
    return EP_OK;
}

// Options of ep_dispatch_ex: pre-quantised input and the scale layout.
static int check_options(const ep_handle_t* h, const float* x_scales, int use_fp8, int scale_ld,
                         int capacity)
{
    if (x_scales && !use_fp8)
        return fail(EP_EINVAL, "x_scales (pre-quantised FP8 input) needs use_fp8 = 1");
    if (x_scales && h->num_tokens > 0 && !aligned(x_scales, 4))
        return fail(EP_EINVAL, "x_scales must be a 4-byte aligned device pointer");
    if (scale_ld != 0) {
        if (!use_fp8)
            return fail(EP_EINVAL, "scale_ld (column-major scales) needs use_fp8 = 1");
        if (scale_ld < capacity || scale_ld % 4 != 0)
            return fail(EP_EINVAL, "scale_ld=%d must be 0, or >= capacity_rows=%d and a multiple of 4",
                        scale_ld, capacity);
    }
    return EP_OK;
}

static int run_dispatch(const ep_handle_t* h, const void* x, const float* w_in, void* recv_x,
                        float* recv_scales, bool fresh, hipStream_t stream,
                        const float* x_scales = nullptr)
{
    moe_ep::DispatchLaunch L;
    L.x = x;
    L.x_scales = x_scales;
    L.align = h->expert_alignment > 1 ? h->expert_alignment : 1;
    L.scale_ld = h->scale_ld;
    L.chunk_cnt = h->chunk_cnt;
    L.T = h->num_tokens;
    L.H = h->hidden;
    L.K = h->num_topk;
    L.E = h->num_experts;
    L.use_fp8 = h->use_fp8;
    L.fresh = fresh;
    L.seq = h->dispatch_seq;
    L.capacity = h->capacity_rows;
    L.pair_code = h->pair_code;
    L.chunk_base = h->chunk_base;
    L.expert_offset = h->expert_offset;
    L.w_in = w_in;
    L.w_copy = h->weights;
    L.slot = h->slot;
    L.src_token = h->src_token;
    L.status = h->status;
    L.recv = recv_x;
    L.scales = recv_scales;
    hipError_t e = moe_ep::launch_dispatch(L, stream);
    if (e != hipSuccess)
        return hip_fail(e, "dispatch launch");
    return EP_OK;
}

int ep_dispatch(const void* x, const float* topk_weights, int hidden, int use_fp8,
                void* recv_x, float* recv_scales, int capacity_rows,
                ep_handle_t* handle, hipStream_t stream)
{
    return ep_dispatch_ex(x, nullptr, topk_weights, hidden, use_fp8, 0, recv_x, recv_scales,
                          capacity_rows, handle, stream);
}

int ep_dispatch_ex(const void* x, const float* x_scales, const float* topk_weights, int hidden,
                   int use_fp8, int scale_ld, void* recv_x, float* recv_scales, int capacity_rows,
                   ep_handle_t* handle, hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 1);
    if (rc)
        return rc;
    if (handle->static_cap)
        return fail(EP_EINVAL, "handle holds a low-latency (static) layout: use ep_dispatch_cached");
    rc = check_rows(handle, x, hidden, use_fp8, recv_x, recv_scales, capacity_rows);
    if (rc)
        return rc;
    rc = check_options(handle, x_scales, use_fp8, scale_ld, capacity_rows);
    if (rc)
        return rc;
    if (topk_weights && !aligned(topk_weights, 4))
        return fail(EP_EINVAL, "topk_weights must be 4-byte aligned");
    ep_handle_t h = *handle;
    h.hidden = hidden;
    h.use_fp8 = use_fp8;
    h.capacity_rows = capacity_rows;
    h.has_weights = topk_weights != nullptr;
    h.scale_ld = scale_ld;
    h.fp8_input = x_scales != nullptr;
    // this dispatch's number: its kernel writes it into the overflow word, so
    // a mark left by an earlier dispatch of the same handle is not read as
    // this one's (no clearing store is needed, the path stays capturable)
    h.dispatch_seq = handle->stage >= 2 && handle->dispatch_seq > 0 &&
                             handle->dispatch_seq < 0x7FFFFFFF
                         ? handle->dispatch_seq + 1
                         : 1;
    rc = run_dispatch(&h, x, topk_weights, recv_x, recv_scales, true, stream, x_scales);
    if (rc)
        return rc;
    h.stage = 2;
    *handle = h;
    return EP_OK;
}

// Arguments of the low-latency dispatch other than the workspace; no HIP call.
static int ll_check(const void* x, const int64_t* topk_idx, const float* topk_weights, int T, int H,
                    int K, int E, int P, int use_fp8, int cap, const void* recv_x,
                    const float* recv_scales, const int32_t* num_tokens_per_partition,
                    const int32_t* num_tokens_per_expert, const uint8_t* is_token_in_partition,
                    const int32_t* num_invalid, const ep_handle_t* handle)
{
    int rc = check_dims(T, K, E, P);
    if (rc)
        return rc;
    if (!handle)
        return fail(EP_EINVAL, "handle is NULL");
    if (T > EP_MAX_LL_TOKENS)
        return fail(EP_EINVAL, "low-latency dispatch takes at most %d tokens (got %d)",
                    EP_MAX_LL_TOKENS, T);
    if (cap < 1 || (int64_t)E * cap >= (int64_t)1 << 31)
        return fail(EP_EINVAL, "num_max_tokens=%d must be >= 1 with E*num_max_tokens < 2^31", cap);
    if (T > 0 && (!topk_idx || !aligned(topk_idx, 8)))
        return fail(EP_EINVAL, "topk_idx must be a non-NULL 8-byte aligned device pointer");
    if (T > 0 && !is_token_in_partition)
        return fail(EP_EINVAL, "is_token_in_partition is NULL");
    if (!num_tokens_per_partition || !num_tokens_per_expert || !num_invalid ||
        !aligned(num_tokens_per_partition, 4) || !aligned(num_tokens_per_expert, 4) ||
        !aligned(num_invalid, 4))
        return fail(EP_EINVAL, "count outputs must be non-NULL 4-byte aligned device pointers");
    if (topk_weights && !aligned(topk_weights, 4))
        return fail(EP_EINVAL, "topk_weights must be 4-byte aligned");
    ep_handle_t probe;               // the dimensions check_rows reads
    memset(&probe, 0, sizeof probe);
    probe.num_tokens = T;
    probe.num_topk = K;
    probe.num_experts = E;
    probe.static_cap = cap;
    rc = check_rows(&probe, x, H, use_fp8, recv_x, recv_scales, 0);
    if (rc)
        return rc;
    if (T > 0 && (!recv_x || !aligned(recv_x, 16)))
        return fail(EP_EINVAL, "recv_x must be a non-NULL 16-byte aligned device pointer");
    if (T > 0 && use_fp8 && (!recv_scales || !aligned(recv_scales, 4)))
        return fail(EP_EINVAL, "recv_scales must be a non-NULL 4-byte aligned device pointer");
    return EP_OK;
}

// The low-latency dispatch on checked arguments, with its handle arrays in
// the workspace `ws`.
static int ll_run(const void* x, const int64_t* topk_idx, const float* topk_weights, int T, int H,
                  int K, int E, int P, int use_fp8, int cap, void* recv_x, float* recv_scales,
                  int32_t* num_tokens_per_partition, int32_t* num_tokens_per_expert,
                  uint8_t* is_token_in_partition, int32_t* num_invalid, void* ws, size_t ws_bytes,
                  ep_handle_t* handle, hipStream_t stream)
{
    const WsLayout L = ws_layout(T, K, E, P);
    char* w = static_cast<char*>(ws);
    ep_handle_t h;
    memset(&h, 0, sizeof h);
    h.magic = EP_HANDLE_MAGIC;
    h.stage = 1;
    h.num_tokens = T;
    h.num_topk = K;
    h.num_experts = E;
    h.num_partitions = P;
    h.num_chunks = (int)(((int64_t)T + kChunk - 1) / kChunk);
    h.ws = ws;
    h.ws_bytes = ws_bytes;
    h.expert_offset = reinterpret_cast<int32_t*>(w + L.expert_offset);
    h.slot = reinterpret_cast<int32_t*>(w + L.slot);
    h.src_token = nullptr;      // static layout: rows are found from slot alone
    h.static_cap = cap;
    h.weights = reinterpret_cast<float*>(w + L.weights);
    h.status = reinterpret_cast<int32_t*>(w + L.status);

    moe_ep::LowLatencyLaunch LL;
    LL.x = x;
    LL.topk_idx = topk_idx;
    LL.w_in = topk_weights;
    LL.T = T;
    LL.H = H;
    LL.K = K;
    LL.E = E;
    LL.P = P;
    LL.cap = cap;
    LL.use_fp8 = use_fp8;
    LL.recv = recv_x;
    LL.scales = recv_scales;
    LL.slot = h.slot;
    LL.w_copy = h.weights;
    LL.status = h.status;
    LL.expert_offset = h.expert_offset;
    LL.num_tokens_per_expert = num_tokens_per_expert;
    LL.num_tokens_per_partition = num_tokens_per_partition;
    LL.is_token_in_partition = is_token_in_partition;
    LL.num_invalid = num_invalid;
    hipError_t e = moe_ep::launch_low_latency_dispatch(LL, stream);
    if (e != hipSuccess)
        return hip_fail(e, "low-latency dispatch launch");
    h.stage = 2;
    h.hidden = H;
    h.use_fp8 = use_fp8;
    h.capacity_rows = E * cap;
    h.has_weights = topk_weights != nullptr;
    h.dispatch_seq = 1;         // the kernel writes 1 or 0 into the overflow word
    *handle = h;
    return EP_OK;
}

int ep_low_latency_dispatch(const void* x, const int64_t* topk_idx, const float* topk_weights,
                            int T, int H, int K, int E, int P, int use_fp8, int cap,
                            void* recv_x, float* recv_scales,
                            int32_t* num_tokens_per_partition, int32_t* num_tokens_per_expert,
                            uint8_t* is_token_in_partition, int32_t* num_invalid,
                            void* ws, size_t ws_bytes, ep_handle_t* handle, hipStream_t stream)
{
    g_err.clear();
    int rc = ll_check(x, topk_idx, topk_weights, T, H, K, E, P, use_fp8, cap, recv_x, recv_scales,
                      num_tokens_per_partition, num_tokens_per_expert, is_token_in_partition,
                      num_invalid, handle);
    if (rc)
        return rc;
    const WsLayout L = ws_layout(T, K, E, P);
    if (!ws || !aligned(ws, kAlign))
        return fail(EP_EINVAL, "workspace must be a non-NULL 256-byte aligned device pointer");
    if (ws_bytes < L.total)
        return fail(EP_EINVAL, "workspace too small: %zu bytes given, %zu needed", ws_bytes, L.total);
    return ll_run(x, topk_idx, topk_weights, T, H, K, E, P, use_fp8, cap, recv_x, recv_scales,
                  num_tokens_per_partition, num_tokens_per_expert, is_token_in_partition,
                  num_invalid, ws, ws_bytes, handle, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The allocation-free low-latency dispatch keeps its handle arrays in one
// device array per GPU (`scratch`), instead of a caller workspace.  Host code
// never passes `scratch` itself to a kernel or a copy -- on the host that name
// is only a stand-in -- but the device address hipGetSymbolAddress returns,
// looked up once per device with that device current.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = EP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's `scratch` (looked up on the first
// call per device).  A stream of another device is refused: the array the
// kernel would reach is the current device's.  Returns EP_OK and sets *ptr,
// or an error code.
int scratch_address(hipStream_t stream, void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamGetDevice");
        if (sdev != dev)
            return fail(EP_EINVAL, "the stream belongs to device %d but device %d is current: make the "
                        "stream's device current first", (int)sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(EP_EINVAL, "device %d is beyond the %d devices the scratch table covers", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, kAlign))
            return fail(EP_EHIP, "scratch array has no 256-byte aligned device address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_low_latency_dispatch_noalloc(const void* x, const int64_t* topk_idx,
                                    const float* topk_weights, int T, int H, int K, int E, int P,
                                    int use_fp8, int cap, void* recv_x, float* recv_scales,
                                    int32_t* num_tokens_per_partition,
                                    int32_t* num_tokens_per_expert,
                                    uint8_t* is_token_in_partition, int32_t* num_invalid,
                                    ep_handle_t* handle, hipStream_t stream)
{
    g_err.clear();
    int rc = ll_check(x, topk_idx, topk_weights, T, H, K, E, P, use_fp8, cap, recv_x, recv_scales,
                      num_tokens_per_partition, num_tokens_per_expert, is_token_in_partition,
                      num_invalid, handle);
    if (rc)
        return rc;
    const size_t need = ws_layout(T, K, E, P).total;
    if (need > kScratchBytes)
        return fail(EP_EINVAL, "T=%d K=%d E=%d P=%d need %zu bytes of scratch; the allocation-free "
                    "dispatch holds %zu (use ep_low_latency_dispatch with a workspace)",
                    T, K, E, P, need, kScratchBytes);
    void* ptr = nullptr;
    rc = scratch_address(stream, &ptr);
    if (rc)
        return rc;
    // every array the kernel leaves in the scratch (slots, weight copy,
    // offsets, status) is written whole by the launch: nothing must start at 0
    return ll_run(x, topk_idx, topk_weights, T, H, K, E, P, use_fp8, cap, recv_x, recv_scales,
                  num_tokens_per_partition, num_tokens_per_expert, is_token_in_partition,
                  num_invalid, ptr, kScratchBytes, handle, stream);
}

int ep_dispatch_cached(const void* x, const ep_handle_t* handle, void* recv_x, float* recv_scales,
                       hipStream_t stream)
{
    return ep_dispatch_cached_ex(x, nullptr, handle, recv_x, recv_scales, stream);
}

int ep_dispatch_cached_ex(const void* x, const float* x_scales, const ep_handle_t* handle,
                          void* recv_x, float* recv_scales, hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 2);
    if (rc)
        return rc;
    rc = check_rows(handle, x, handle->hidden, handle->use_fp8, recv_x, recv_scales,
                    handle->capacity_rows);
    if (rc)
        return rc;
    if (handle->fp8_input && !x_scales && handle->num_tokens > 0)
        return fail(EP_EINVAL, "the handle was dispatched from FP8 input: pass x_scales");
    if (!handle->fp8_input && x_scales)
        return fail(EP_EINVAL, "the handle was dispatched from BF16 input: x_scales must be NULL");
    rc = check_options(handle, x_scales, handle->use_fp8, handle->scale_ld, handle->capacity_rows);
    if (rc)
        return rc;
    return run_dispatch(handle, x, nullptr, recv_x, recv_scales, false, stream, x_scales);
}

int ep_combine(const void* y, const ep_handle_t* handle, const float* topk_weights, void* out,
               hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 2);
    if (rc)
        return rc;
    const int T = handle->num_tokens;
    const float* w = topk_weights ? topk_weights : (handle->has_weights ? handle->weights : nullptr);
    if (!w && T > 0)
        return fail(EP_EINVAL, "no weights: pass topk_weights or give them to ep_dispatch");
    if (w && !aligned(w, 4))
        return fail(EP_EINVAL, "topk_weights must be 4-byte aligned");
    if (T > 0 && (!out || !aligned(out, 16)))
        return fail(EP_EINVAL, "out must be a non-NULL 16-byte aligned device pointer");
    if (T > 0 && handle->capacity_rows > 0 && (!y || !aligned(y, 16)))
        return fail(EP_EINVAL, "y must be a non-NULL 16-byte aligned device pointer (a receive-row buffer, "
                    "also when no pair was dispatched)");
    hipError_t e = moe_ep::launch_combine(y, T, handle->hidden, handle->num_topk, handle->slot, w,
                                          out, stream);
    if (e != hipSuccess)
        return hip_fail(e, "combine launch");
    return EP_OK;
}

int ep_dispatch_backward(const void* grad_recv, const ep_handle_t* handle, void* grad_x,
                         hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 2);
    if (rc)
        return rc;
    const int T = handle->num_tokens;
    if (T > 0 && (!grad_x || !aligned(grad_x, 16)))
        return fail(EP_EINVAL, "grad_x must be a non-NULL 16-byte aligned device pointer");
    if (T > 0 && handle->capacity_rows > 0 && (!grad_recv || !aligned(grad_recv, 16)))
        return fail(EP_EINVAL, "grad_recv must be a non-NULL 16-byte aligned device pointer (a receive-row "
                    "buffer, also when no pair was dispatched)");
    hipError_t e = moe_ep::launch_combine(grad_recv, T, handle->hidden, handle->num_topk,
                                          handle->slot, nullptr, grad_x, stream);
    if (e != hipSuccess)
        return hip_fail(e, "dispatch backward launch");
    return EP_OK;
}

static int run_combine_fp8(const void* y, const float* y_scales, const ep_handle_t* handle,
                           const float* w, void* out, const char* what, hipStream_t stream)
{
    const int T = handle->num_tokens;
    const int H = handle->hidden;
    if (H % 128 != 0)
        return fail(EP_EINVAL, "FP8 rows need hidden %% 128 == 0 (hidden=%d)", H);
    if (T > 0 && (!out || !aligned(out, 16)))
        return fail(EP_EINVAL, "%s must be a non-NULL 16-byte aligned device pointer",
                    w ? "out" : "grad_x");
    if (T > 0 && handle->capacity_rows > 0 && (!y || !aligned(y, 16)))
        return fail(EP_EINVAL, "the FP8 rows must be a non-NULL 16-byte aligned device pointer");
    if (T > 0 && handle->capacity_rows > 0 && (!y_scales || !aligned(y_scales, 4)))
        return fail(EP_EINVAL, "the FP8 scales must be a non-NULL 4-byte aligned device pointer");
    hipError_t e = moe_ep::launch_combine_fp8(y, y_scales, handle->scale_ld, T, H, handle->num_topk,
                                              handle->slot, w, out, stream);
    if (e != hipSuccess)
        return hip_fail(e, what);
    return EP_OK;
}

int ep_combine_fp8(const void* y, const float* y_scales, const ep_handle_t* handle,
                   const float* topk_weights, void* out, hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 2);
    if (rc)
        return rc;
    const int T = handle->num_tokens;
    const float* w = topk_weights ? topk_weights : (handle->has_weights ? handle->weights : nullptr);
    if (!w && T > 0)
        return fail(EP_EINVAL, "no weights: pass topk_weights or give them to ep_dispatch");
    if (w && !aligned(w, 4))
        return fail(EP_EINVAL, "topk_weights must be 4-byte aligned");
    if (!w)                       // T == 0: nothing is launched; any non-null marks "weighted"
        w = handle->weights;
    return run_combine_fp8(y, y_scales, handle, w, out, "FP8 combine launch", stream);
}

int ep_dispatch_backward_fp8(const void* grad_recv, const float* grad_scales,
                             const ep_handle_t* handle, void* grad_x, hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 2);
    if (rc)
        return rc;
    return run_combine_fp8(grad_recv, grad_scales, handle, nullptr, grad_x,
                           "FP8 dispatch backward launch", stream);
}

int ep_combine_backward(const void* grad_out, const void* y, const ep_handle_t* handle,
                        const float* topk_weights, void* grad_y, float* grad_w,
                        hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 2);
    if (rc)
        return rc;
    const int T = handle->num_tokens;
    const float* w = topk_weights ? topk_weights : (handle->has_weights ? handle->weights : nullptr);
    if (!w && T > 0)
        return fail(EP_EINVAL, "no weights: pass topk_weights or give them to ep_dispatch");
    if (w && !aligned(w, 4))
        return fail(EP_EINVAL, "topk_weights must be 4-byte aligned");
    if (T > 0 && (!grad_out || !aligned(grad_out, 16)))
        return fail(EP_EINVAL, "grad_out must be a non-NULL 16-byte aligned device pointer");
    const bool rows = T > 0 && handle->capacity_rows > 0;
    if (rows && (!grad_y || !aligned(grad_y, 16)))
        return fail(EP_EINVAL, "grad_y must be a non-NULL 16-byte aligned device pointer");
    if (grad_w && !aligned(grad_w, 4))
        return fail(EP_EINVAL, "grad_w must be 4-byte aligned");
    if (grad_w && rows && (!y || !aligned(y, 16)))
        return fail(EP_EINVAL, "grad_w needs y: a non-NULL 16-byte aligned device pointer");
    hipError_t e = moe_ep::launch_combine_backward(grad_out, y, T, handle->hidden,
                                                   handle->num_topk, handle->slot, w, grad_y,
                                                   grad_w, stream);
    if (e != hipSuccess)
        return hip_fail(e, "combine backward launch");
    return EP_OK;
}

int ep_handle_recv_counts_async(const ep_handle_t* handle, int32_t* host_buf, hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(handle, 1);
    if (rc)
        return rc;
    if (!host_buf)
        return fail(EP_EINVAL, "host_buf is NULL");
    // expert_offset [E+1] is followed by the 4 status words in the workspace
    hipError_t e = hipMemcpyAsync(host_buf, handle->expert_offset,
                                  sizeof(int32_t) * (handle->num_experts + 1 + 4),
                                  hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess)
        return hip_fail(e, "reading counts");
    return EP_OK;
}

int ep_recv_counts_decode(const ep_handle_t* handle, const int32_t* host_buf,
                          int32_t* host_counts, int32_t* host_num_recv)
{
    g_err.clear();
    int rc = check_handle(handle, 1);
    if (rc)
        return rc;
    if (!host_buf)
        return fail(EP_EINVAL, "host_buf is NULL");
    const int E = handle->num_experts;
    const int32_t* off = host_buf;
    const int32_t* st = host_buf + E + 1;
    // offsets written by the scan are non-decreasing; the difference is taken
    // modulo 2^32 so that any buffer content decodes without overflow
    if (host_counts)
        for (int i = 0; i < E; ++i)
            host_counts[i] = (int32_t)((uint32_t)off[i + 1] - (uint32_t)off[i]);
    if (host_num_recv)
        *host_num_recv = off[E];
    // the overflow word counts only when it holds this handle's latest
    // dispatch number; a dense layout drops pairs exactly when N exceeds the
    // capacity, which also covers a copy taken before dispatch marked it
    const bool dense = !handle->static_cap && handle->expert_alignment <= 1;
    const bool marked = st[0] != 0 && st[0] == handle->dispatch_seq;
    if (handle->stage >= 2 && (marked || (dense && off[E] > handle->capacity_rows)))
        return fail(EP_ECAPACITY, "dispatch dropped pairs: they did not fit capacity_rows=%d",
                    handle->capacity_rows);
    if (st[1] > 0)
        return fail(EP_EIDS, "topk_idx held %d out-of-range or repeated ids", st[1]);
    return EP_OK;
}

int ep_handle_recv_counts(const ep_handle_t* handle, int32_t* host_counts, int32_t* host_num_recv,
                          hipStream_t stream)
{
    int32_t buf[EP_MAX_EXPERTS + 1 + 4];
    int rc = ep_handle_recv_counts_async(handle, buf, stream);
    if (rc)
        return rc;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return hip_fail(e, "reading counts");
    return ep_recv_counts_decode(handle, buf, host_counts, host_num_recv);
}

int ep_rank_routing(const int64_t* topk_idx, int T, int K, int E, int P, int64_t* part_idx,
                    hipStream_t stream)
{
    g_err.clear();
    int rc = check_dims(T, K, E, P);
    if (rc)
        return rc;
    if (T > 0 && (!topk_idx || !aligned(topk_idx, 8)))
        return fail(EP_EINVAL, "topk_idx must be a non-NULL 8-byte aligned device pointer");
    if (T > 0 && (!part_idx || !aligned(part_idx, 8)))
        return fail(EP_EINVAL, "part_idx must be a non-NULL 8-byte aligned device pointer");
    hipError_t e = moe_ep::launch_rank_routing(topk_idx, T, K, E, P, part_idx, stream);
    if (e != hipSuccess)
        return hip_fail(e, "rank routing launch");
    return EP_OK;
}

int ep_pack_metadata(const int64_t* topk_idx, const float* topk_weights, int K, int E,
                     const int64_t* part_idx, const ep_handle_t* h, int64_t* local_idx,
                     float* local_w, hipStream_t stream)
{
    g_err.clear();
    int rc = check_handle(h, 2);
    if (rc)
        return rc;
    const int T = h->num_tokens;
    const int P = h->num_experts;          // the pack's "experts" are the destinations
    rc = check_dims(T, K, E, P);
    if (rc)
        return rc;
    const int Kp = K < P ? K : P;
    if (h->num_topk != Kp || h->num_partitions != P || h->static_cap || h->expert_alignment > 1)
        return fail(EP_EINVAL, "pack_handle must be a dense layout of part_idx over the %d destinations "
                    "with top-%d (got E=%d P=%d K=%d)", P, Kp, h->num_experts, h->num_partitions,
                    h->num_topk);
    if (T > 0 && (!topk_idx || !aligned(topk_idx, 8) || !part_idx || !aligned(part_idx, 8)))
        return fail(EP_EINVAL, "topk_idx and part_idx must be non-NULL 8-byte aligned device pointers");
    if (T > 0 && (!topk_weights || !aligned(topk_weights, 4)))
        return fail(EP_EINVAL, "topk_weights must be a non-NULL 4-byte aligned device pointer");
    if (T > 0 && h->capacity_rows > 0 &&
        (!local_idx || !aligned(local_idx, 8) || !local_w || !aligned(local_w, 4)))
        return fail(EP_EINVAL, "local_idx (8-byte) and local_w (4-byte) must be non-NULL aligned device "
                    "pointers of capacity_rows*K entries");
    hipError_t e = moe_ep::launch_pack_metadata(topk_idx, topk_weights, part_idx, h->slot, T, K, E, P,
                                                local_idx, local_w, stream);
    if (e != hipSuccess)
        return hip_fail(e, "pack metadata launch");
    return EP_OK;
}

int ep_e4m3fn_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream)
{
    g_err.clear();
    if (n < 0)
        return fail(EP_EINVAL, "n must be >= 0");
    if (n > 0 && (!in || !out || !aligned(in, 4)))
        return fail(EP_EINVAL, "in/out must be non-NULL device pointers (in 4-byte aligned)");
    hipError_t e = moe_ep::launch_e4m3fn_encode(in, out, n, stream);
    if (e != hipSuccess)
        return hip_fail(e, "e4m3fn encode launch");
    return EP_OK;
}

}  // extern "C"
