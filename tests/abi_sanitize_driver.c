/*
 * Host-side checks of the C ABI under AddressSanitizer and UndefinedBehavior-
 * Sanitizer, linked against a host-only build of the library (no device code;
 * nothing here reaches a GPU):
 *   - workspace sizing over the whole range of dimensions, valid and invalid;
 *   - argument validation of every entry point: each call below is refused
 *     before its first HIP call, with EP_EINVAL and a message;
 *   - the host decode of the count buffer (ep_recv_counts_decode) over
 *     arbitrary buffer contents and handle states, and its refusal of
 *     handles whose dimensions are out of range.
 * Prints "abi sanitizer run: ok" when every check holds.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_ep.h"

static int failures = 0;

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

/* the call must be refused as an invalid argument, with a message */
#define REFUSED(call)                                                            \
    do {                                                                         \
        int rc_ = (call);                                                        \
        CHECK(rc_ == EP_EINVAL);                                                 \
        CHECK(ep_last_error()[0] != '\0');                                       \
    } while (0)

static uint64_t rng = 0x243F6A8885A308D3ull;

static uint64_t next_u64(void) /* splitmix64 */
{
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int dims_valid(int T, int K, int E, int P)
{
    return T >= 0 && K >= 1 && K <= EP_MAX_TOPK && E >= 1 && E <= EP_MAX_EXPERTS && P >= 1 &&
           P <= EP_MAX_PARTITIONS && E % P == 0 && (int64_t)T * K < ((int64_t)1 << 31);
}

static void workspace_sizes(void)
{
    const int Ts[] = {INT_MIN, -1, 0, 1, 255, 256, 257, 8192, 1 << 20, (1 << 27) - 1, INT_MAX};
    const int Ks[] = {INT_MIN, -1, 0, 1, 2, 8, 16, 17, INT_MAX};
    const int Es[] = {INT_MIN, -1, 0, 1, 8, 256, 1024, 1025, INT_MAX};
    const int Ps[] = {INT_MIN, -1, 0, 1, 3, 8, 64, 65, INT_MAX};
    for (size_t a = 0; a < sizeof Ts / sizeof *Ts; ++a)
        for (size_t b = 0; b < sizeof Ks / sizeof *Ks; ++b)
            for (size_t c = 0; c < sizeof Es / sizeof *Es; ++c)
                for (size_t d = 0; d < sizeof Ps / sizeof *Ps; ++d) {
                    const int T = Ts[a], K = Ks[b], E = Es[c], P = Ps[d];
                    const size_t n = ep_workspace_bytes(T, K, E, P);
                    if (!dims_valid(T, K, E, P)) {
                        CHECK(n == 0);
                        continue;
                    }
                    CHECK(n > 0);
                    /* at least the per-pair slot, code and weight arrays */
                    CHECK(n >= (size_t)T * K * 12);
                    if (T > 0)
                        CHECK(ep_workspace_bytes(T - 1, K, E, P) <= n);
                }
}

static void argument_validation(void)
{
    ep_handle_t h;
    memset(&h, 0, sizeof h);
    int64_t ids[8] = {0};
    float w[8] = {0};
    int32_t i32[64] = {0};
    uint8_t u8[64] = {0};
    char ws[4096];

    /* layout: bad dimensions, NULL pointers, a workspace that is too small */
    REFUSED(ep_get_dispatch_layout(ids, -1, 2, 4, 2, i32, i32, u8, i32, ws, sizeof ws, &h, NULL));
    REFUSED(ep_get_dispatch_layout(ids, 4, 0, 4, 2, i32, i32, u8, i32, ws, sizeof ws, &h, NULL));
    REFUSED(ep_get_dispatch_layout(ids, 4, 2, 5, 2, i32, i32, u8, i32, ws, sizeof ws, &h, NULL));
    REFUSED(ep_get_dispatch_layout(ids, 4, 2, 4, 2, i32, i32, u8, i32, ws, sizeof ws, NULL, NULL));
    REFUSED(ep_get_dispatch_layout(NULL, 4, 2, 4, 2, i32, i32, u8, i32, ws, sizeof ws, &h, NULL));
    REFUSED(ep_get_dispatch_layout(ids, 4, 2, 4, 2, i32, i32, u8, i32, ws, 16, &h, NULL));
    REFUSED(ep_get_dispatch_layout(ids, 4, 2, 4, 2, i32, i32, u8, i32, NULL, sizeof ws, &h, NULL));
    REFUSED(ep_get_dispatch_layout_aligned(ids, 4, 2, 4, 2, 0, i32, i32, u8, i32, ws, sizeof ws, &h,
                                           NULL));
    REFUSED(ep_get_dispatch_layout_aligned(ids, 4, 2, 4, 2, EP_MAX_ALIGNMENT + 1, i32, i32, u8, i32,
                                           ws, sizeof ws, &h, NULL));

    /* calls on a handle no layout call filled */
    REFUSED(ep_dispatch(u8, w, 256, 1, u8, (float*)i32, 8, &h, NULL));
    REFUSED(ep_dispatch_ex(u8, NULL, w, 256, 1, 0, u8, (float*)i32, 8, &h, NULL));
    REFUSED(ep_dispatch_cached(u8, &h, u8, (float*)i32, NULL));
    REFUSED(ep_dispatch_cached_ex(u8, NULL, &h, u8, (float*)i32, NULL));
    REFUSED(ep_combine(u8, &h, NULL, u8, NULL));
    REFUSED(ep_combine_fp8(u8, (float*)i32, &h, NULL, u8, NULL));
    REFUSED(ep_dispatch_backward(u8, &h, u8, NULL));
    REFUSED(ep_dispatch_backward_fp8(u8, (float*)i32, &h, u8, NULL));
    REFUSED(ep_combine_backward(u8, NULL, &h, NULL, u8, NULL, NULL));
    REFUSED(ep_handle_recv_counts(&h, i32, i32, NULL));
    REFUSED(ep_handle_recv_counts_async(&h, i32, NULL));
    REFUSED(ep_recv_counts_decode(&h, i32, i32, i32));
    REFUSED(ep_pack_metadata(ids, w, 2, 4, ids, &h, ids, w, NULL));
    /* and on no handle at all */
    REFUSED(ep_dispatch(u8, w, 256, 1, u8, (float*)i32, 8, NULL, NULL));
    REFUSED(ep_combine(u8, NULL, NULL, u8, NULL));
    REFUSED(ep_recv_counts_decode(NULL, i32, i32, i32));

    /* a layout-stage handle (magic set, not dispatched) for the calls that
       need a dispatched one; its pointers are never followed */
    ep_handle_t s;
    memset(&s, 0, sizeof s);
    s.magic = EP_HANDLE_MAGIC;
    s.stage = 1;
    s.num_tokens = 4;
    s.num_topk = 2;
    s.num_experts = 4;
    s.num_partitions = 2;
    s.expert_alignment = 1;
    REFUSED(ep_combine(u8, &s, NULL, u8, NULL));
    REFUSED(ep_dispatch_backward(u8, &s, u8, NULL));
    REFUSED(ep_combine_backward(u8, NULL, &s, NULL, u8, NULL, NULL));
    REFUSED(ep_dispatch_cached(u8, &s, u8, (float*)i32, NULL));
    /* dispatch arguments on it: hidden size and FP8 block rule */
    REFUSED(ep_dispatch(u8, w, 0, 0, u8, NULL, 8, &s, NULL));
    REFUSED(ep_dispatch(u8, w, 12, 0, u8, NULL, 8, &s, NULL));
    REFUSED(ep_dispatch(u8, w, EP_MAX_HIDDEN + 8, 0, u8, NULL, 8, &s, NULL));
    REFUSED(ep_dispatch(u8, w, 264, 1, u8, (float*)i32, 8, &s, NULL));
    REFUSED(ep_dispatch(u8, w, 256, 1, u8, NULL, 8, &s, NULL));
    REFUSED(ep_dispatch(u8, w, 256, 0, u8, NULL, -1, &s, NULL));

    /* a handle with the magic but corrupted dimensions */
    ep_handle_t bad = s;
    bad.stage = 2;
    const int bad_dims[][4] = {{-1, 2, 4, 2}, {4, 0, 4, 2}, {4, 17, 4, 2}, {4, 2, 0, 2},
                               {4, 2, 4096, 2}, {4, 2, 4, 0}, {4, 2, 6, 4}, {INT_MAX, 2, 4, 2}};
    for (size_t i = 0; i < sizeof bad_dims / sizeof *bad_dims; ++i) {
        bad.num_tokens = bad_dims[i][0];
        bad.num_topk = bad_dims[i][1];
        bad.num_experts = bad_dims[i][2];
        bad.num_partitions = bad_dims[i][3];
        REFUSED(ep_recv_counts_decode(&bad, i32, i32, i32));
        REFUSED(ep_combine(u8, &bad, NULL, u8, NULL));
        REFUSED(ep_handle_recv_counts_async(&bad, i32, NULL));
    }

    /* low-latency dispatch: more tokens than one call takes, bad dims */
    REFUSED(ep_low_latency_dispatch(u8, ids, w, EP_MAX_LL_TOKENS + 1, 256, 2, 4, 2, 1, 8, u8,
                                    (float*)i32, i32, i32, u8, i32, ws, sizeof ws, &h, NULL));
    REFUSED(ep_low_latency_dispatch(u8, ids, w, 4, 256, 2, 5, 2, 1, 8, u8, (float*)i32, i32, i32,
                                    u8, i32, ws, sizeof ws, &h, NULL));
    REFUSED(ep_low_latency_dispatch_noalloc(u8, ids, w, EP_MAX_LL_TOKENS + 1, 256, 2, 4, 2, 1, 8,
                                            u8, (float*)i32, i32, i32, u8, i32, &h, NULL));

    /* destination routing and the FP8 encoder */
    REFUSED(ep_rank_routing(ids, 4, 2, 5, 2, ids, NULL));
    REFUSED(ep_rank_routing(NULL, 4, 2, 4, 2, ids, NULL));
    REFUSED(ep_rank_routing(ids, 4, 2, 4, 2, NULL, NULL));
    REFUSED(ep_e4m3fn_encode(NULL, u8, 4, NULL));
    REFUSED(ep_e4m3fn_encode((const float*)i32, NULL, 4, NULL));
    REFUSED(ep_e4m3fn_encode((const float*)i32, u8, -1, NULL));
}

static void count_decode_fuzz(void)
{
    static int32_t buf[EP_MAX_EXPERTS + 1 + 4];
    static int32_t counts[EP_MAX_EXPERTS];
    const int Ps[] = {1, 2, 4, 8, 16, 64};
    for (int it = 0; it < 200000; ++it) {
        ep_handle_t d;
        memset(&d, 0, sizeof d);
        d.magic = EP_HANDLE_MAGIC;
        d.stage = 1 + (int)(next_u64() % 2);
        const int P = Ps[next_u64() % (sizeof Ps / sizeof *Ps)];
        const int E = P * (1 + (int)(next_u64() % (EP_MAX_EXPERTS / P)));
        d.num_experts = E;
        d.num_partitions = P;
        d.num_topk = 1 + (int)(next_u64() % EP_MAX_TOPK);
        d.num_tokens = (int)(next_u64() % 100000);
        d.capacity_rows = (int32_t)next_u64();
        d.dispatch_seq = (int32_t)(next_u64() % 4);
        d.static_cap = (next_u64() % 4 == 0) ? 1 + (int)(next_u64() % 64) : 0;
        d.expert_alignment = (int)(next_u64() % 3 == 0 ? 128 : 1);
        const int mode = (int)(next_u64() % 3);
        for (int i = 0; i < E + 5; ++i) {
            if (mode == 0)          /* arbitrary words */
                buf[i] = (int32_t)next_u64();
            else if (mode == 1)     /* small values, overflow word and invalid count included */
                buf[i] = (int32_t)(next_u64() % 7) - 1;
            else                    /* well-formed: non-decreasing offsets */
                buf[i] = i <= E ? (i ? buf[i - 1] + (int32_t)(next_u64() % 50) : 0)
                                : (int32_t)(next_u64() % 3);
        }
        int32_t n = -12345;
        const int rc = ep_recv_counts_decode(&d, buf, (next_u64() & 1) ? counts : NULL, &n);
        CHECK(rc == EP_OK || rc == EP_ECAPACITY || rc == EP_EIDS);
        CHECK(n == buf[E]);
        if (mode == 2 && rc == EP_OK) {
            int64_t sum = 0;
            int32_t chk[EP_MAX_EXPERTS];
            CHECK(ep_recv_counts_decode(&d, buf, chk, NULL) == EP_OK);
            for (int e = 0; e < E; ++e) {
                CHECK(chk[e] >= 0);
                sum += chk[e];
            }
            CHECK(sum == buf[E]);
        }
    }
}

int main(void)
{
    CHECK(ep_version() == EP_VERSION);
    CHECK(ep_last_error() != NULL);
    workspace_sizes();
    argument_validation();
    count_decode_fuzz();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi sanitizer run: ok\n");
    return 0;
}
