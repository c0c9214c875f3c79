/*
 * The C ABI from plain C, without Python or torch: random routing and rows
 * from a splitmix64 stream, device buffers from the HIP runtime, then
 * ep_get_dispatch_layout -> ep_dispatch (FP8 and BF16) -> ep_handle_recv_counts
 * -> ep_combine, and the allocation-free low-latency dispatch twice in a row
 * (the second batch smaller) -> ep_handle_recv_counts -> ep_combine, each
 * output compared byte for byte with the CPU oracle (liboracle, test
 * infrastructure).  Prints "c abi driver: ok" and exits 0 on success.  Built
 * by the package build step; run by a GPU test.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_ep.h"
#include "oracle.h"

#define CHECK_HIP(x)                                                             \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(2);                                                             \
        }                                                                        \
    } while (0)
#define CHECK_EP(x)                                                              \
    do {                                                                         \
        int r_ = (x);                                                            \
        if (r_ != EP_OK) {                                                       \
            fprintf(stderr, "%s:%d: rc=%d %s\n", __FILE__, __LINE__, r_, ep_last_error()); \
            exit(3);                                                             \
        }                                                                        \
    } while (0)

static uint64_t g_s = 0x1234567ull;
static uint64_t next_u64(void)
{
    uint64_t z = (g_s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int run(int T, int H, int K, int E, int P, int use_fp8)
{
    const size_t TK = (size_t)T * K;
    int64_t* idx = malloc(TK * 8);
    float* w = malloc(TK * 4);
    uint16_t* x = malloc((size_t)T * H * 2);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int64_t e;
            int dup;
            do {                                  /* distinct experts per token */
                e = (int64_t)(next_u64() % (uint64_t)E);
                dup = 0;
                for (int j = 0; j < k; ++j)
                    dup |= idx[(size_t)t * K + j] == e;
            } while (dup);
            idx[(size_t)t * K + k] = (next_u64() % 20 == 0) ? -1 : e;
            w[(size_t)t * K + k] = (float)(next_u64() % 1000) / 1000.0f;
        }
    for (size_t i = 0; i < (size_t)T * H; ++i) {
        /* bf16 of a value in [-4, 4): sign, exponent 125..128, random mantissa */
        uint16_t b = (uint16_t)(((next_u64() & 1) << 15) | ((125 + next_u64() % 4) << 7) | (next_u64() & 0x7F));
        x[i] = b;
    }

    /* the oracle's answer */
    int32_t* cnt = malloc(E * 4);
    int32_t* pc = malloc(P * 4);
    uint8_t* mask = malloc((size_t)T * P);
    uint8_t* valid = malloc(TK);
    int32_t ninv = 0;
    if (oracle_layout(idx, T, K, E, P, cnt, pc, mask, &ninv, valid) != 0)
        return 10;
    int32_t* off = malloc((E + 1) * 4);
    oracle_expert_offsets(cnt, E, off);
    const int N = off[E];
    int32_t* slot = malloc(TK * 4);
    int32_t* src = malloc((size_t)(N > 0 ? N : 1) * 4);
    int32_t ovf = 0;
    oracle_slots(idx, valid, T, K, off, E, (int)TK, slot, src, &ovf);
    const size_t elt = use_fp8 ? 1 : 2;
    const int nb = H / 128;
    void* recv_ref = calloc((size_t)(N > 0 ? N : 1) * H, elt);
    float* sc_ref = calloc((size_t)(N > 0 ? N : 1) * (nb > 0 ? nb : 1), 4);
    oracle_dispatch(x, T, H, K, slot, use_fp8, recv_ref, use_fp8 ? sc_ref : NULL);
    uint16_t* y = malloc((size_t)(N > 0 ? N : 1) * H * 2);
    for (size_t i = 0; i < (size_t)N * H; ++i)
        y[i] = (uint16_t)(((next_u64() & 1) << 15) | ((124 + next_u64() % 4) << 7) | (next_u64() & 0x7F));
    uint16_t* out_ref = malloc((size_t)T * H * 2);
    oracle_combine(y, T, H, K, slot, w, out_ref);

    /* the library through its C ABI */
    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    void *d_idx, *d_w, *d_x, *d_recv, *d_sc = NULL, *d_y, *d_out, *d_ws, *d_ntpp, *d_ntpe, *d_mask, *d_ninv;
    const size_t ws_bytes = ep_workspace_bytes(T, K, E, P);
    CHECK_HIP(hipMalloc(&d_idx, TK * 8));
    CHECK_HIP(hipMalloc(&d_w, TK * 4));
    CHECK_HIP(hipMalloc(&d_x, (size_t)T * H * 2));
    CHECK_HIP(hipMalloc(&d_recv, TK * H * elt));
    if (use_fp8)
        CHECK_HIP(hipMalloc(&d_sc, TK * nb * 4));
    CHECK_HIP(hipMalloc(&d_y, TK * H * 2));
    CHECK_HIP(hipMalloc(&d_out, (size_t)T * H * 2));
    CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    CHECK_HIP(hipMalloc(&d_ntpp, P * 4));
    CHECK_HIP(hipMalloc(&d_ntpe, E * 4));
    CHECK_HIP(hipMalloc(&d_mask, (size_t)T * P));
    CHECK_HIP(hipMalloc(&d_ninv, 4));
    CHECK_HIP(hipMemcpy(d_idx, idx, TK * 8, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, w, TK * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, (size_t)T * H * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_y, y, (size_t)N * H * 2, hipMemcpyHostToDevice));

    ep_handle_t h;
    CHECK_EP(ep_get_dispatch_layout(d_idx, T, K, E, P, d_ntpp, d_ntpe, d_mask, d_ninv, d_ws, ws_bytes,
                                    &h, s));
    CHECK_EP(ep_dispatch(d_x, d_w, H, use_fp8, d_recv, d_sc, (int)TK, &h, s));
    int32_t* counts = malloc(E * 4);
    int32_t nrecv = -1;
    CHECK_EP(ep_handle_recv_counts(&h, counts, &nrecv, s));
    CHECK_EP(ep_combine(d_y, &h, NULL, d_out, s));
    CHECK_HIP(hipStreamSynchronize(s));

    int bad = 0;
    int32_t* g32 = malloc((size_t)(E > P ? E : P) * 4);
    CHECK_HIP(hipMemcpy(g32, d_ntpe, E * 4, hipMemcpyDeviceToHost));
    bad |= memcmp(g32, cnt, E * 4) != 0;
    bad |= memcmp(counts, cnt, E * 4) != 0 || nrecv != N;
    CHECK_HIP(hipMemcpy(g32, d_ntpp, P * 4, hipMemcpyDeviceToHost));
    bad |= memcmp(g32, pc, P * 4) != 0;
    uint8_t* gm = malloc((size_t)T * P);
    CHECK_HIP(hipMemcpy(gm, d_mask, (size_t)T * P, hipMemcpyDeviceToHost));
    bad |= memcmp(gm, mask, (size_t)T * P) != 0;
    int32_t* gs = malloc(TK * 4);
    CHECK_HIP(hipMemcpy(gs, h.slot, TK * 4, hipMemcpyDeviceToHost));
    bad |= memcmp(gs, slot, TK * 4) != 0;
    void* grecv = malloc((size_t)(N > 0 ? N : 1) * H * elt);
    CHECK_HIP(hipMemcpy(grecv, d_recv, (size_t)N * H * elt, hipMemcpyDeviceToHost));
    bad |= memcmp(grecv, recv_ref, (size_t)N * H * elt) != 0;
    if (use_fp8) {
        float* gsc = malloc((size_t)(N > 0 ? N : 1) * nb * 4);
        CHECK_HIP(hipMemcpy(gsc, d_sc, (size_t)N * nb * 4, hipMemcpyDeviceToHost));
        bad |= memcmp(gsc, sc_ref, (size_t)N * nb * 4) != 0;
        free(gsc);
    }
    uint16_t* gout = malloc((size_t)T * H * 2);
    CHECK_HIP(hipMemcpy(gout, d_out, (size_t)T * H * 2, hipMemcpyDeviceToHost));
    bad |= memcmp(gout, out_ref, (size_t)T * H * 2) != 0;
    printf("T=%d H=%d K=%d E=%d P=%d fp8=%d N=%d: %s\n", T, H, K, E, P, use_fp8, N, bad ? "MISMATCH" : "match");

    hipFree(d_idx); hipFree(d_w); hipFree(d_x); hipFree(d_recv); if (d_sc) hipFree(d_sc);
    hipFree(d_y); hipFree(d_out); hipFree(d_ws); hipFree(d_ntpp); hipFree(d_ntpe); hipFree(d_mask);
    hipFree(d_ninv);
    CHECK_HIP(hipStreamDestroy(s));
    free(idx); free(w); free(x); free(cnt); free(pc); free(mask); free(valid); free(off); free(slot);
    free(src); free(recv_ref); free(sc_ref); free(y); free(out_ref); free(counts); free(g32); free(gm);
    free(gs); free(grecv); free(gout);
    return bad;
}

/* The allocation-free low-latency dispatch: no workspace; the handle's arrays
 * live in the library's per-GPU array.  Layout outputs, slots, the rows and
 * scales of every dispatched pair, the received counts and combine against
 * the oracle. */
static int run_noalloc(int T, int H, int K, int E, int P, int cap, int use_fp8)
{
    const size_t TK = (size_t)T * K;
    const size_t rows = (size_t)E * cap;
    int64_t* idx = malloc(TK * 8);
    float* w = malloc(TK * 4);
    uint16_t* x = malloc((size_t)T * H * 2);
    for (size_t i = 0; i < TK; ++i) {
        idx[i] = (next_u64() % 16 == 0) ? -1 : (int64_t)(next_u64() % (uint64_t)E);   /* repeats possible */
        w[i] = (float)(next_u64() % 1000) / 1000.0f;
    }
    for (size_t i = 0; i < (size_t)T * H; ++i)
        x[i] = (uint16_t)(((next_u64() & 1) << 15) | ((125 + next_u64() % 4) << 7) | (next_u64() & 0x7F));

    int32_t* cnt = malloc(E * 4);
    int32_t* pc = malloc(P * 4);
    uint8_t* mask = malloc((size_t)T * P);
    uint8_t* valid = malloc(TK);
    int32_t ninv = 0, ovf = 0;
    if (oracle_layout(idx, T, K, E, P, cnt, pc, mask, &ninv, valid) != 0)
        return 10;
    int32_t* slot = malloc(TK * 4);
    oracle_slots_static(idx, valid, T, K, E, cap, slot, &ovf);
    const size_t elt = use_fp8 ? 1 : 2;
    const int nb = H / 128;
    void* recv_ref = calloc(rows * H, elt);
    float* sc_ref = calloc(rows * (nb > 0 ? nb : 1), 4);
    oracle_dispatch(x, T, H, K, slot, use_fp8, recv_ref, use_fp8 ? sc_ref : NULL);
    uint16_t* y = malloc(rows * H * 2);
    for (size_t i = 0; i < rows * H; ++i)
        y[i] = (uint16_t)(((next_u64() & 1) << 15) | ((124 + next_u64() % 4) << 7) | (next_u64() & 0x7F));
    uint16_t* out_ref = malloc((size_t)T * H * 2);
    oracle_combine(y, T, H, K, slot, w, out_ref);

    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    void *d_idx, *d_w, *d_x, *d_recv, *d_sc = NULL, *d_y, *d_out, *d_ntpp, *d_ntpe, *d_mask, *d_ninv;
    CHECK_HIP(hipMalloc(&d_idx, TK * 8));
    CHECK_HIP(hipMalloc(&d_w, TK * 4));
    CHECK_HIP(hipMalloc(&d_x, (size_t)T * H * 2));
    CHECK_HIP(hipMalloc(&d_recv, rows * H * elt));
    if (use_fp8)
        CHECK_HIP(hipMalloc(&d_sc, rows * nb * 4));
    CHECK_HIP(hipMalloc(&d_y, rows * H * 2));
    CHECK_HIP(hipMalloc(&d_out, (size_t)T * H * 2));
    CHECK_HIP(hipMalloc(&d_ntpp, P * 4));
    CHECK_HIP(hipMalloc(&d_ntpe, E * 4));
    CHECK_HIP(hipMalloc(&d_mask, (size_t)T * P));
    CHECK_HIP(hipMalloc(&d_ninv, 4));
    CHECK_HIP(hipMemcpy(d_idx, idx, TK * 8, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, w, TK * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, (size_t)T * H * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_y, y, rows * H * 2, hipMemcpyHostToDevice));

    ep_handle_t h;
    CHECK_EP(ep_low_latency_dispatch_noalloc(d_x, d_idx, d_w, T, H, K, E, P, use_fp8, cap, d_recv, d_sc,
                                             d_ntpp, d_ntpe, d_mask, d_ninv, &h, s));
    int32_t* counts = malloc(E * 4);
    int32_t nrecv = -1;
    const int st = ep_handle_recv_counts(&h, counts, &nrecv, s);
    CHECK_EP(ep_combine(d_y, &h, NULL, d_out, s));
    CHECK_HIP(hipStreamSynchronize(s));

    int bad = st != (ovf ? EP_ECAPACITY : (ninv ? EP_EIDS : EP_OK));
    int N = 0;
    for (int e = 0; e < E; ++e) {
        const int c = cnt[e] < cap ? cnt[e] : cap;
        bad |= counts[e] != c;
        N += c;
    }
    bad |= nrecv != N || h.ws_bytes != EP_NOALLOC_SCRATCH_BYTES;
    int32_t* g32 = malloc((size_t)(E > P ? E : P) * 4);
    CHECK_HIP(hipMemcpy(g32, d_ntpe, E * 4, hipMemcpyDeviceToHost));
    bad |= memcmp(g32, cnt, E * 4) != 0;
    CHECK_HIP(hipMemcpy(g32, d_ntpp, P * 4, hipMemcpyDeviceToHost));
    bad |= memcmp(g32, pc, P * 4) != 0;
    uint8_t* gm = malloc((size_t)T * P);
    CHECK_HIP(hipMemcpy(gm, d_mask, (size_t)T * P, hipMemcpyDeviceToHost));
    bad |= memcmp(gm, mask, (size_t)T * P) != 0;
    int32_t* gs = malloc(TK * 4);
    CHECK_HIP(hipMemcpy(gs, h.slot, TK * 4, hipMemcpyDeviceToHost));
    bad |= memcmp(gs, slot, TK * 4) != 0;
    uint8_t* grecv = malloc(rows * H * elt);
    float* gsc = malloc(rows * (nb > 0 ? nb : 1) * 4);
    CHECK_HIP(hipMemcpy(grecv, d_recv, rows * H * elt, hipMemcpyDeviceToHost));
    if (use_fp8)
        CHECK_HIP(hipMemcpy(gsc, d_sc, rows * nb * 4, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < TK; ++i) {          /* rows past an expert's count are not written */
        if (slot[i] < 0)
            continue;
        const size_t r = (size_t)slot[i];
        bad |= memcmp(grecv + r * H * elt, (const uint8_t*)recv_ref + r * H * elt, H * elt) != 0;
        if (use_fp8)
            bad |= memcmp(gsc + r * nb, sc_ref + r * nb, (size_t)nb * 4) != 0;
    }
    uint16_t* gout = malloc((size_t)T * H * 2);
    CHECK_HIP(hipMemcpy(gout, d_out, (size_t)T * H * 2, hipMemcpyDeviceToHost));
    bad |= memcmp(gout, out_ref, (size_t)T * H * 2) != 0;
    printf("no-alloc T=%d H=%d K=%d E=%d P=%d cap=%d fp8=%d dropped=%d: %s\n", T, H, K, E, P, cap, use_fp8,
           ovf, bad ? "MISMATCH" : "match");

    hipFree(d_idx); hipFree(d_w); hipFree(d_x); hipFree(d_recv); if (d_sc) hipFree(d_sc);
    hipFree(d_y); hipFree(d_out); hipFree(d_ntpp); hipFree(d_ntpe); hipFree(d_mask); hipFree(d_ninv);
    CHECK_HIP(hipStreamDestroy(s));
    free(idx); free(w); free(x); free(cnt); free(pc); free(mask); free(valid); free(slot);
    free(recv_ref); free(sc_ref); free(y); free(out_ref); free(counts); free(g32); free(gm);
    free(gs); free(grecv); free(gsc); free(gout);
    return bad;
}

int main(void)
{
    int bad = 0;
    bad |= run(1000, 1024, 8, 64, 8, 1);
    bad |= run(257, 520, 4, 16, 4, 0);
    bad |= run(3000, 7168, 8, 256, 8, 1);
    bad |= run_noalloc(128, 7168, 8, 256, 8, 16, 1);
    bad |= run_noalloc(37, 1024, 4, 32, 4, 2, 0);
    if (bad) {
        printf("c abi driver: FAILED\n");
        return 1;
    }
    printf("c abi driver: ok\n");
    return 0;
}
