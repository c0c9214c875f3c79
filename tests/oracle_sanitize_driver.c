/*
 * Drives every oracle entry point over random and edge-case inputs so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer can check the
 * oracle's own memory accesses and integer arithmetic.  Exits 0 when every
 * call returned; the sanitizers abort on the first error they find.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    /* splitmix64 */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void run_case(int T, int H, int K, int E, int P, int cap_mode, int A)
{
    const size_t TK = (size_t)T * K;
    int64_t* idx = xmalloc(sizeof(int64_t) * TK);
    for (size_t i = 0; i < TK; ++i) {
        uint32_t r = rnd() % 100;
        if (r < 5)
            idx[i] = -1 - (int64_t)(rnd() % 7);          /* masked */
        else if (r < 8)
            idx[i] = E + (int64_t)(rnd() % 5);           /* out of range */
        else if (r < 12 && i % K)
            idx[i] = idx[i - 1];                          /* repeated */
        else
            idx[i] = rnd() % E;
    }
    float* w = xmalloc(sizeof(float) * TK);
    for (size_t i = 0; i < TK; ++i)
        w[i] = (float)(rnd() % 1000) / 999.0f;
    uint16_t* x = xmalloc(sizeof(uint16_t) * (size_t)T * H);
    for (size_t i = 0; i < (size_t)T * H; ++i) {
        uint16_t b = (uint16_t)rnd();
        if ((b & 0x7F80) == 0x7F80)
            b &= 0xBFFF;                                  /* finite */
        x[i] = b;
    }

    int32_t* cnt = xmalloc(sizeof(int32_t) * E);
    int32_t* pc = xmalloc(sizeof(int32_t) * P);
    uint8_t* mask = xmalloc((size_t)T * P);
    int32_t ninv = 0;
    uint8_t* valid = xmalloc(TK);
    if (oracle_layout(idx, T, K, E, P, cnt, pc, mask, &ninv, valid) != 0) {
        fprintf(stderr, "layout rejected valid dims\n");
        exit(3);
    }
    int32_t* off = xmalloc(sizeof(int32_t) * (E + 1));
    if (A > 1)
        oracle_expert_offsets_aligned(cnt, E, A, off);
    else
        oracle_expert_offsets(cnt, E, off);
    int N = off[E];
    int cap = cap_mode == 0 ? N : (cap_mode == 1 ? N / 2 : 0);
    int32_t* slot = xmalloc(sizeof(int32_t) * TK);
    int32_t* src = xmalloc(sizeof(int32_t) * (cap > 0 ? cap : 1));
    int32_t ovf = 0;
    oracle_slots(idx, valid, T, K, off, E, cap, slot, src, &ovf);

    const int nb = H / 128;
    const int fp8 = H % 128 == 0;                          /* FP8 needs whole 128-blocks */
    uint8_t* q = calloc((size_t)(cap > 0 ? cap : 1) * H, 1);
    float* sc = calloc((size_t)(cap > 0 ? cap : 1) * (nb > 0 ? nb : 1), sizeof(float));
    uint16_t* rb = calloc((size_t)(cap > 0 ? cap : 1) * H, sizeof(uint16_t));
    if (fp8)
        oracle_dispatch(x, T, H, K, slot, 1, q, sc);
    oracle_dispatch(x, T, H, K, slot, 0, rb, NULL);
    uint16_t* out = xmalloc(sizeof(uint16_t) * (size_t)T * H);
    oracle_combine(rb, T, H, K, slot, w, out);
    oracle_dispatch_backward(rb, T, H, K, slot, out);
    float* gw = xmalloc(sizeof(float) * TK);
    oracle_combine_backward(out, rb, T, H, K, slot, w, rb, gw);
    if (fp8) {
        oracle_combine_fp8(q, sc, T, H, K, slot, w, out);
        oracle_combine_fp8(q, sc, T, H, K, slot, NULL, out);
        float* xs = xmalloc(sizeof(float) * (size_t)T * nb);
        uint8_t* xq = xmalloc((size_t)T * H);
        for (size_t i = 0; i < (size_t)T * nb; ++i)
            xs[i] = (float)(rnd() % 100);
        for (size_t i = 0; i < (size_t)T * H; ++i)
            xq[i] = (uint8_t)rnd();
        oracle_dispatch_fp8_input(xq, xs, T, H, K, slot, q, sc);
        free(xs);
        free(xq);
    }
    /* static-capacity layout of the low-latency path */
    int32_t sovf = 0;
    int scap = 1 + (int)(rnd() % 4);
    oracle_slots_static(idx, valid, T, K, E, scap, slot, &sovf);

    /* expert parallelism over P ranks: destination routing, the pack's slots
     * (layout and slots on the destinations) and the packed rows' metadata */
    const int Kp = K < P ? K : P;
    int64_t* part = xmalloc(sizeof(int64_t) * ((size_t)T * Kp > 0 ? (size_t)T * Kp : 1));
    oracle_rank_routing(idx, T, K, E, P, part);
    int32_t* pcnt = xmalloc(sizeof(int32_t) * P);
    int32_t* ppc = xmalloc(sizeof(int32_t) * P);
    uint8_t* pmask = xmalloc((size_t)T * P + 1);
    uint8_t* pvalid = xmalloc((size_t)T * Kp + 1);
    int32_t pinv = 0;
    if (oracle_layout(part, T, Kp, P, P, pcnt, ppc, pmask, &pinv, pvalid) != 0 || pinv != 0) {
        fprintf(stderr, "rank routing gave an invalid destination list\n");
        exit(5);
    }
    int32_t* poff = xmalloc(sizeof(int32_t) * (P + 1));
    oracle_expert_offsets(pcnt, P, poff);
    const int prows = poff[P];
    int32_t* pslot = xmalloc(sizeof(int32_t) * ((size_t)T * Kp + 1));
    int32_t* psrc = xmalloc(sizeof(int32_t) * (prows > 0 ? prows : 1));
    int32_t povf = 0;
    oracle_slots(part, pvalid, T, Kp, poff, P, prows, pslot, psrc, &povf);
    int64_t* lidx = xmalloc(sizeof(int64_t) * ((size_t)prows * K + 1));
    float* lw = xmalloc(sizeof(float) * ((size_t)prows * K + 1));
    oracle_pack_metadata(idx, w, part, pslot, T, K, E, P, lidx, lw);
    free(part); free(pcnt); free(ppc); free(pmask); free(pvalid); free(poff); free(pslot); free(psrc);
    free(lidx); free(lw);

    free(idx); free(w); free(x); free(cnt); free(pc); free(mask); free(valid); free(off);
    free(slot); free(src); free(q); free(sc); free(rb); free(out); free(gw);
}

int main(void)
{
    /* codec helpers over every bf16 pattern and a sweep of fp32 values */
    for (uint32_t b = 0; b < 65536; ++b) {
        float f = oracle_bf16_to_f32((uint16_t)b);
        (void)oracle_bf16_rne(f == f ? f : 0.0f);
        (void)oracle_e4m3fn_rne_sat(f == f ? f : 0.0f);
    }
    for (int c = 0; c < 256; ++c)
        (void)oracle_e4m3fn_to_f32((uint8_t)c);
    /* dims: empty, single, ragged, maximum K, E and P */
    const int cases[][6] = {
        {0, 128, 8, 16, 4, 1},   {1, 128, 1, 1, 1, 1},    {33, 256, 3, 8, 2, 4},
        {300, 136, 6, 40, 8, 1}, {257, 384, 16, 64, 16, 32}, {64, 128, 16, 1024, 64, 7},
        {500, 256, 8, 256, 8, 128},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i)
        for (int cap_mode = 0; cap_mode < 3; ++cap_mode)
            run_case(cases[i][0], cases[i][1], cases[i][2], cases[i][3], cases[i][4], cap_mode,
                     cases[i][5]);
    /* rejected dims return -1 without touching the outputs */
    int32_t dummy = 0;
    if (oracle_layout(NULL, 10, 0, 8, 2, &dummy, &dummy, NULL, &dummy, NULL) != -1 ||
        oracle_layout(NULL, 10, 2, 9, 2, &dummy, &dummy, NULL, &dummy, NULL) != -1) {
        fprintf(stderr, "invalid dims accepted\n");
        return 4;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
