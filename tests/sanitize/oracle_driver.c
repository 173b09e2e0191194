/*
 * Exercises every function of the CPU oracle (oracle/moe_oracle.c) for the
 * AddressSanitizer / UndefinedBehaviorSanitizer build of tests/test_sanitizers.py:
 * element decoders over their whole domains, block and row quantization,
 * dequantization, the MX dot, routing (with invalid ids, duplicates and a
 * capacity that is too small) and the forward (token subsets, both activation
 * modes, every optional output), on small shapes, with a few closed-form
 * results so that the run also checks what it computes.  Exit status 0 on
 * success; the sanitizers abort on any finding.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint32_t rng_state = 12345u;
static uint32_t rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}

static uint16_t bf16_bits_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);          /* values used below are bf16-exact */
}

int main(void)
{
    /* element decoders, whole domains */
    for (int c = 0; c < 16; ++c) CHECK(fabs(oracle_e2m1_value(c)) <= 6.0);
    for (int s = 0; s < 255; ++s) CHECK(oracle_e8m0_value(s) == ldexp(1.0, s - 127));
    CHECK(isnan(oracle_e8m0_value(255)));
    for (uint32_t b = 0; b < 65536; ++b) {
        double v = oracle_bf16_value((uint16_t)b);
        if (!isnan(v)) CHECK(oracle_bf16_round(v) == (uint16_t)b || v == 0.0);
    }
    CHECK(oracle_bf16_round(1e300) == 0x7F80);

    /* block quantization: random blocks and edge blocks, both entry points */
    uint8_t codes[32], scale;
    double x[32];
    uint16_t xb[32];
    for (int it = 0; it < 2000; ++it) {
        int e = (int)(rnd() % 300) - 150;
        for (int i = 0; i < 32; ++i) {
            x[i] = ldexp(((double)(rnd() % 2001) - 1000.0) / 256.0, e);
            xb[i] = oracle_bf16_round(x[i]);
            x[i] = oracle_bf16_value(xb[i]);
        }
        oracle_mx_quant_block_f64(x, codes, &scale);
        uint8_t codes2[32], scale2;
        oracle_mx_quant_block_bf16(xb, codes2, &scale2);
        CHECK(scale == scale2 && memcmp(codes, codes2, 32) == 0);
    }
    memset(x, 0, sizeof x);
    oracle_mx_quant_block_f64(x, codes, &scale);
    CHECK(scale == 0);

    /* rows: quantize (several thread counts), dequantize, dot */
    enum { ROWS = 7, COLS = 96 };
    uint16_t xr[ROWS * COLS];
    for (int i = 0; i < ROWS * COLS; ++i) xr[i] = bf16_bits_of((float)((int)(rnd() % 64) - 32) / 8.0f);
    uint8_t packed[ROWS * COLS / 2], scales[ROWS * COLS / 32];
    double deq[ROWS * COLS];
    for (int nt = 1; nt <= 9; nt += 4) {
        CHECK(oracle_mx_quantize_rows(xr, ROWS, COLS, packed, scales, nt) == 0);
        CHECK(oracle_mx_dequantize_rows(packed, scales, ROWS, COLS, deq) == 0);
    }
    CHECK(oracle_mx_quantize_rows(xr, ROWS, 33, packed, scales, 1) != 0);
    double dot = oracle_mx_dot(packed, scales, packed + COLS / 2, scales + COLS / 32, COLS);
    double ref = 0.0;
    for (int i = 0; i < COLS; ++i) ref += deq[i] * deq[COLS + i];
    CHECK(dot == ref);

    /* routing: invalid ids, duplicates, too small a capacity */
    enum { M = 13, K = 4, E = 5, BM = 16 };
    int32_t ids[M * K];
    float tw[M * K];
    for (int i = 0; i < M * K; ++i) {
        ids[i] = (int32_t)(rnd() % (E + 3)) - 1;
        tw[i] = (float)(rnd() % 100) / 100.0f;
    }
    ids[1] = ids[0];
    const int64_t cap = M * K + E * (BM - 1) + BM;
    int32_t sr[M * K + E * (BM - 1) + BM], be[(M * K + E * (BM - 1) + BM) / BM], nv[2];
    float sw[M * K + E * (BM - 1) + BM];
    CHECK(oracle_route(ids, tw, M, K, E, BM, sr, sw, be, nv, cap) == 0);
    CHECK(nv[0] % BM == 0 && nv[1] <= M * K);
    CHECK(oracle_route(ids, tw, M, K, E, BM, sr, sw, be, nv, 3) != 0);

    /* forward: closed form hidden == 2^-8, all weight codes 1.0 at scale 127:
     * h = bf16(silu(1)) requantized to 0.75, out = 0.75 * 256 = 192 */
    {
        const int D = 256, I = 256;
        uint16_t h[D];
        for (int i = 0; i < D; ++i) h[i] = bf16_bits_of(1.0f / 256.0f);
        uint8_t* w13 = malloc((size_t)2 * I * D / 2);
        uint8_t* w13s = malloc((size_t)2 * I * D / 32);
        uint8_t* w2 = malloc((size_t)D * I / 2);
        uint8_t* w2s = malloc((size_t)D * I / 32);
        memset(w13, 0x22, (size_t)2 * I * D / 2);
        memset(w13s, 127, (size_t)2 * I * D / 32);
        memset(w2, 0x22, (size_t)D * I / 2);
        memset(w2s, 127, (size_t)D * I / 32);
        int32_t id1 = 0;
        float w1 = 1.0f;
        uint16_t out[D], hout[I];
        double of[D];
        CHECK(oracle_forward(h, w13, w13s, w2, w2s, &id1, &w1, 1, D, I, 1, 1, NULL, 1, 1, 1,
                             out, of, hout) == 0);
        for (int d = 0; d < D; ++d) CHECK(of[d] == 192.0);
        free(w13);
        free(w13s);
        free(w2);
        free(w2s);
    }
    /* forward: random case, token subset, both activation modes, all outputs */
    {
        const int D = 256, I = 256, MM = 6, KK = 3, EE = 4;
        uint16_t* h = malloc(sizeof(uint16_t) * MM * D);
        for (int i = 0; i < MM * D; ++i) h[i] = bf16_bits_of((float)((int)(rnd() % 64) - 32) / 16.0f);
        size_t n13 = (size_t)EE * 2 * I * D / 2, n2 = (size_t)EE * D * I / 2;
        uint8_t* w13 = malloc(n13);
        uint8_t* w13s = malloc(n13 / 16);
        uint8_t* w2 = malloc(n2);
        uint8_t* w2s = malloc(n2 / 16);
        for (size_t i = 0; i < n13; ++i) w13[i] = (uint8_t)rnd();
        for (size_t i = 0; i < n13 / 16; ++i) w13s[i] = (uint8_t)(120 + rnd() % 6);
        for (size_t i = 0; i < n2; ++i) w2[i] = (uint8_t)rnd();
        for (size_t i = 0; i < n2 / 16; ++i) w2s[i] = (uint8_t)(120 + rnd() % 6);
        int32_t fid[MM * KK];
        float fw[MM * KK];
        for (int i = 0; i < MM * KK; ++i) {
            fid[i] = (int32_t)(rnd() % (EE + 2)) - 1;
            fw[i] = 0.5f;
        }
        int32_t toks[3] = {5, 0, 2};
        uint16_t* out = malloc(sizeof(uint16_t) * MM * D);
        double* of = malloc(sizeof(double) * MM * D);
        uint16_t* hout = malloc(sizeof(uint16_t) * MM * KK * I);
        uint16_t sub[3 * 256];
        for (int aq = 0; aq <= 1; ++aq) {
            CHECK(oracle_forward(h, w13, w13s, w2, w2s, fid, fw, MM, D, I, EE, KK, NULL, MM, aq, 3,
                                 out, of, hout) == 0);
            CHECK(oracle_forward(h, w13, w13s, w2, w2s, fid, fw, MM, D, I, EE, KK, toks, 3, aq, 2,
                                 sub, NULL, NULL) == 0);
            for (int j = 0; j < 3; ++j) CHECK(memcmp(sub + j * D, out + toks[j] * D, 2 * D) == 0);
        }
        CHECK(oracle_forward(h, w13, w13s, w2, w2s, fid, fw, MM, 100, I, EE, KK, NULL, MM, 1, 1,
                             out, NULL, NULL) != 0);
        free(h);
        free(w13);
        free(w13s);
        free(w2);
        free(w2s);
        free(out);
        free(of);
        free(hout);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
