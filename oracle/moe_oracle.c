/*
 * Plain CPU oracle for the fused MXFP4 Mixture-of-Experts forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * Everything is computed the slow, obvious way in fp64: every E2M1 / e8m0
 * value is decoded to a double, every dot product is a plain loop, every
 * (token, slot) pair is processed one after the other.
 *
 * Sources (the three web pages this work follows):
 *   [P1] kernelindex.com, amd-moe-mxfp4 submission 754773 ("flower_moe.py"):
 *        the FP4 pipeline quantizes the activations before stage 1, re-quantizes
 *        the bf16 SwiGLU output before stage 2, and applies the routing weight
 *        in stage 2 only (the `custom_kernel` FP4 branch; CK kernel name field
 *        MulRoutedWeight0; doweight_stage1=False).  Sorting workspace sizes
 *        (sorted ids / weights / per-block expert ids / num_valid).
 *   [P2] kernelindex.com, amd-moe-mxfp4 submission 723815 ("solution.py"):
 *        the E2M1 and e8m0 device decoders, `_dequant` (low nibble first,
 *        2^(s-127) per 32 along the last dimension), `_reference_forward`
 *        (gate rows 0..I-1, up rows I..2I-1, silu(gate)*up, per (token, slot)
 *        loop), invalid expert ids skipped by the routing kernels.
 *   OCP Microscaling Formats (MX) v1.0: scale = 2^(floor(log2(amax)) - emax)
 *        with emax = 2 for E2M1, round-to-nearest-even, saturating.
 *
 * Readings where the pages are silent are listed next to the code that
 * takes them; the full list is kept with the design notes.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

/* ------------------------------------------------------------------------- */
/* Element decoders                                                          */
/* ------------------------------------------------------------------------- */

/* E2M1 code -> value.  [P2] device decoder `fp4_to_f32`: sign is bit 3, the
 * exponent is bits 2..1, the mantissa is bit 0; exponent 0 is subnormal
 * (mant * 0.5), otherwise (1 + mant * 0.5) * 2^(exp - 1). */
double oracle_e2m1_value(int code)
{
    int sign = (code >> 3) & 1;
    int exp = (code >> 1) & 3;
    int mant = code & 1;
    double v = (exp == 0) ? mant * 0.5 : (1.0 + mant * 0.5) * ldexp(1.0, exp - 1);
    return sign ? -v : v;
}

/* e8m0 scale byte -> 2^(s - 127).  [P2] `e8m0_to_f32`.  The byte 255 is NaN
 * in the OCP MX definition; the pages never produce it. */
double oracle_e8m0_value(int s)
{
    if (s == 255) return NAN;
    return ldexp(1.0, s - 127);
}

double oracle_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to bfloat16, round-to-nearest-even, directly from the double
 * (no detour through float, which would round twice). */
uint16_t oracle_bf16_round(double x)
{
    if (isnan(x)) return 0x7FC0;
    int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint16_t sign = (uint16_t)(neg << 15);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                /* floor(log2 a) */
    double quantum = (e < -126) ? ldexp(1.0, -133) : ldexp(1.0, e - 7);
    double n = nearbyint(a / quantum);   /* ties to even in the default mode */
    double r = n * quantum;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)r;            /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* ------------------------------------------------------------------------- */
/* MXFP4 quantization of one 32-element block (OCP MX v1.0)                  */
/* ------------------------------------------------------------------------- */

static const double kE2M1Grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Nearest grid point to v >= 0; on a tie the point with the even index (even
 * mantissa bit) wins; anything above the largest point saturates to it. */
static int e2m1_nearest_index(double v)
{
    if (v >= kE2M1Grid[7]) return 7;
    int best = 0;
    double best_d = fabs(v - kE2M1Grid[0]);
    for (int j = 1; j < 8; ++j) {
        double d = fabs(v - kE2M1Grid[j]);
        if (d < best_d || (d == best_d && (j % 2 == 0) && (best % 2 == 1))) {
            best = j;
            best_d = d;
        }
    }
    return best;
}

/* x: 32 doubles (exact bf16 values).  codes: 32 unpacked E2M1 codes.
 * Scale rule: X = 2^(floor(log2(amax)) - 2), 2 being the largest E2M1
 * exponent (6 = 1.5 * 2^2); the e8m0 byte is clamped to [0, 254]; an all-zero
 * block gets byte 0.  Each element is divided by X (exact: a power of two)
 * and rounded to nearest even onto the E2M1 grid, saturating at 6.  The sign
 * is kept, so a negative value that rounds to zero gives code 0x8. */
void oracle_mx_quant_block_f64(const double* x, uint8_t* codes, uint8_t* scale)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs(x[i]);
        if (a > amax) amax = a;
    }
    int s;
    if (amax == 0.0) {
        s = 0;
    } else {
        int ex;
        frexp(amax, &ex);
        int e = ex - 1;                  /* floor(log2 amax), exact */
        s = e - 2 + 127;
        if (s < 0) s = 0;
        if (s > 254) s = 254;
    }
    double X = ldexp(1.0, s - 127);
    for (int i = 0; i < 32; ++i) {
        double v = fabs(x[i]) / X;
        int idx = e2m1_nearest_index(v);
        int neg = signbit(x[i]) ? 1 : 0;
        codes[i] = (uint8_t)((neg << 3) | idx);
    }
    *scale = (uint8_t)s;
}

void oracle_mx_quant_block_bf16(const uint16_t* x, uint8_t* codes, uint8_t* scale)
{
    double v[32];
    for (int i = 0; i < 32; ++i) v[i] = oracle_bf16_value(x[i]);
    oracle_mx_quant_block_f64(v, codes, scale);
}

/* Pack 2 codes per byte: element 2j in the low nibble, 2j+1 in the high
 * nibble ([P2] `_dequant` unpacks low then high). */
static void pack_codes(const uint8_t* codes, int n, uint8_t* packed)
{
    for (int j = 0; j < n / 2; ++j)
        packed[j] = (uint8_t)((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4));
}

static int unpack_code(const uint8_t* packed, int64_t i)
{
    uint8_t b = packed[i >> 1];
    return (i & 1) ? (b >> 4) : (b & 0xF);
}

/* ------------------------------------------------------------------------- */
/* Threads                                                                   */
/* ------------------------------------------------------------------------- */

typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end);

typedef struct {
    range_fn fn;
    void* ctx;
    int64_t begin, end;
} range_job;

static void* run_range(void* p)
{
    range_job* j = (range_job*)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

/* Split [0, n) into contiguous pieces, one per thread. */
static void parallel_for(int64_t n, int nthreads, range_fn fn, void* ctx)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t th[256];
    range_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = n * t / nthreads;
        jobs[t].end = n * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, run_range, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------- */
/* Row quantization (weights and activations alike)                          */
/* ------------------------------------------------------------------------- */

typedef struct {
    const uint16_t* x;
    int64_t cols;
    uint8_t* packed;
    uint8_t* scales;
} quant_ctx;

static void quant_rows_range(void* p, int64_t r0, int64_t r1)
{
    quant_ctx* c = (quant_ctx*)p;
    uint8_t codes[32];
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t b = 0; b < c->cols / 32; ++b) {
            const uint16_t* src = c->x + r * c->cols + b * 32;
            oracle_mx_quant_block_bf16(src, codes, &c->scales[r * (c->cols / 32) + b]);
            pack_codes(codes, 32, c->packed + r * (c->cols / 2) + b * 16);
        }
    }
}

/* x: bf16 [rows, cols] row-major, cols % 32 == 0.
 * packed: [rows, cols/2] codes; scales: [rows, cols/32] e8m0 bytes. */
int oracle_mx_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols,
                            uint8_t* packed, uint8_t* scales, int nthreads)
{
    if (cols % 32 != 0 || rows < 0) return 1;
    quant_ctx c = {x, cols, packed, scales};
    parallel_for(rows, nthreads, quant_rows_range, &c);
    return 0;
}

/* Dequantize [rows, cols] MXFP4 back to doubles. */
int oracle_mx_dequantize_rows(const uint8_t* packed, const uint8_t* scales,
                              int64_t rows, int64_t cols, double* out)
{
    if (cols % 32 != 0) return 1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < cols; ++i)
            out[r * cols + i] = oracle_e2m1_value(unpack_code(packed + r * (cols / 2), i)) *
                                oracle_e8m0_value(scales[r * (cols / 32) + i / 32]);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Block-scaled dot product                                                  */
/* ------------------------------------------------------------------------- */

/* sum over the K/32 blocks of  (sum_j e2m1(a_j) * e2m1(w_j)) * 2^(sa-127) * 2^(sw-127).
 * The inner sum is exact in a double (multiples of 0.25, |sum| <= 1152). */
double oracle_mx_dot(const uint8_t* a_packed, const uint8_t* a_scales,
                     const uint8_t* w_packed, const uint8_t* w_scales, int64_t K)
{
    double total = 0.0;
    for (int64_t b = 0; b < K / 32; ++b) {
        double block = 0.0;
        for (int j = 0; j < 32; ++j) {
            int64_t i = b * 32 + j;
            block += oracle_e2m1_value(unpack_code(a_packed, i)) *
                     oracle_e2m1_value(unpack_code(w_packed, i));
        }
        total += block * oracle_e8m0_value(a_scales[b]) * oracle_e8m0_value(w_scales[b]);
    }
    return total;
}

/* ------------------------------------------------------------------------- */
/* Routing: expert-sorted, block-padded route lists                          */
/* ------------------------------------------------------------------------- */

/* A route is r = t*k + s (token t, slot s).  For every expert e in ascending
 * order, its routes in ascending r, then padding up to a multiple of bm
 * (padding route id M*k, weight 0).  Experts without routes get no rows.
 * block_expert[b] is the expert of rows [b*bm, (b+1)*bm).
 * num_valid[0] = padded rows, num_valid[1] = valid routes.
 * Ids outside [0, E) are skipped ([P2] routing kernels).
 * Returns 1 if cap is too small for the padded list. */
int oracle_route(const int32_t* ids, const float* tw, int M, int k, int E, int bm,
                 int32_t* sorted_route, float* sorted_w, int32_t* block_expert,
                 int32_t* num_valid, int64_t cap)
{
    int64_t R = (int64_t)M * k;
    int64_t pos = 0, valid = 0;
    for (int e = 0; e < E; ++e) {
        int64_t n = 0;
        for (int64_t r = 0; r < R; ++r) {
            if (ids[r] != e) continue;
            if (pos >= cap) return 1;
            sorted_route[pos] = (int32_t)r;
            sorted_w[pos] = tw[r];
            ++pos;
            ++n;
        }
        valid += n;
        while (n % bm != 0) {
            if (pos >= cap) return 1;
            sorted_route[pos] = (int32_t)R;
            sorted_w[pos] = 0.0f;
            ++pos;
            ++n;
        }
        for (int64_t b = (pos - n) / bm; b < pos / bm; ++b) block_expert[b] = e;
    }
    num_valid[0] = (int32_t)pos;
    num_valid[1] = (int32_t)valid;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Forward                                                                   */
/* ------------------------------------------------------------------------- */

typedef struct {
    const uint16_t* hidden;
    const uint8_t *w13, *w13s, *w2, *w2s;
    const int32_t* ids;
    const float* tw;
    int M, D, I, E, k, act_quant;
    const int32_t* tokens;
    uint16_t* out;
    double* out_f64;
    uint16_t* h_out; /* optional [ntok, k, I] bf16 */
} fwd_ctx;

static double silu(double g) { return g / (1.0 + exp(-g)); }

static void forward_range(void* p, int64_t i0, int64_t i1)
{
    fwd_ctx* c = (fwd_ctx*)p;
    const int D = c->D, I = c->I;
    uint8_t* a1q = (uint8_t*)malloc((size_t)D / 2);
    uint8_t* a1s = (uint8_t*)malloc((size_t)D / 32);
    double* a1f = (double*)malloc(sizeof(double) * (size_t)D);   /* act_quant off */
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
    uint8_t* a2q = (uint8_t*)malloc((size_t)I / 2);
    uint8_t* a2s = (uint8_t*)malloc((size_t)I / 32);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    uint8_t codes[32];

    const int64_t w13_row = D / 2, w13s_row = D / 32;
    const int64_t w2_row = I / 2, w2s_row = I / 32;
    const int64_t w13_e = (int64_t)2 * I * w13_row, w13s_e = (int64_t)2 * I * w13s_row;
    const int64_t w2_e = (int64_t)D * w2_row, w2s_e = (int64_t)D * w2s_row;

    for (int64_t i = i0; i < i1; ++i) {
        int t = c->tokens ? c->tokens[i] : (int)i;
        const uint16_t* x = c->hidden + (int64_t)t * D;

        /* Step 1: quantize the token's activation row per 32 along D [P1]. */
        for (int b = 0; b < D / 32; ++b) {
            oracle_mx_quant_block_bf16(x + b * 32, codes, &a1s[b]);
            pack_codes(codes, 32, a1q + b * 16);
        }
        for (int d = 0; d < D; ++d) a1f[d] = oracle_bf16_value(x[d]);
        for (int d = 0; d < D; ++d) acc[d] = 0.0;

        for (int s = 0; s < c->k; ++s) {
            int64_t r = (int64_t)t * c->k + s;
            int e = c->ids[r];
            if (e < 0 || e >= c->E) continue;      /* [P2]: invalid ids skipped */
            double w = (double)c->tw[r];
            const uint8_t* we13 = c->w13 + e * w13_e;
            const uint8_t* se13 = c->w13s + e * w13s_e;
            const uint8_t* we2 = c->w2 + e * w2_e;
            const uint8_t* se2 = c->w2s + e * w2s_e;

            /* Step 2: gate row n and up row I+n [P2 `_reference_forward`],
             * h = bf16(silu(g) * u) (bf16 intermediate, [P1] a2 buffer). */
            for (int n = 0; n < I; ++n) {
                double g, u;
                if (c->act_quant) {
                    g = oracle_mx_dot(a1q, a1s, we13 + n * w13_row, se13 + n * w13s_row, D);
                    u = oracle_mx_dot(a1q, a1s, we13 + (int64_t)(I + n) * w13_row,
                                      se13 + (int64_t)(I + n) * w13s_row, D);
                } else {
                    g = 0.0;
                    u = 0.0;
                    for (int d = 0; d < D; ++d) {
                        double wg = oracle_e2m1_value(unpack_code(we13 + n * w13_row, d)) *
                                    oracle_e8m0_value(se13[n * w13s_row + d / 32]);
                        double wu = oracle_e2m1_value(unpack_code(we13 + (int64_t)(I + n) * w13_row, d)) *
                                    oracle_e8m0_value(se13[(int64_t)(I + n) * w13s_row + d / 32]);
                        g += a1f[d] * wg;
                        u += a1f[d] * wu;
                    }
                }
                h[n] = oracle_bf16_round(silu(g) * u);
            }
            if (c->h_out) memcpy(c->h_out + ((int64_t)i * c->k + s) * I, h, sizeof(uint16_t) * I);

            /* Step 3: re-quantize h per 32 along I [P1 inter-stage quant]. */
            if (c->act_quant) {
                for (int b = 0; b < I / 32; ++b) {
                    oracle_mx_quant_block_bf16(h + b * 32, codes, &a2s[b]);
                    pack_codes(codes, 32, a2q + b * 16);
                }
            }

            /* Step 4: down projection, weighted by the routing weight (stage 2
             * only [P1]), accumulated over the slots in fp64. */
            for (int d = 0; d < D; ++d) {
                double y;
                if (c->act_quant) {
                    y = oracle_mx_dot(a2q, a2s, we2 + d * w2_row, se2 + d * w2s_row, I);
                } else {
                    y = 0.0;
                    for (int n = 0; n < I; ++n)
                        y += oracle_bf16_value(h[n]) *
                             oracle_e2m1_value(unpack_code(we2 + d * w2_row, n)) *
                             oracle_e8m0_value(se2[d * w2s_row + n / 32]);
                }
                acc[d] += w * y;
            }
        }
        /* One rounding to bf16 at the end. */
        for (int d = 0; d < D; ++d) {
            c->out[(int64_t)i * D + d] = oracle_bf16_round(acc[d]);
            if (c->out_f64) c->out_f64[(int64_t)i * D + d] = acc[d];
        }
    }
    free(a1q);
    free(a1s);
    free(a1f);
    free(h);
    free(a2q);
    free(a2s);
    free(acc);
}

int oracle_forward(const uint16_t* hidden, const uint8_t* w13, const uint8_t* w13s,
                   const uint8_t* w2, const uint8_t* w2s, const int32_t* ids, const float* tw,
                   int M, int D, int I, int E, int k, const int32_t* tokens, int ntok,
                   int act_quant, int nthreads, uint16_t* out, double* out_f64, uint16_t* h_out)
{
    if (M < 0 || D <= 0 || I <= 0 || E <= 0 || k <= 0) return 1;
    if (D % 32 != 0 || I % 32 != 0) return 1;
    if (tokens) {
        for (int i = 0; i < ntok; ++i)
            if (tokens[i] < 0 || tokens[i] >= M) return 1;
    } else {
        ntok = M;
    }
    fwd_ctx c = {hidden, w13, w13s, w2, w2s, ids, tw, M, D, I, E, k, act_quant,
                 tokens, out, out_f64, h_out};
    parallel_for(ntok, nthreads, forward_range, &c);
    return 0;
}
