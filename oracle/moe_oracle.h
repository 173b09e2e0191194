/*
 * Plain CPU oracle for the fused MXFP4 MoE forward -- TEST INFRASTRUCTURE ONLY.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * Shares nothing with the HIP library.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double oracle_e2m1_value(int code);
double oracle_e8m0_value(int s);
double oracle_bf16_value(uint16_t b);
uint16_t oracle_bf16_round(double x);

void oracle_mx_quant_block_f64(const double* x, uint8_t* codes, uint8_t* scale);
void oracle_mx_quant_block_bf16(const uint16_t* x, uint8_t* codes, uint8_t* scale);
int oracle_mx_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols,
                            uint8_t* packed, uint8_t* scales, int nthreads);
int oracle_mx_dequantize_rows(const uint8_t* packed, const uint8_t* scales,
                              int64_t rows, int64_t cols, double* out);
double oracle_mx_dot(const uint8_t* a_packed, const uint8_t* a_scales,
                     const uint8_t* w_packed, const uint8_t* w_scales, int64_t K);

int oracle_route(const int32_t* ids, const float* tw, int M, int k, int E, int bm,
                 int32_t* sorted_route, float* sorted_w, int32_t* block_expert,
                 int32_t* num_valid, int64_t cap);

int oracle_forward(const uint16_t* hidden, const uint8_t* w13, const uint8_t* w13s,
                   const uint8_t* w2, const uint8_t* w2s, const int32_t* ids, const float* tw,
                   int M, int D, int I, int E, int k, const int32_t* tokens, int ntok,
                   int act_quant, int nthreads, uint16_t* out, double* out_f64,
                   uint16_t* h_out);

#ifdef __cplusplus
}
#endif

#endif
