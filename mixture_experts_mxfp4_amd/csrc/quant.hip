// Dynamic MXFP4 quantization of bf16 rows (OCP MX v1.0, RNE, saturating).
//
// The pipeline of kernelindex submission 754773 quantizes the hidden states
// per 32 elements before the gate_up GEMM (`_flower_fused_quant`, FP4 branch).
// Here four lanes own one 32-element block (8 bf16 = 16 bytes each); the block
// maximum is reduced across the four lanes, each lane writes 4 code bytes and
// the first lane the scale byte.  The same pass optionally clears an fp32
// buffer of the same element count (the stage-2 accumulator), so the forward
// needs no separate memset.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kQuantThreads = 256;

// scale_G = 0: scales row-major [rows][cols/32]; otherwise the grouped
// activation layout of act_scale_pos(., scale_G).
__global__ void __launch_bounds__(kQuantThreads)
quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int scale_G,
                  float* __restrict__ zero_f32)
{
    const int64_t chunks_per_row = cols / 8;
    const int64_t n_chunks = rows * chunks_per_row;
    const int64_t stride = int64_t(gridDim.x) * kQuantThreads;
    for (int64_t i0 = int64_t(blockIdx.x) * kQuantThreads; i0 < n_chunks; i0 += stride) {
        const int64_t i = i0 + threadIdx.x;
        const bool in = i < n_chunks;          // whole 4-lane groups are in or out
        uint4 v = in ? *reinterpret_cast<const uint4*>(x + i * 8) : make_uint4(0, 0, 0, 0);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            amax = max(amax, w[j] & 0x7FFFu);
            amax = max(amax, (w[j] >> 16) & 0x7FFFu);
        }
        amax = max(amax, uint32_t(__shfl_xor(int(amax), 1)));
        amax = max(amax, uint32_t(__shfl_xor(int(amax), 2)));
        const uint32_t s = mx_scale_from_amax(amax);
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t c0 = mx_code(w[j] & 0xFFFFu, s), c1 = mx_code(w[j] >> 16, s);
            packed |= (c0 | (c1 << 4)) << (8 * j);
        }
        if (in) {
            reinterpret_cast<uint32_t*>(codes)[i] = packed;
            if ((i & 3) == 0) {
                const int64_t row = i / chunks_per_row;
                const int kb = int((i % chunks_per_row) / 4);
                const int64_t kbs = cols / 32;
                const int pos = scale_G ? act_scale_pos(kb, scale_G) : kb;
                scales[row * kbs + pos] = uint8_t(s);
            }
            if (zero_f32) {
                float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                reinterpret_cast<float4*>(zero_f32 + i * 8)[0] = z;
                reinterpret_cast<float4*>(zero_f32 + i * 8)[1] = z;
            }
        }
    }
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                             uint8_t* scales, int scale_G, float* zero_f32, int n_cu,
                             hipStream_t stream)
{
    const int64_t n_chunks = rows * (cols / 8);
    if (n_chunks == 0) return hipSuccess;
    int64_t blocks = (n_chunks + kQuantThreads - 1) / kQuantThreads;
    const int64_t max_blocks = int64_t(n_cu) * 16;
    if (blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL(quant_rows_kernel, dim3(unsigned(blocks)), dim3(kQuantThreads), 0,
                       stream, x, rows, cols, codes, scales, scale_G, zero_f32);
    return hipGetLastError();
}

}  // namespace moe
