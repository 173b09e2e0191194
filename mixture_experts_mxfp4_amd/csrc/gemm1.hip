// Stage 1: grouped gate_up GEMM on gfx950 block-scaled FP4 MFMA with a fused
// SwiGLU and MXFP4 re-quantization epilogue.
//
// Semantics (kernelindex submission 754773, FP4 branch of `custom_kernel`;
// kernelindex submission 723815, `_reference_forward`): for every row of the
// expert-sorted route list, g = Q(x) . gate_row and u = Q(x) . up_row over
// K = D, h = bf16(silu(g) * u) (the stage-1 kernel of 754773 writes a bf16
// intermediate, `..._silu_FP4X2_FP4X2_B16`, and does not apply the routing
// weight, `MulRoutedWeight0`), then h is quantized to MXFP4 per 32 columns
// exactly as the inter-stage quant of 754773 does, so stage 2 reads FP4.
//
// Tiling: a workgroup (4 waves) owns one block of BM = 16*RT sorted rows (one
// expert) and one 64-row group of the prepared gate_up weight = 32 gate + 32
// up columns = one MXFP4 group of h.  The four waves split the K dimension;
// each wave runs RT x 4 MFMA tiles of 16x16x128, streaming its weight
// fragments (1 KiB each, contiguous) with non-temporal loads and gathering the
// block's activation rows by token id.  Partial sums meet in LDS; the epilogue
// quantizes h with cross-lane reductions and writes it in the fragment order
// that stage 2 loads directly.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kGemmThreads = 256;

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

template <int RT, int G>
__global__ void __launch_bounds__(kGemmThreads)
gemm1_swiglu_quant_kernel(const uint8_t* __restrict__ a1q, const uint8_t* __restrict__ a1s,
                          const uint8_t* __restrict__ w13p, const uint8_t* __restrict__ w13sp,
                          const int32_t* __restrict__ sorted_route,
                          const int32_t* __restrict__ block_expert,
                          const int32_t* __restrict__ num_valid, uint8_t* __restrict__ a2q,
                          uint8_t* __restrict__ a2s, uint16_t* __restrict__ h_dbg, int M, int D,
                          int I, int topk)
{
    constexpr int BM = 16 * RT;
    __shared__ float red[4][RT][4][4][kWave];   // [wave][row tile][slice][i][lane]

    const int c = blockIdx.x;          // MXFP4 group of h = 64-row group of w13p
    const int blk = blockIdx.y;
    if (blk * BM >= num_valid[0]) return;
    const int e = block_expert[blk];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int R = M * topk;
    const int KT = D / 128, NKG = KT / G;
    const int64_t a_row = D / 2, as_row = D / 32;

    const uint8_t* a_ptr[RT];
    const uint8_t* as_ptr[RT];
    bool ok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        int sr = sorted_route[blk * BM + rt * 16 + lane % 16];
        ok[rt] = sr < R;
        int64_t tok = ok[rt] ? sr / topk : 0;
        a_ptr[rt] = a1q + tok * a_row + (lane / 16) * 16;
        as_ptr[rt] = a1s + tok * as_row + (lane / 16) * G;
    }
    const uint8_t* wb = w13p + int64_t(e) * (2 * I) * a_row + int64_t(c) * KT * 4096 + lane * 16;
    const uint8_t* sb = w13sp + int64_t(e) * (2 * I) * as_row + int64_t(c) * NKG * 256 * G + lane * G;

    v4f acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[rt][q] = v4f{0.f, 0.f, 0.f, 0.f};

    const int kg0 = wave * NKG / 4, kg1 = (wave + 1) * NKG / 4;
    for (int kg = kg0; kg < kg1; ++kg) {
        uint32_t sw[4], sa[RT];
#pragma unroll
        for (int q = 0; q < 4; ++q) sw[q] = ld_scales<G>(sb + (kg * 4 + q) * 64 * G);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sa[rt] = ok[rt] ? ld_scales<G>(as_ptr[rt] + kg * 4 * G) : 0u;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int kt = kg * G + j;
            uint4 b[4], a[RT];
#pragma unroll
            for (int q = 0; q < 4; ++q) b[q] = ld16_nt(wb + int64_t(kt * 4 + q) * 1024);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                a[rt] = ok[rt] ? ld16(a_ptr[rt] + kt * 64) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[rt][q] = mfma_fp4_16x16x128(a[rt], b[q], acc[rt][q],
                                                    (sa[rt] >> (8 * j)) & 0xFFu,
                                                    (sw[q] >> (8 * j)) & 0xFFu);
        }
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][rt][q][i][lane] = acc[rt][q][i];
    __syncthreads();

    const int KT2 = I / 128;
    const int G2 = (I % 512 == 0) ? 4 : 2;
    for (int rt = wave; rt < RT; rt += 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                s4[q] = red[0][rt][q][i][lane] + red[1][rt][q][i][lane] +
                        red[2][rt][q][i][lane] + red[3][rt][q][i][lane];
            // slices 0,1 = gate columns c*32 + lane%16 (+16), slices 2,3 = up
            const uint32_t h0 = f32_to_bf16_rne(silu_f32(s4[0]) * s4[2]);
            const uint32_t h1 = f32_to_bf16_rne(silu_f32(s4[1]) * s4[3]);
            const int row = 4 * (lane / 16) + i;                  // row within the tile
            const int64_t srow = int64_t(blk) * BM + rt * 16 + row;  // sorted row
            if (h_dbg) {
                h_dbg[srow * I + c * 32 + lane % 16] = uint16_t(h0);
                h_dbg[srow * I + c * 32 + 16 + lane % 16] = uint16_t(h1);
            }
            // MXFP4 group = the 32 columns held by the 16 lanes of this row
            uint32_t amax = max(h0 & 0x7FFFu, h1 & 0x7FFFu);
            amax = max(amax, uint32_t(__shfl_xor(int(amax), 1)));
            amax = max(amax, uint32_t(__shfl_xor(int(amax), 2)));
            amax = max(amax, uint32_t(__shfl_xor(int(amax), 4)));
            amax = max(amax, uint32_t(__shfl_xor(int(amax), 8)));
            const uint32_t s = mx_scale_from_amax(amax);
            const uint32_t c0 = mx_code(h0, s), c1 = mx_code(h1, s);
            // bytes: element 2b in the low nibble, 2b+1 in the high nibble
            const uint32_t o0 = uint32_t(__shfl_xor(int(c0), 1));
            const uint32_t o1 = uint32_t(__shfl_xor(int(c1), 1));
            const uint32_t blo = c0 | (o0 << 4), bhi = c1 | (o1 << 4);
            const uint32_t plo = blo | (uint32_t(__shfl_down(int(blo), 2)) << 8);
            const uint32_t phi = bhi | (uint32_t(__shfl_down(int(bhi), 2)) << 8);
            const uint32_t qlo = plo | (uint32_t(__shfl_down(int(plo), 4)) << 16);
            const uint32_t qhi = phi | (uint32_t(__shfl_down(int(phi), 4)) << 16);
            const uint32_t d1 = uint32_t(__shfl_down(int(qlo), 8));
            const uint32_t d3 = uint32_t(__shfl_down(int(qhi), 8));
            if (lane % 16 == 0) {
                const int64_t rowtile = int64_t(blk) * RT + rt;
                const int kt2 = c / 4;
                const int L = (c % 4) * 16 + row;
                *reinterpret_cast<uint4*>(a2q + ((rowtile * KT2 + kt2) * 64 + L) * 16) =
                    make_uint4(qlo, d1, qhi, d3);
                a2s[((rowtile * (KT2 / G2) + kt2 / G2) * 64 + L) * G2 + kt2 % G2] = uint8_t(s);
            }
        }
    }
}

template <int RT, int G>
static hipError_t launch_g1(const Gemm1Args& a, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm1_swiglu_quant_kernel<RT, G>), dim3(a.I / 32, a.nb_cap),
                       dim3(kGemmThreads), 0, stream, a.a1q, a.a1s, a.w13p, a.w13sp,
                       a.sorted_route, a.block_expert, a.num_valid, a.a2q, a.a2s, a.h_dbg, a.M,
                       a.D, a.I, a.topk);
    return hipGetLastError();
}

hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t stream)
{
    if (a.nb_cap == 0) return hipSuccess;
    const bool g4 = (a.D % 512) == 0;
    switch (a.block_m) {
    case 16: return g4 ? launch_g1<1, 4>(a, stream) : launch_g1<1, 2>(a, stream);
    case 32: return g4 ? launch_g1<2, 4>(a, stream) : launch_g1<2, 2>(a, stream);
    case 64: return g4 ? launch_g1<4, 4>(a, stream) : launch_g1<4, 2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// Fragment-order a2 (codes + scales) -> canonical row-major [cap][I/2], [cap][I/32].
__global__ void a2_to_canonical_kernel(const uint8_t* __restrict__ a2q,
                                       const uint8_t* __restrict__ a2s, int64_t rows, int I,
                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int ng = I / 32, KT2 = I / 128, G2 = (I % 512 == 0) ? 4 : 2;
    const int64_t n = rows * ng;
    for (int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < n;
         idx += int64_t(gridDim.x) * blockDim.x) {
        const int64_t row = idx / ng;
        const int c = int(idx % ng);
        const int64_t rowtile = row / 16;
        const int kt2 = c / 4, L = (c % 4) * 16 + int(row % 16);
        const uint4 v = ld16(a2q + ((rowtile * KT2 + kt2) * 64 + L) * 16);
        if (codes) *reinterpret_cast<uint4*>(codes + row * (I / 2) + c * 16) = v;
        if (scales)
            scales[row * ng + c] = a2s[((rowtile * (KT2 / G2) + kt2 / G2) * 64 + L) * G2 + kt2 % G2];
    }
}

hipError_t launch_a2_to_canonical(const uint8_t* a2q, const uint8_t* a2s, int64_t rows, int I,
                                  uint8_t* codes, uint8_t* scales, hipStream_t stream)
{
    const int64_t n = rows * (I / 32);
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(a2_to_canonical_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, a2q,
                       a2s, rows, I, codes, scales);
    return hipGetLastError();
}

}  // namespace moe
