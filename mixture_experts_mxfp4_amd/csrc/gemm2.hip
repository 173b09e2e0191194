// Stage 2: grouped down-projection GEMM on gfx950 block-scaled FP4 MFMA; the
// epilogue multiplies by the routing weight and accumulates per token.
//
// Semantics (kernelindex submission 754773: stage 2 receives the sorted
// routing weights and accumulates atomically, `mode: atomic`; kernelindex
// submission 723815 `_reference_forward`: out[t] += w * (act @ W_down^T)):
// y = Q(h) . down_row over K = I for each sorted row, then
// out[token, :] += sorted_w[row] * y.  Sums go to an fp32 accumulator with
// hardware fp32 atomics (the per-token order of the topk contributions is not
// fixed, every order is a valid fp32 sum); a final pass rounds once to bf16.
//
// Tiling: a workgroup (4 waves) owns one block of BM = 16*RT sorted rows and
// 256 output columns; each wave owns 64 columns = 4 MFMA tiles per row tile
// and runs the whole K = I loop, streaming 1 KiB weight fragments with
// non-temporal loads; the A fragments (h, already in MFMA fragment order from
// stage 1) are contiguous 1 KiB loads as well.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kGemmThreads = 256;

template <int RT, int G>
__global__ void __launch_bounds__(kGemmThreads)
gemm2_weighted_kernel(const uint8_t* __restrict__ a2q, const uint8_t* __restrict__ a2s,
                      const uint8_t* __restrict__ w2p, const uint8_t* __restrict__ w2sp,
                      const int32_t* __restrict__ sorted_route, const float* __restrict__ sorted_w,
                      const int32_t* __restrict__ block_expert,
                      const int32_t* __restrict__ num_valid, float* __restrict__ acc_out, int M,
                      int D, int I, int topk)
{
    constexpr int BM = 16 * RT;
    const int blk = blockIdx.y;
    if (blk * BM >= num_valid[0]) return;
    const int e = block_expert[blk];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int n64 = blockIdx.x * 4 + wave;
    const int KT = I / 128, NKG = KT / G;
    const int R = M * topk;

    const uint8_t* wb = w2p + int64_t(e) * D * (I / 2) + int64_t(n64) * KT * 4096 + lane * 16;
    const uint8_t* sb = w2sp + int64_t(e) * D * (I / 32) + int64_t(n64) * NKG * 256 * G + lane * G;
    const int64_t rowtile0 = int64_t(blk) * RT;

    v4f acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[rt][q] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kg = 0; kg < NKG; ++kg) {
        uint32_t sw[4], sa[RT];
#pragma unroll
        for (int q = 0; q < 4; ++q) sw[q] = ld_scales<G>(sb + (kg * 4 + q) * 64 * G);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            sa[rt] = ld_scales<G>(a2s + (((rowtile0 + rt) * NKG + kg) * 64 + lane) * G);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int kt = kg * G + j;
            uint4 b[4], a[RT];
#pragma unroll
            for (int q = 0; q < 4; ++q) b[q] = ld16_nt(wb + int64_t(kt * 4 + q) * 1024);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                a[rt] = ld16(a2q + (((rowtile0 + rt) * KT + kt) * 64 + lane) * 16);
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
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t srow = int64_t(blk) * BM + rt * 16 + 4 * (lane / 16) + i;
            const int sr = sorted_route[srow];
            if (sr < R) {
                const float w = sorted_w[srow];
                float* dst = acc_out + int64_t(sr / topk) * D + n64 * 64 + lane % 16;
#pragma unroll
                for (int q = 0; q < 4; ++q) unsafeAtomicAdd(dst + q * 16, w * acc[rt][q][i]);
            }
        }
    }
}

template <int RT, int G>
static hipError_t launch_g2(const Gemm2Args& a, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm2_weighted_kernel<RT, G>), dim3(a.D / 256, a.nb_cap),
                       dim3(kGemmThreads), 0, stream, a.a2q, a.a2s, a.w2p, a.w2sp, a.sorted_route,
                       a.sorted_w, a.block_expert, a.num_valid, a.acc, a.M, a.D, a.I, a.topk);
    return hipGetLastError();
}

hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t stream)
{
    if (a.nb_cap == 0) return hipSuccess;
    const bool g4 = (a.I % 512) == 0;
    switch (a.block_m) {
    case 16: return g4 ? launch_g2<1, 4>(a, stream) : launch_g2<1, 2>(a, stream);
    case 32: return g4 ? launch_g2<2, 4>(a, stream) : launch_g2<2, 2>(a, stream);
    case 64: return g4 ? launch_g2<4, 4>(a, stream) : launch_g2<4, 2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// fp32 accumulator -> bf16 output, one rounding (8 elements per thread).
__global__ void finalize_bf16_kernel(const float* __restrict__ acc, uint16_t* __restrict__ out,
                                     int64_t n8)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n8;
         i += int64_t(gridDim.x) * blockDim.x) {
        const float4 lo = reinterpret_cast<const float4*>(acc + i * 8)[0];
        const float4 hi = reinterpret_cast<const float4*>(acc + i * 8)[1];
        uint4 o;
        o.x = f32_to_bf16_rne(lo.x) | (f32_to_bf16_rne(lo.y) << 16);
        o.y = f32_to_bf16_rne(lo.z) | (f32_to_bf16_rne(lo.w) << 16);
        o.z = f32_to_bf16_rne(hi.x) | (f32_to_bf16_rne(hi.y) << 16);
        o.w = f32_to_bf16_rne(hi.z) | (f32_to_bf16_rne(hi.w) << 16);
        *reinterpret_cast<uint4*>(out + i * 8) = o;
    }
}

hipError_t launch_finalize(const float* acc, uint16_t* out, int64_t n, int n_cu,
                           hipStream_t stream)
{
    const int64_t n8 = n / 8;
    if (n8 == 0) return hipSuccess;
    int64_t blocks = (n8 + 255) / 256;
    if (blocks > int64_t(n_cu) * 16) blocks = int64_t(n_cu) * 16;
    hipLaunchKernelGGL(finalize_bf16_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, acc,
                       out, n8);
    return hipGetLastError();
}

}  // namespace moe
