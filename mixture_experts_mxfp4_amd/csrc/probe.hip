// Register-only rate probe of the gfx950 block-scaled FP4 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, or v_mfma_scale_f32_16x16x128_f8f6f4;
// both operands E2M1): what the matrix cores sustain with no memory traffic
// at all, the practical ceiling against which the LDS-tiled GEMMs' rate is
// read.  The published dense MXFP4 peak assumes every SIMD issuing one
// 32x32x64 MFMA per 32 cycles at 2.4 GHz; the probe reports the rate it
// reaches, the shader clock it ran at (the cycle counter against the
// constant-rate real-time clock) and the share of that per-clock FP4 rate,
// for operands with random bits (as real weights and activations have) or
// with a single set bit per 32-bit word.
#include <vector>

#include "moe_common.h"
#include "probe.h"

namespace moe {

constexpr int kProbeThreads = 256;      // four waves; two workgroups per CU

// Independent accumulator chains per wave: four 32x32 tiles, or eight 16x16
// tiles (the same accumulator registers).
template <bool kSmall>
constexpr int probe_chains() { return kSmall ? 8 : 4; }

template <bool kSmall>
__global__ void __launch_bounds__(kProbeThreads)
mfma_probe_kernel(int iters, int random_ops, uint64_t* __restrict__ rec, float* __restrict__ sink)
{
    constexpr int kProbeChains = probe_chains<kSmall>();
    constexpr int kAcc = kSmall ? 4 : 16;                 // accumulators per lane and tile
    typedef float acc_t __attribute__((ext_vector_type(kAcc)));
    const int lane = threadIdx.x % kWave;
    const int gw = blockIdx.x * (kProbeThreads / kWave) + threadIdx.x / kWave;
    v8i a[kProbeChains], b[kProbeChains];
    uint32_t x = 0x9E3779B9u * uint32_t(gw * kWave + lane + 1);
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t va = 0, vb = 0;
            if (k < 4) {                 // an FP4 operand of either shape is the low four words
                if (random_ops) {
                    x ^= x << 13; x ^= x >> 17; x ^= x << 5;
                    va = x;
                    x ^= x << 13; x ^= x >> 17; x ^= x << 5;
                    vb = x;
                } else {
                    va = 1u;             // E2M1 code 1 (0.5) in one nibble, zeros elsewhere
                    vb = 1u;
                }
            }
            a[c][k] = int(va);
            b[c][k] = int(vb);
        }
    }
    acc_t acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int i = 0; i < kAcc; ++i) acc[c][i] = 0.0f;

    const uint64_t t0 = uint64_t(wall_clock64());
    const uint64_t c0 = uint64_t(clock64());
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) {
            if constexpr (kSmall)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[c], b[c], acc[c], 4, 4, 0, 127, 0,
                                                                         127);
            else
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c], b[c], acc[c], 4, 4, 0, 127, 0,
                                                                         127);
        }
    }
    const uint64_t c1 = uint64_t(clock64());
    const uint64_t t1 = uint64_t(wall_clock64());

    // keep every chain's result live
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int i = 0; i < kAcc; ++i) s += acc[c][i];
    if (s == 1.2345f) sink[gw] = s;
    if (lane == 0) {
        rec[2 * gw] = t1 - t0;
        rec[2 * gw + 1] = c1 - c0;
    }
}

// One block-scaled FP4 MFMA on given operands, one wave: the unit check of
// the operand, scale and result layouts every GEMM kernel here relies on.  A
// and B are R x K E2M1 codes (two per byte, element 2j in the low nibble) with
// one e8m0 scale per 32 elements, R x K = 16 x 128 (16x16x128) or 32 x 64
// (32x32x64); lane l holds row l % R and 32-element chunk l / R of each.
// The lane's scale byte goes into byte SEL of a 32-bit word whose other bytes
// are 0xFF (the e8m0 NaN), so a wrong byte select gives NaN.  out[i][j] =
// sum_k A[i][k] B[j][k] (fp32, row-major R x R): the first operand's rows
// run down the result, the second's across.
template <int R, int SEL>
__global__ void __launch_bounds__(kWave)
mfma_unit_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
                 const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs, float* __restrict__ out)
{
    constexpr int K = R == 16 ? 128 : 64;
    const int lane = threadIdx.x;
    const int row = lane % R, chunk = lane / R;
    const uint4 av = *reinterpret_cast<const uint4*>(a + row * (K / 2) + chunk * 16);
    const uint4 bv = *reinterpret_cast<const uint4*>(b + row * (K / 2) + chunk * 16);
    const uint32_t fill = ~(0xFFu << (8 * SEL));
    const uint32_t sa = fill | (uint32_t(as[row * (K / 32) + chunk]) << (8 * SEL));
    const uint32_t sb = fill | (uint32_t(bs[row * (K / 32) + chunk]) << (8 * SEL));
    const v8i A = {int(av.x), int(av.y), int(av.z), int(av.w), 0, 0, 0, 0};
    const v8i B = {int(bv.x), int(bv.y), int(bv.z), int(bv.w), 0, 0, 0, 0};
    if constexpr (R == 16) {
        v4f c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, SEL, int(sa), SEL, int(sb));
#pragma unroll
        for (int i = 0; i < 4; ++i) out[(4 * (lane / 16) + i) * 16 + lane % 16] = c[i];
    } else {
        v16f c;
#pragma unroll
        for (int i = 0; i < 16; ++i) c[i] = 0.f;
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, SEL, int(sa), SEL, int(sb));
#pragma unroll
        for (int i = 0; i < 16; ++i) out[((i / 4) * 8 + (lane / 32) * 4 + i % 4) * 32 + lane % 32] = c[i];
    }
}

template <int R>
static hipError_t launch_mfma_unit(int sel, const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                   const uint8_t* bs, float* out, hipStream_t stream)
{
    switch (sel) {
    case 0: hipLaunchKernelGGL((mfma_unit_kernel<R, 0>), dim3(1), dim3(kWave), 0, stream, a, as, b, bs, out); break;
    case 1: hipLaunchKernelGGL((mfma_unit_kernel<R, 1>), dim3(1), dim3(kWave), 0, stream, a, as, b, bs, out); break;
    case 2: hipLaunchKernelGGL((mfma_unit_kernel<R, 2>), dim3(1), dim3(kWave), 0, stream, a, as, b, bs, out); break;
    default: hipLaunchKernelGGL((mfma_unit_kernel<R, 3>), dim3(1), dim3(kWave), 0, stream, a, as, b, bs, out); break;
    }
    return hipGetLastError();
}

hipError_t run_mfma_unit(int rows, int sel, const uint8_t* a, const uint8_t* as, const uint8_t* b,
                         const uint8_t* bs, float* out, hipStream_t stream)
{
    return rows == 16 ? launch_mfma_unit<16>(sel, a, as, b, bs, out, stream)
                      : launch_mfma_unit<32>(sel, a, as, b, bs, out, stream);
}

hipError_t run_mfma_probe(int random_ops, int small_tile, int iters, int n_cu, int wall_khz,
                          hipStream_t stream, ProbeResult* out)
{
    auto kernel = small_tile ? mfma_probe_kernel<true> : mfma_probe_kernel<false>;
    const int chains = small_tile ? probe_chains<true>() : probe_chains<false>();
    // FLOP per MFMA: 2 x 16 x 16 x 128 or 2 x 32 x 32 x 64
    const double flop_per_op = small_tile ? 2.0 * 16 * 16 * 128 : 2.0 * 32 * 32 * 64;
    const int blocks = 2 * n_cu;
    const int waves = blocks * (kProbeThreads / kWave);
    uint64_t* rec = nullptr;
    float* sink = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipMalloc(&rec, sizeof(uint64_t) * 2 * size_t(waves));
    if (err == hipSuccess) err = hipMalloc(&sink, sizeof(float) * size_t(waves));
    if (err == hipSuccess) err = hipEventCreate(&e0);
    if (err == hipSuccess) err = hipEventCreate(&e1);
    if (err == hipSuccess) {
        // a short run first, so that the measured one starts with the clocks settled
        hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kProbeThreads), 0, stream, iters / 4 + 1,
                           random_ops, rec, sink);
        err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e0, stream);
    if (err == hipSuccess) {
        hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kProbeThreads), 0, stream, iters, random_ops,
                           rec, sink);
        err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e1, stream);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    std::vector<uint64_t> h(2 * size_t(waves));
    if (err == hipSuccess)
        err = hipMemcpy(h.data(), rec, sizeof(uint64_t) * h.size(), hipMemcpyDeviceToHost);
    if (err == hipSuccess) {
        double ticks = 0.0, cycles = 0.0;
        for (int w = 0; w < waves; ++w) {
            ticks += double(h[2 * w]);
            cycles += double(h[2 * w + 1]);
        }
        const double flop = double(waves) * iters * chains * flop_per_op;
        out->ms = ms;
        out->tflops = flop / (double(ms) * 1e-3) / 1e12;
        out->shader_mhz = ticks > 0 ? cycles / ticks * (double(wall_khz) / 1000.0) : 0.0;
        // one 32x32x64 MFMA per 32 cycles per SIMD, four SIMDs per CU
        const double per_clock = double(n_cu) * 4 * (2.0 * 32 * 32 * 64) / 32.0;
        out->per_clock_frac =
            out->shader_mhz > 0 ? out->tflops * 1e12 / (per_clock * out->shader_mhz * 1e6) : 0.0;
    }
    // clean-up errors would not change the measurement already taken
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (rec) (void)hipFree(rec);
    if (sink) (void)hipFree(sink);
    return err;
}

}  // namespace moe
