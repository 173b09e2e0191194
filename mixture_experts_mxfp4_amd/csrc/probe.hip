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
