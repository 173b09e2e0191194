// FP4 MFMA rate probe (probe.hip): a measurement aid for the roofline of the
// LDS-tiled GEMMs, not part of the forward.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

struct ProbeResult {
    double ms;               // the measured launch (events)
    double tflops;           // FP4 MFMA rate over it
    double shader_mhz;       // mean shader clock of its waves
    double per_clock_frac;   // rate over the FP4 peak per clock: one 32x32x64 MFMA per 32 cycles per SIMD
};

// Two workgroups of four waves per CU, each wave `iters` x 4 independent
// 32x32x64 MFMAs (small_tile: 8 independent 16x16x128 ones) on register
// operands (random bits, or one set bit per word), after a short settling
// launch.  Allocates and frees its own record buffers.
hipError_t run_mfma_probe(int random_ops, int small_tile, int iters, int n_cu, int wall_khz,
                          hipStream_t stream, ProbeResult* out);

// One block-scaled FP4 MFMA (rows 16: 16x16x128, 32: 32x32x64) on row-major
// E2M1 operands with per-32 e8m0 scales, the scale in byte `sel` (0-3) of its
// word; out = A . B^T, fp32 row-major rows x rows.  One wave; arguments
// checked by the caller.
hipError_t run_mfma_unit(int rows, int sel, const uint8_t* a, const uint8_t* as, const uint8_t* b,
                         const uint8_t* bs, float* out, hipStream_t stream);

}  // namespace moe
