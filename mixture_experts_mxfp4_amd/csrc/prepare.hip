// Weight preparation: permute raw MXFP4 codes and e8m0 scales into the layout
// the grouped GEMMs stream (a bijection; the same kernel runs it backwards).
//
// The pages ship pre-shuffled weights and scales beside the raw ones
// (kernelindex submissions 754773 and 723815, `*_shuffled` inputs); the
// shuffle here is this library's own, chosen for gfx950's 16x16x128 FP4 MFMA:
//
//   codes  [N/64][K/128][4][64 lanes][16 B]   one MFMA B fragment = 1 KiB
//   scales [N/64][K/128][64 lanes][4 B]       byte q of lane L's word: slice q
//
// Lane L of slice q of 64-row group n64 at K tile kt holds row
// n64*64 + q*16 + L%16 and elements kt*128 + (L/16)*32 .. +32, so a wave reads
// each fragment as one contiguous, fully coalesced 1 KiB and the four slices
// of a group at one K tile as 4 KiB, plus one 256-byte scale block holding
// every lane's four slice scales as one word.  For gate_up the rows are interleaved so
// that a 64-row group c holds gate rows c*32..+31 then up rows I+c*32..+31:
// one workgroup then owns matching gate/up columns, which the fused SwiGLU and
// its MXFP4 requant (per 32 columns) need.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kPrepThreads = 256;

// raw row of prepared row pr (gate_up interleave when gate_up_I > 0)
__device__ __forceinline__ int64_t raw_row(int64_t pr, int gate_up_I)
{
    if (gate_up_I == 0) return pr;
    int64_t c = pr / 64, q = (pr % 64) / 16, j = pr % 16;
    return (q < 2 ? 0 : gate_up_I) + c * 32 + (q & 1) * 16 + j;
}

// One thread per 16-byte code fragment slot and per 4-byte scale word.
__global__ void __launch_bounds__(kPrepThreads)
prepare_kernel(const uint8_t* __restrict__ src_codes, const uint8_t* __restrict__ src_scales,
               uint8_t* __restrict__ dst_codes, uint8_t* __restrict__ dst_scales, int E, int N,
               int K, int gate_up_I, int inverse)
{
    const int KT = K / 128;
    const int64_t frags_per_e = int64_t(N / 64) * KT * 4 * 64;
    const int64_t words_per_e = int64_t(N / 64) * KT * 64;
    const int64_t n_frag = int64_t(E) * frags_per_e;
    const int64_t n_total = n_frag + int64_t(E) * words_per_e;
    const int64_t stride = int64_t(gridDim.x) * kPrepThreads;
    for (int64_t i = int64_t(blockIdx.x) * kPrepThreads + threadIdx.x; i < n_total; i += stride) {
        if (i < n_frag) {
            const int64_t e = i / frags_per_e, f = i % frags_per_e;
            const int L = int(f % 64);
            const int q = int((f / 64) % 4);
            const int64_t kt = (f / 256) % KT;
            const int64_t n64 = f / (256 * int64_t(KT));
            const int64_t row = raw_row(n64 * 64 + q * 16 + L % 16, gate_up_I);
            const int64_t raw = e * int64_t(N) * (K / 2) + row * (K / 2) + kt * 64 + (L / 16) * 16;
            const int64_t prep = e * int64_t(N) * (K / 2) + f * 16;
            if (!inverse) *reinterpret_cast<uint4*>(dst_codes + prep) = ld16(src_codes + raw);
            else *reinterpret_cast<uint4*>(dst_codes + raw) = ld16(src_codes + prep);
        } else {
            const int64_t j = i - n_frag;
            const int64_t e = j / words_per_e, f = j % words_per_e;
            const int L = int(f % 64);
            const int64_t kt = (f / 64) % KT;
            const int64_t n64 = f / (64 * int64_t(KT));
            const int64_t base = e * int64_t(N) * (K / 32);
            for (int q = 0; q < 4; ++q) {
                const int64_t row = raw_row(n64 * 64 + q * 16 + L % 16, gate_up_I);
                const int64_t raw = base + row * (K / 32) + kt * 4 + L / 16;
                const int64_t prep = base + f * 4 + q;
                if (!inverse) dst_scales[prep] = src_scales[raw];
                else dst_scales[raw] = src_scales[prep];
            }
        }
    }
}

hipError_t launch_prepare(const uint8_t* src_codes, const uint8_t* src_scales, uint8_t* dst_codes,
                          uint8_t* dst_scales, int E, int N, int K, int gate_up_I, int inverse,
                          int n_cu, hipStream_t stream)
{
    const int KT = K / 128;
    const int64_t n_total = int64_t(E) * (N / 64) * 64 * KT * 5;
    int64_t blocks = (n_total + kPrepThreads - 1) / kPrepThreads;
    if (blocks > int64_t(n_cu) * 32) blocks = int64_t(n_cu) * 32;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(prepare_kernel, dim3(unsigned(blocks)), dim3(kPrepThreads), 0, stream,
                       src_codes, src_scales, dst_codes, dst_scales, E, N, K, gate_up_I, inverse);
    return hipGetLastError();
}

}  // namespace moe
