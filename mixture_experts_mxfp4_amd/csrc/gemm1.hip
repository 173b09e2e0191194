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
// expert) and NG 64-row groups of the prepared gate_up weight; a group is 32
// gate + 32 up columns = one MXFP4 group of h.  Workgroups take (group, block)
// units in the XCD-aware order of xcd_unit.  The four waves split the K
// dimension; each wave runs NG x RT x 4 MFMA tiles of 16x16x128, streaming its weight
// fragments (1 KiB each, contiguous) and gathering the block's activation rows
// by token id.  With paired 32-row blocks (gemm1_swiglu_quant_kernel_paired)
// a pair's two workgroups take the pair's 64 rows for one group each.  Weight
// loads are non-temporal, except for experts with several units: their units
// at one group pair run side by side on one XCD, and cached loads let all but
// the first find the slice in L2 (prefill at E=257: stage-1 fetch 604 -> 575
// MB, 124.5 -> 118 us).  Partial sums meet in LDS; the epilogue quantizes h
// with cross-lane reductions and writes it in sorted-row order in the
// fragment layout (moe_common.h) that stage 2 loads contiguously.
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kGemmThreads = 256;
// Row tiles per LDS reduction pass of the epilogue: two keep the pass at 32
// KiB of LDS for four waves, whatever the block size.
constexpr int kRedTiles = 2;

// Loads of U consecutive K tiles are issued before their MFMAs so that every
// wave keeps U x NG x 4 KiB of weight fragments in flight (U = 2 at 64-row
// blocks with two groups would spill).
template <int RT, int NG>
constexpr int g1_unroll() { return NG == 1 ? (RT <= 2 ? 4 : 2) : (RT <= 2 ? 2 : 1); }

// One unit: the 16*RT sorted rows from row0 (all of expert e) times the NG
// MXFP4 groups of h from c0.  red: the LDS of the partial-sum passes.
template <int RT, int NG, typename Red>
__device__ __forceinline__ void g1_unit(const uint8_t* __restrict__ a1q, const uint8_t* __restrict__ a1s,
                                        const uint8_t* __restrict__ w13p, const uint8_t* __restrict__ w13sp,
                                        const int32_t* __restrict__ sorted_route,
                                        uint8_t* __restrict__ a2q, uint8_t* __restrict__ a2s,
                                        uint16_t* __restrict__ h_dbg, int M, int D, int I, int topk,
                                        int64_t cap, int64_t row0, int c0, int e, bool shared_w, Red& red)
{
    constexpr int U = g1_unroll<RT, NG>();
    // the partial sums meet in LDS kRedTiles row tiles at a time:
    // red[wave][row tile][slice][i][lane]
    constexpr int RTH = RT < kRedTiles ? RT : kRedTiles;
    constexpr int WPT = 4 / RTH;          // waves finishing each row tile of a pass
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int R = M * topk;
    const int KT = D / 128;
    const int64_t a_row = D / 2, as_row = D / 32;

    const uint8_t* a_ptr[RT];
    const uint8_t* as_ptr[RT];
    bool ok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int sr = sorted_route[row0 + rt * 16 + lane % 16];
        ok[rt] = sr < R;
        const int64_t tok = ok[rt] ? sr / topk : 0;
        a_ptr[rt] = a1q + tok * a_row + (lane / 16) * 16;
        as_ptr[rt] = a1s + tok * as_row;
    }
    // the NG consecutive groups' weight fragments and scale words
    const uint8_t* wb = w13p + int64_t(e) * I * D + int64_t(c0) * KT * 4096 + lane * 16;
    const uint8_t* sb = w13sp + int64_t(e) * I * D / 16 + int64_t(c0) * KT * 256 + lane * 4;
    const int ash = 8 * (lane / 16);     // this lane's 32-block inside an A scale word

    v4f acc[NG][RT][4];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[g][rt][q] = v4f{0.f, 0.f, 0.f, 0.f};

    auto steps = [&](auto u_const, auto nt_const, int kt) {
        constexpr int UU = decltype(u_const)::value;
        constexpr bool NT = decltype(nt_const)::value;
        uint32_t sw[UU][NG], sa[UU][RT];
        uint4 b[UU][NG][4], a[UU][RT];
#pragma unroll
        for (int u = 0; u < UU; ++u) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                sw[u][g] = *reinterpret_cast<const uint32_t*>(sb + int64_t(g) * KT * 256 + (kt + u) * 256);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    b[u][g][q] = NT ? ld16_nt(wb + (int64_t(g) * KT + kt + u) * 4096 + q * 1024)
                                    : ld16(wb + (int64_t(g) * KT + kt + u) * 4096 + q * 1024);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                sa[u][rt] = ok[rt] ? *reinterpret_cast<const uint32_t*>(as_ptr[rt] + (kt + u) * 4) : 0u;
                a[u][rt] = ok[rt] ? ld16(a_ptr[rt] + (kt + u) * 64) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < UU; ++u)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[g][rt][q] = mfma_fp4_16x16x128(a[u][rt], b[u][g][q], acc[g][rt][q],
                                                           (sa[u][rt] >> ash) & 0xFFu,
                                                           (sw[u][g] >> (8 * q)) & 0xFFu);
    };
    auto kloop = [&](auto nt_const) {
        const int kt1 = (wave + 1) * KT / 4;
        int kt = wave * KT / 4;
        for (; kt + U <= kt1; kt += U) steps(std::integral_constant<int, U>{}, nt_const, kt);
        for (; kt < kt1; ++kt) steps(std::integral_constant<int, 1>{}, nt_const, kt);
    };
    if (shared_w)
        kloop(std::false_type{});
    else
        kloop(std::true_type{});

#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int c = c0 + g;
#pragma unroll
        for (int p = 0; p < RT; p += RTH) {
            if (g > 0 || p > 0) __syncthreads();   // red is reused pass by pass
#pragma unroll
            for (int r = 0; r < RTH; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i) red[wave][r][q][i][lane] = acc[g][p + r][q][i];
            __syncthreads();

            // wave w finishes rows i = (w % WPT) * (4 / WPT) ... of row tile w / WPT
            const int r = wave / WPT, rt = p + r;
#pragma unroll
            for (int ii = 0; ii < 4 / WPT; ++ii) {
                const int i = (wave % WPT) * (4 / WPT) + ii;
                float s4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    s4[q] = red[0][r][q][i][lane] + red[1][r][q][i][lane] +
                            red[2][r][q][i][lane] + red[3][r][q][i][lane];
                // slices 0,1 = gate columns c*32 + lane%16 (+16), slices 2,3 = up
                const uint32_t h0 = f32_to_bf16_rne(silu_fast(s4[0]) * s4[2]);
                const uint32_t h1 = f32_to_bf16_rne(silu_fast(s4[1]) * s4[3]);
                const int row = 4 * (lane / 16) + i;                     // row within the tile
                const int64_t srow = row0 + rt * 16 + row;               // sorted row
                if (h_dbg) {
                    h_dbg[srow * I + c * 32 + lane % 16] = uint16_t(h0);
                    h_dbg[srow * I + c * 32 + 16 + lane % 16] = uint16_t(h1);
                }
                // MXFP4 group = the 32 columns held by the 16 lanes of this row
                // (one DPP row): columns lane%16 (h0) and 16 + lane%16 (h1)
                const uint32_t s = mx_scale_from_amax(row16_max(max(h0 & 0x7FFFu, h1 & 0x7FFFu)));
                const uint32_t qlo = pack8_codes(mx_code(h0, s));   // bytes 0-3 on lane%16 == 0
                const uint32_t qhi = pack8_codes(mx_code(h1, s));   // bytes 8-11
                const uint32_t d1 = from_lane_plus<8>(qlo);         // bytes 4-7
                const uint32_t d3 = from_lane_plus<8>(qhi);         // bytes 12-15
                if (lane % 16 == 0) {
                    *reinterpret_cast<uint4*>(a2q + frag_code_off(srow, c / 4, c % 4, I / 128)) =
                        make_uint4(qlo, d1, qhi, d3);
                    a2s[frag_scale_off(srow, c / 4, cap) + c % 4] = uint8_t(s);
                }
            }
        }
    }
}

// Uniform blocks of BM = 16*RT rows: one unit per (group pair, block).
template <int RT, int NG>
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2)))
gemm1_swiglu_quant_kernel(const uint8_t* __restrict__ a1q, const uint8_t* __restrict__ a1s,
                          const uint8_t* __restrict__ w13p, const uint8_t* __restrict__ w13sp,
                          const int32_t* __restrict__ sorted_route,
                          const int32_t* __restrict__ block_expert,
                          const int32_t* __restrict__ num_valid, uint8_t* __restrict__ a2q,
                          uint8_t* __restrict__ a2s, uint16_t* __restrict__ h_dbg, int M, int D,
                          int I, int topk, int64_t cap, uint64_t* clk)
{
    constexpr int BM = 16 * RT;
    constexpr int RTH = RT < kRedTiles ? RT : kRedTiles;
    __shared__ float red[4][RTH][4][4][kWave];
    span_begin(clk);
    int xg, blk;                          // NG-group pair xg of block blk (XCD-aware order)
    const int nb_used = num_valid[0] / BM;
    if (xcd_unit(I / (32 * NG), nb_used, xg, blk)) {
        const int e = block_expert[blk];
        // an expert with several blocks: its blocks at this xg run side by side on
        // one XCD and share the weight slice through L2 (cached loads)
        const bool shared_w = (blk > 0 && block_expert[blk - 1] == e) ||
                              (blk + 1 < nb_used && block_expert[blk + 1] == e);
        g1_unit<RT, NG>(a1q, a1s, w13p, w13sp, sorted_route, a2q, a2s, h_dbg, M, D, I, topk, cap,
                        int64_t(blk) * BM, xg * NG, e, shared_w, red);
    }
    span_end(clk);
}

// 32-row blocks, where the blocks of an expert with few of them run in pairs
// as 64-row units (paired_block): the workgroup of block j of a pair takes
// the pair's 64 rows for group j of the group pair (same accumulator count
// as a 32-row unit of two groups), so the pair reads each weight group once
// and both workgroups work.  An expert with 33 to 64 routes then reads its
// weights once, not once per block; a Zipf-hot expert's many blocks keep
// 32-row units.
template <int NG>
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2)))
gemm1_swiglu_quant_kernel_paired(const uint8_t* __restrict__ a1q, const uint8_t* __restrict__ a1s,
                   const uint8_t* __restrict__ w13p, const uint8_t* __restrict__ w13sp,
                   const int32_t* __restrict__ sorted_route, const int4* __restrict__ block_info,
                   const int32_t* __restrict__ num_valid, uint8_t* __restrict__ a2q,
                   uint8_t* __restrict__ a2s, uint16_t* __restrict__ h_dbg, int M, int D, int I,
                   int topk, int64_t cap, uint64_t* clk)
{
    __shared__ float red[4][kRedTiles][4][4][kWave];
    span_begin(clk);
    int xg, blk;
    if (xcd_unit(I / (32 * NG), num_valid[0] / 32, xg, blk)) {
        const int4 bi = block_info[blk];      // expert, its first block, its block count, routes
        // other units of the expert read the same weight slice: cached loads
        if (!paired_block(bi, blk)) {
            g1_unit<2, NG>(a1q, a1s, w13p, w13sp, sorted_route, a2q, a2s, h_dbg, M, D, I, topk, cap,
                           int64_t(blk) * 32, xg * NG, bi.x, bi.z > 1, red);
        } else {
            const int j = (blk - bi.y) & 1;
            g1_unit<4, NG / 2>(a1q, a1s, w13p, w13sp, sorted_route, a2q, a2s, h_dbg, M, D, I, topk,
                               cap, int64_t(blk - j) * 32, xg * NG + j * (NG / 2), bi.x, bi.z > 2,
                               red);
        }
    }
    span_end(clk);
}

template <int RT>
static hipError_t launch_g1(const Gemm1Args& a, hipStream_t stream, const KernelEvents& ev)
{
    constexpr int NG = stream_stage1_groups(16 * RT);
    MOE_LAUNCH((gemm1_swiglu_quant_kernel<RT, NG>), dim3(tile_grid(a.I / (32 * NG), a.nb_cap)),
               dim3(kGemmThreads), 0,
               stream, ev, a.a1q, a.a1s, a.w13p, a.w13sp, a.sorted_route, a.block_expert,
               a.num_valid, a.a2q, a.a2s, a.h_dbg, a.M, a.D, a.I, a.topk, a.cap, a.clk);
    return hipGetLastError();
}

static hipError_t launch_g1_paired(const Gemm1Args& a, hipStream_t stream, const KernelEvents& ev)
{
    constexpr int NG = stream_stage1_groups(32);
    if (!a.block_info) return hipErrorInvalidValue;
    MOE_LAUNCH((gemm1_swiglu_quant_kernel_paired<NG>), dim3(tile_grid(a.I / (32 * NG), a.nb_cap)),
               dim3(kGemmThreads), 0, stream, ev, a.a1q, a.a1s, a.w13p, a.w13sp, a.sorted_route,
               reinterpret_cast<const int4*>(a.block_info), a.num_valid, a.a2q, a.a2s, a.h_dbg,
               a.M, a.D, a.I, a.topk, a.cap, a.clk);
    return hipGetLastError();
}

hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t stream, const KernelEvents& ev)
{
    if (a.nb_cap == 0) return hipSuccess;
    switch (a.block_m) {
    case 16: return launch_g1<1>(a, stream, ev);
    case 32: return a.pair_blocks ? launch_g1_paired(a, stream, ev) : launch_g1<2>(a, stream, ev);
    case 64: return launch_g1<4>(a, stream, ev);
    default: return hipErrorInvalidValue;
    }
}

// Fragment-layout a2 -> canonical row-major [cap][I/2] codes, [cap][I/32] scales.
__global__ void a2_to_canonical_kernel(const uint8_t* __restrict__ a2q,
                                       const uint8_t* __restrict__ a2s, int64_t cap, int I,
                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int ng = I / 32;
    const int64_t n = cap * ng;
    for (int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < n;
         idx += int64_t(gridDim.x) * blockDim.x) {
        const int64_t row = idx / ng;
        const int c = int(idx % ng);
        if (codes)
            *reinterpret_cast<uint4*>(codes + row * (I / 2) + c * 16) =
                ld16(a2q + frag_code_off(row, c / 4, c % 4, I / 128));
        if (scales) scales[row * ng + c] = a2s[frag_scale_off(row, c / 4, cap) + c % 4];
    }
}

hipError_t launch_a2_to_canonical(const uint8_t* a2q, const uint8_t* a2s, int64_t cap, int I,
                                  uint8_t* codes, uint8_t* scales, hipStream_t stream)
{
    const int64_t n = cap * (I / 32);
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(a2_to_canonical_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, a2q,
                       a2s, cap, I, codes, scales);
    return hipGetLastError();
}

}  // namespace moe
