// Stage 2: grouped down-projection GEMM on gfx950 block-scaled FP4 MFMA; the
// epilogue multiplies by the routing weight; a final pass sums the topk
// contributions of every token.
//
// Semantics (kernelindex submission 754773: stage 2 receives the sorted
// routing weights and accumulates the experts' contributions per token;
// kernelindex submission 723815 `_reference_forward`: out[t] += w * (act @
// W_down^T)): y = Q(h) . down_row over K = I for each sorted row, and
// out[t, :] = sum over the token's valid slots s of topk_w[t, s] * y(t, s).
//
// The pages accumulate with atomics (`mode: atomic`).  On MI355X fp32 atomics
// to L2 sustain ~0.27 G element-adds per microsecond, which made them the
// bottleneck of the prefill shapes; instead each sorted row's weighted result
// is stored once, as bf16, at its route index r = t*topk + s (plain coalesced
// stores, no read-modify-write), and a reduction kernel adds the topk rows of
// each token in a fixed slot order in fp32 and rounds once to bf16.  The
// result is deterministic.  The extra rounding of each weighted contribution
// to bf16 is bounded by 2^-9 of that contribution.
//
// Tiling: a workgroup (4 waves) owns one block of BM = 16*RT sorted rows and
// 256*NG output columns (units in the XCD-aware order of xcd_unit); each wave
// owns NG groups of 64 columns (4 MFMA tiles per row tile each) and runs the
// whole K = I loop for each, streaming 1 KiB weight fragments; the A
// fragments (MXFP4 h, written by stage 1 in the fragment layout) are
// contiguous 1 KiB loads as well.  With paired 32-row blocks
// (gemm2_simple_kernel_paired) a pair's two workgroups take the pair's 64
// rows for half of the 256-column tile each.  Weight loads are non-temporal,
// except in the simple kernels for experts with several units, whose units at
// one column tile share the slice through L2 (64 tokens on E=33: 47.6 -> 44.9
// us).
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kGemmThreads = 256;

// K tiles per load batch.  64-row units take one: batching more raised the register count
// (five waves per SIMD fit at one) and measured slower on the 1100-token prefill.
template <int RT>
constexpr int g2_unroll() { return RT <= 2 ? 4 : 1; }

// Staged output rows of a unit of 16*RT rows x 64*NQ columns: the row's bf16
// plus 16 B, so that consecutive rows start four banks apart.
template <int NQ>
constexpr int stage_row() { return 64 * NQ * 2 + 16; }
template <int RT, int NQ>
constexpr int stage_bytes() { return 16 * RT * stage_row<NQ>(); }

// One unit: the 16*RT sorted rows from row0 (all of expert e) times the
// 64*NQ output columns from col0 (each wave NQ 16-column MFMA tiles of one
// prepared 64-row group).  stage, s_route: LDS of at least 16*RT staged rows
// and routes.
template <int RT, int NQ>
__device__ __forceinline__ void g2_unit(const uint8_t* __restrict__ a2q, const uint8_t* __restrict__ a2s,
                                        const uint8_t* __restrict__ w2p, const uint8_t* __restrict__ w2sp,
                                        const int32_t* __restrict__ sorted_route,
                                        const float* __restrict__ sorted_w, uint16_t* __restrict__ partial,
                                        int M, int D, int I, int topk, int64_t cap, int64_t row0, int col0,
                                        int e, bool shared_w, uint8_t* stage, int32_t* s_route)
{
    static_assert(NQ == 2 || NQ == 4, "a wave covers half or all of a 64-row weight group");
    constexpr int BM = 16 * RT;
    constexpr int U = g2_unroll<RT>();
    constexpr int kCols = 64 * NQ;          // output columns of the unit
    constexpr int kRow = stage_row<NQ>();
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wcol = col0 + wave * 16 * NQ; // the wave's first output column
    const int n64 = wcol / 64, q0 = (wcol % 64) / 16;
    const int KT = I / 128;
    const int R = M * topk;

    const uint8_t* wb = w2p + int64_t(e) * D * (I / 2) + int64_t(n64) * KT * 4096 + q0 * 1024 + lane * 16;
    const uint8_t* sb = w2sp + int64_t(e) * D * (I / 32) + int64_t(n64) * KT * 256 + lane * 4;
    // A operand: the 1 KiB fragment of row tile rt at K tile kt; scales kt-major
    const uint8_t* a_ptr[RT];
    const uint8_t* as_ptr[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int64_t r0 = row0 + rt * 16;
        a_ptr[rt] = a2q + frag_code_off(r0, 0, 0, KT) + lane * 16;
        as_ptr[rt] = a2s + frag_scale_off(r0 + lane % 16, 0, cap);
    }
    const int ash = 8 * (lane / 16);

    v4f acc[RT][NQ];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[rt][q] = v4f{0.f, 0.f, 0.f, 0.f};

    auto steps = [&](auto u_const, auto nt_const, int kt) {
        constexpr int UU = decltype(u_const)::value;
        constexpr bool NT = decltype(nt_const)::value;
        uint32_t sw[UU], sa[UU][RT];
        uint4 b[UU][NQ], a[UU][RT];
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            // byte q0 + q of the group's scale word: column tile q of this wave
            sw[u] = *reinterpret_cast<const uint32_t*>(sb + (kt + u) * 256) >> (8 * q0);
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                b[u][q] = NT ? ld16_nt(wb + int64_t((kt + u) * 4 + q) * 1024)
                             : ld16(wb + int64_t((kt + u) * 4 + q) * 1024);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                sa[u][rt] = *reinterpret_cast<const uint32_t*>(as_ptr[rt] + (kt + u) * cap * 4);
                a[u][rt] = ld16(a_ptr[rt] + (kt + u) * 1024);
            }
        }
#pragma unroll
        for (int u = 0; u < UU; ++u)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    // weights as the first operand: acc[rt][q] holds the transposed
                    // 16x16 tile (lane: row rt*16 + lane%16, columns 4*(lane/16) + i)
                    acc[rt][q] = mfma_fp4_16x16x128(b[u][q], a[u][rt], acc[rt][q],
                                                    (sw[u] >> (8 * q)) & 0xFFu,
                                                    (sa[u][rt] >> ash) & 0xFFu);
    };
    auto kloop = [&](auto nt_const) {
        int kt = 0;
        for (; kt + U <= KT; kt += U) steps(std::integral_constant<int, U>{}, nt_const, kt);
        for (; kt < KT; ++kt) steps(std::integral_constant<int, 1>{}, nt_const, kt);
    };
    if (shared_w)
        kloop(std::false_type{});
    else
        kloop(std::true_type{});

    // Epilogue: the routing weight times the sum, rounded to bf16, goes through
    // LDS as the unit's BM x kCols tile; then 4*NQ consecutive lanes store one
    // row's contiguous 2*kCols bytes of its route's partial row (padding rows
    // skipped).
    if (threadIdx.x < BM) s_route[threadIdx.x] = sorted_route[row0 + threadIdx.x];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int row = rt * 16 + lane % 16;
        const float w = sorted_w[row0 + row];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int col = wave * 16 * NQ + q * 16 + 4 * (lane / 16);
            uint2 v;
            v.x = f32x2_to_bf16x2(w * acc[rt][q][0], w * acc[rt][q][1]);
            v.y = f32x2_to_bf16x2(w * acc[rt][q][2], w * acc[rt][q][3]);
            *reinterpret_cast<uint2*>(stage + row * kRow + col * 2) = v;
        }
    }
    __syncthreads();
    constexpr int kChunks = kCols / 8;                  // 16-byte chunks per row
#pragma unroll
    for (int k = 0; k < BM * kChunks / kGemmThreads; ++k) {
        const int c = k * kGemmThreads + threadIdx.x;   // row c / kChunks, chunk c % kChunks
        const int row = c / kChunks, ch = c % kChunks;
        const int sr = s_route[row];
        const uint4 v = *reinterpret_cast<const uint4*>(stage + row * kRow + ch * 16);
        if (sr < R)
            *reinterpret_cast<uint4*>(partial + int64_t(sr) * D + col0 + ch * 8) = v;
    }
}

// Uniform blocks of BM = 16*RT rows: one unit per (256-column tile, block).
// Four waves per SIMD at least: the register allocation then fits 128
// registers (116 VGPRs at 64-row blocks, no accumulation registers) instead
// of taking 150 and three waves; one wave more per SIMD keeps more weight
// loads in flight (prefill stage 2 90 -> 88.5 us, 128 tokens on E=33 19 -> 17
// us).
template <int RT>
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4)))
gemm2_simple_kernel(const uint8_t* __restrict__ a2q, const uint8_t* __restrict__ a2s,
                    const uint8_t* __restrict__ w2p, const uint8_t* __restrict__ w2sp,
                    const int32_t* __restrict__ sorted_route, const float* __restrict__ sorted_w,
                    const int32_t* __restrict__ block_expert,
                    const int32_t* __restrict__ num_valid, uint16_t* __restrict__ partial,
                    int M, int D, int I, int topk, int64_t cap)
{
    constexpr int BM = 16 * RT;
    __shared__ __attribute__((aligned(16))) uint8_t stage[stage_bytes<RT, 4>()];
    __shared__ int32_t s_route[BM];
    int ct, blk;                           // 256-column tile ct of block blk (XCD-aware order)
    const int nb_used = num_valid[0] / BM;
    if (!xcd_unit(D / 256, nb_used, ct, blk)) return;
    const int e = block_expert[blk];
    // an expert with several blocks: its blocks at this ct run side by side on
    // one XCD and share the weight slice through L2 (cached loads)
    const bool shared_w = (blk > 0 && block_expert[blk - 1] == e) ||
                          (blk + 1 < nb_used && block_expert[blk + 1] == e);
    g2_unit<RT, 4>(a2q, a2s, w2p, w2sp, sorted_route, sorted_w, partial, M, D, I, topk, cap,
                   int64_t(blk) * BM, ct * 256, e, shared_w, stage, s_route);
}

// 32-row blocks, where the blocks of an expert with few of them run in pairs
// as 64-row units (paired_block, the same rule as stage 1): the workgroup of
// block j of a pair takes the pair's 64 rows for column half j of the tile
// (same accumulator count as a 32-row unit of the whole tile, and the same
// staged bytes).
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4)))
gemm2_simple_kernel_paired(const uint8_t* __restrict__ a2q, const uint8_t* __restrict__ a2s,
                   const uint8_t* __restrict__ w2p, const uint8_t* __restrict__ w2sp,
                   const int32_t* __restrict__ sorted_route, const float* __restrict__ sorted_w,
                   const int4* __restrict__ block_info, const int32_t* __restrict__ num_valid,
                   uint16_t* __restrict__ partial, int M, int D, int I, int topk, int64_t cap)
{
    // staged rows: 32 x 256 or 64 x 128 columns
    __shared__ __attribute__((aligned(16))) uint8_t stage[stage_bytes<2, 4>() > stage_bytes<4, 2>()
                                                          ? stage_bytes<2, 4>() : stage_bytes<4, 2>()];
    __shared__ int32_t s_route[64];
    int ct, blk;                           // 256-column tile ct of block blk (XCD-aware order)
    if (!xcd_unit(D / 256, num_valid[0] / 32, ct, blk)) return;
    const int4 bi = block_info[blk];       // expert, its first block, its block count, routes
    // other units of the expert at this ct run side by side on one XCD and
    // share the weight slice through L2 (cached loads)
    if (!paired_block(bi, blk)) {
        g2_unit<2, 4>(a2q, a2s, w2p, w2sp, sorted_route, sorted_w, partial, M, D, I, topk, cap,
                      int64_t(blk) * 32, ct * 256, bi.x, bi.z > 1, stage, s_route);
    } else {
        const int j = (blk - bi.y) & 1;
        g2_unit<4, 2>(a2q, a2s, w2p, w2sp, sorted_route, sorted_w, partial, M, D, I, topk, cap,
                      int64_t(blk - j) * 32, ct * 256 + j * 128, bi.x, bi.z > 2, stage, s_route);
    }
}

// Each wave walks NG 64-column groups (group g of the wave's workgroup lies
// at n64 = blockIdx.x*4*NG + g*4 + wave, so the four waves stream adjacent
// groups); the K tiles of the whole walk are processed U at a time, and the
// loads of the next U tiles are issued before the MFMAs of the current ones
// (register double buffering), keeping 2 x U x 4 KiB in flight per wave.
template <int RT, int U, int NG>
__global__ void __launch_bounds__(kGemmThreads)
gemm2_weighted_kernel(const uint8_t* __restrict__ a2q, const uint8_t* __restrict__ a2s,
                      const uint8_t* __restrict__ w2p, const uint8_t* __restrict__ w2sp,
                      const int32_t* __restrict__ sorted_route, const float* __restrict__ sorted_w,
                      const int32_t* __restrict__ block_expert,
                      const int32_t* __restrict__ num_valid, uint16_t* __restrict__ partial,
                      int M, int D, int I, int topk, int64_t cap)
{
    constexpr int BM = 16 * RT;
    int ct, blk;                           // column range ct of block blk (XCD-aware order)
    if (!xcd_unit(D / (256 * NG), num_valid[0] / BM, ct, blk)) return;
    const int e = block_expert[blk];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int KT = I / 128;                 // a multiple of U
    const int R = M * topk;
    const int n64_0 = ct * 4 * NG + wave;

    const uint8_t* wexp = w2p + int64_t(e) * D * (I / 2) + lane * 16;
    const uint8_t* sexp = w2sp + int64_t(e) * D * (I / 32) + lane * 4;
    // A operand: the 1 KiB fragment of row tile rt at K tile kt; scales kt-major
    const uint8_t* a_ptr[RT];
    const uint8_t* as_ptr[RT];
    int sr[RT][4];
    float wt[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int64_t row0 = int64_t(blk) * BM + rt * 16;
        a_ptr[rt] = a2q + frag_code_off(row0, 0, 0, KT) + lane * 16;
        as_ptr[rt] = a2s + frag_scale_off(row0 + lane % 16, 0, cap);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sr[rt][i] = sorted_route[row0 + 4 * (lane / 16) + i];
            wt[rt][i] = sorted_w[row0 + 4 * (lane / 16) + i];
        }
    }
    const int ash = 8 * (lane / 16);

    struct Chunk {
        uint32_t sw[U], sa[U][RT];
        uint4 b[U][4], a[U][RT];
    };
    // chunk c covers K tiles (c*U .. c*U+U-1) mod KT of group c*U / KT
    auto load = [&](Chunk& ch, int c) {
        const int g = (c * U) / KT, kt0 = (c * U) % KT;
        const int64_t n64 = n64_0 + g * 4;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kt = kt0 + u;
            ch.sw[u] = *reinterpret_cast<const uint32_t*>(sexp + (n64 * KT + kt) * 256);
#pragma unroll
            for (int q = 0; q < 4; ++q) ch.b[u][q] = ld16_nt(wexp + ((n64 * KT + kt) * 4 + q) * 1024);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                ch.sa[u][rt] = *reinterpret_cast<const uint32_t*>(as_ptr[rt] + int64_t(kt) * cap * 4);
                ch.a[u][rt] = ld16(a_ptr[rt] + kt * 1024);
            }
        }
    };
    v4f acc[RT][4];
    auto zero = [&]() {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[rt][q] = v4f{0.f, 0.f, 0.f, 0.f};
    };
    auto compute = [&](const Chunk& ch) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[rt][q] = mfma_fp4_16x16x128(ch.a[u][rt], ch.b[u][q], acc[rt][q],
                                                    (ch.sa[u][rt] >> ash) & 0xFFu,
                                                    (ch.sw[u] >> (8 * q)) & 0xFFu);
    };
    auto store = [&](int c) {            // after the last chunk of a group
        const int64_t n64 = n64_0 + ((c * U) / KT) * 4;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint16_t* dst = partial + int64_t(sr[rt][i]) * D + n64 * 64 + lane % 16;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // columns lane%16 and lane%16 + 1 as one dword from the even lane
                    const uint32_t v = f32_to_bf16_rne(wt[rt][i] * acc[rt][q][i]);
                    const uint32_t pair = v | (dpp<kDppXor1>(v) << 16);
                    if (sr[rt][i] < R && (lane & 1) == 0)
                        *reinterpret_cast<uint32_t*>(dst + q * 16) = pair;
                }
            }
        }
    };

    const int nchunks = NG * KT / U;
    Chunk c0, c1;
    zero();
    load(c0, 0);
    for (int c = 0; c < nchunks; c += 2) {
        if (c + 1 < nchunks) load(c1, c + 1);
        compute(c0);
        if (((c + 1) * U) % KT == 0) { store(c); zero(); }
        if (c + 1 >= nchunks) break;
        if (c + 2 < nchunks) load(c0, c + 2);
        compute(c1);
        if (((c + 2) * U) % KT == 0) { store(c + 1); zero(); }
    }
}

template <int RT, int U, int NG>
static hipError_t launch_g2(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev)
{
    MOE_LAUNCH((gemm2_weighted_kernel<RT, U, NG>), dim3(tile_grid(a.D / (256 * NG), a.nb_cap)),
               dim3(kGemmThreads), 0, stream, ev, a.a2q, a.a2s, a.w2p, a.w2sp, a.sorted_route,
               a.sorted_w, a.block_expert, a.num_valid, a.partial, a.M, a.D, a.I, a.topk, a.cap);
    return hipGetLastError();
}

template <int RT>
static hipError_t launch_g2_simple(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev)
{
    MOE_LAUNCH((gemm2_simple_kernel<RT>), dim3(tile_grid(a.D / 256, a.nb_cap)), dim3(kGemmThreads), 0,
               stream, ev, a.a2q, a.a2s, a.w2p, a.w2sp, a.sorted_route, a.sorted_w,
               a.block_expert, a.num_valid, a.partial, a.M, a.D, a.I, a.topk, a.cap);
    return hipGetLastError();
}

static hipError_t launch_g2_paired(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev)
{
    if (!a.block_info) return hipErrorInvalidValue;
    MOE_LAUNCH(gemm2_simple_kernel_paired, dim3(tile_grid(a.D / 256, a.nb_cap)), dim3(kGemmThreads), 0,
               stream, ev, a.a2q, a.a2s, a.w2p, a.w2sp, a.sorted_route, a.sorted_w,
               reinterpret_cast<const int4*>(a.block_info), a.num_valid, a.partial, a.M, a.D, a.I,
               a.topk, a.cap);
    return hipGetLastError();
}

// Few rows per block (decode, block_m 16): each wave walks two column groups
// with double-buffered loads, which keeps enough weight bytes in flight with
// half the workgroups.  Larger blocks keep one group per wave (their
// register budget goes to the extra row tiles).
hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev)
{
    if (a.nb_cap == 0) return hipSuccess;
    switch (a.block_m) {
    case 16:
        return (a.D / 256) % 2 == 0 ? launch_g2<1, 2, 2>(a, stream, ev)
                                    : launch_g2<1, 2, 1>(a, stream, ev);
    case 32: return a.pair_blocks ? launch_g2_paired(a, stream, ev) : launch_g2_simple<2>(a, stream, ev);
    case 64: return launch_g2_simple<4>(a, stream, ev);
    default: return hipErrorInvalidValue;
    }
}

// out[t, :] = bf16( sum_{s < topk, 0 <= ids[t,s] < E} partial[t*topk + s, :] ),
// fp32 sum in slot order.  A thread owns VEC columns of one token and issues
// the loads of all of the token's slot ids and partial rows at once (KMAX >=
// topk slots; a slot whose id is out of range was never written by stage 2:
// its row is loaded but not added), so a token costs one memory round trip.
// Partial rows are read once: non-temporal loads.
template <int VEC, int KMAX>
__global__ void __launch_bounds__(256)
reduce_slots_kernel(const uint16_t* __restrict__ partial, const int32_t* __restrict__ ids, int M,
                    int D, int E, int topk, uint16_t* __restrict__ out)
{
    constexpr int W = VEC / 2;          // 32-bit words per thread and row
    const int64_t per_row = D / VEC;
    const int64_t nv = int64_t(M) * per_row;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nv;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t t = i / per_row;
        const int64_t col = (i % per_row) * VEC;
        int e[KMAX];
        uint32_t v[KMAX][W];
#pragma unroll
        for (int u = 0; u < KMAX; ++u) {
            if (u < topk) {
                e[u] = ids[t * topk + u];
                const uint16_t* src = partial + (t * topk + u) * D + col;
                if constexpr (W == 1) {
                    v[u][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
                } else {
                    const uint4 x = ld16_nt(reinterpret_cast<const uint8_t*>(src));
                    v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
                }
            }
        }
        float acc[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int u = 0; u < KMAX; ++u) {
            if (u < topk && e[u] >= 0 && e[u] < E) {
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    acc[2 * j] += bf16_to_f32(v[u][j] & 0xFFFFu);
                    acc[2 * j + 1] += bf16_to_f32(v[u][j] >> 16);
                }
            }
        }
        uint32_t o[W];
#pragma unroll
        for (int j = 0; j < W; ++j)
            o[j] = f32_to_bf16_rne(acc[2 * j]) | (f32_to_bf16_rne(acc[2 * j + 1]) << 16);
        if constexpr (W == 1)
            *reinterpret_cast<uint32_t*>(out + t * D + col) = o[0];
        else
            *reinterpret_cast<uint4*>(out + t * D + col) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

template <int VEC>
static void launch_reduce_vec(dim3 grid, hipStream_t stream, const KernelEvents& ev,
                              const uint16_t* partial, const int32_t* ids, int M, int D, int E,
                              int topk, uint16_t* out)
{
    if (topk <= 8)
        MOE_LAUNCH((reduce_slots_kernel<VEC, 8>), grid, dim3(256), 0, stream, ev, partial, ids, M,
                   D, E, topk, out);
    else if (topk <= 12)          // top-9 (shared expert + 8): 76 instead of 96 registers at
                                  // VEC 8, six waves per SIMD (large prefill 102 -> 95 us)
        MOE_LAUNCH((reduce_slots_kernel<VEC, 12>), grid, dim3(256), 0, stream, ev, partial, ids, M,
                   D, E, topk, out);
    else if (topk <= 16)
        MOE_LAUNCH((reduce_slots_kernel<VEC, 16>), grid, dim3(256), 0, stream, ev, partial, ids, M,
                   D, E, topk, out);
    else
        MOE_LAUNCH((reduce_slots_kernel<VEC, 32>), grid, dim3(256), 0, stream, ev, partial, ids, M,
                   D, E, topk, out);
}

// Few tokens: two columns per thread (enough threads to cover the latency);
// many tokens: eight columns per thread (16-byte accesses).
hipError_t launch_reduce_slots(const uint16_t* partial, const int32_t* ids, int M, int D, int E,
                               int topk, uint16_t* out, int n_cu, hipStream_t stream,
                               const KernelEvents& ev)
{
    if (int64_t(M) * D == 0) return hipSuccess;
    if (topk < 1 || topk > 32) return hipErrorInvalidValue;
    const bool narrow = int64_t(M) * (D / 2) <= int64_t(n_cu) * 1024;
    const int64_t nv = int64_t(M) * (D / (narrow ? 2 : 8));
    int64_t blocks = (nv + 255) / 256;
    if (blocks > int64_t(n_cu) * 16) blocks = int64_t(n_cu) * 16;
    const dim3 grid{unsigned(blocks)};
    if (narrow) launch_reduce_vec<2>(grid, stream, ev, partial, ids, M, D, E, topk, out);
    else launch_reduce_vec<8>(grid, stream, ev, partial, ids, M, D, E, topk, out);
    return hipGetLastError();
}

}  // namespace moe
