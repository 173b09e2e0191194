// LDS-tiled grouped GEMMs for many routes per expert (prefill shapes), on the
// gfx950 block-scaled FP4 MFMA v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Same two stages as the streaming kernels (gemm1.hip / gemm2.hip hold the
// semantics and the passages of the pages they follow), tiled for operand
// reuse instead of streaming:
//   workgroup tile  256 sorted rows (one expert block, block_m = 256) x 256
//                   output columns; 8 waves as 4 x 2, each 64 rows x 128
//                   columns = 2 x 4 MFMA tiles of 32x32 (128 fp32 accumulators
//                   per lane);
//   K pipeline      K advances 128 elements per stage; 4 stages live in LDS
//                   (34 KiB each: A and B codes, A and B scales) and are filled
//                   by direct global->LDS loads (global_load_lds), so three
//                   stages are in flight while one is consumed, without
//                   staging registers;
//   LDS layout      codes as [16-row slice][32-element chunk][row%16][16 B]:
//                   a quarter-wave reads 256 contiguous bytes per fragment (no
//                   bank conflicts), and the prepared weight fragments already
//                   have this order, so B is copied verbatim.
// Per stage a wave issues 16 MFMAs of 32x32x64 (512 cycles) against 6 KiB of
// LDS fragment reads; the workgroup fetches 34 KiB per stage, 2 x 256 x 256 x
// 128 / 34 KiB = 480 FLOP per byte of L2 traffic.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kTThreads = 512;
constexpr int kTM = 256;                 // rows per tile (= block_m of this path)
constexpr int kTN = 256;                 // columns per tile
#ifndef MOE_TILE_STAGES
#define MOE_TILE_STAGES 4
#endif
constexpr int kStages = MOE_TILE_STAGES;
constexpr int kOffB = kTM * 64;          // A codes 16 KiB, then B codes 16 KiB
constexpr int kOffAS = kOffB + kTN * 64; // A scales: [row][4 B]
constexpr int kOffBS = kOffAS + kTM * 4; // B scales: [n64 group][lane][4 slices]
constexpr int kStageBytes = kOffBS + kTN * 4;
constexpr int kLoadsPerStage = 5;        // global_load_lds per wave per stage

size_t tile_lds_bytes() { return size_t(kStages) * kStageBytes; }

// Direct global->LDS loads.  Lane l's 16 (or 4) bytes land at LDS address
// m0 + l*16 (l*4); `lds_addr` must be wave-uniform.  They are issued from
// inline assembly so that the compiler does not treat them as LDS writes and
// drain the whole prefetch pipeline (s_waitcnt vmcnt(0)) before every LDS
// read; completion is tracked explicitly with wait_barrier<N>() instead.  m0
// is saved and restored around the load.
__device__ __forceinline__ uint32_t lds_address(const uint8_t* p)
{
    return uint32_t(uintptr_t((__attribute__((address_space(3))) const uint8_t*)(p)));
}
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(g), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_addr)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(g), "s"(lds_addr) : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding,
// then join the workgroup barrier (no other counters, no cache fences).
template <int N>
__device__ __forceinline__ void wait_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ v16f mfma_fp4_32x32x64(uint4 a, uint4 b, v16f c, uint32_t sa,
                                                   uint32_t sb)
{
    v8i A = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
    v8i B = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, int(sa), 0,
                                                            int(sb));
}

// Byte offset of (row, 32-element chunk c) in a [slice][chunk][row%16][16 B] tile.
__device__ __forceinline__ int tile_off(int row, int c) { return ((row >> 4) * 4 + c) * 256 + (row & 15) * 16; }

struct TileArgs {
    const uint8_t* a;          // A codes, sorted rows, fragment layout (a1f or a2q)
    const uint8_t* as;         // A scales, fragment layout (kt-major)
    const uint8_t* wp;         // prepared weight codes
    const uint8_t* wsp;        // prepared weight scales
    const int32_t* sorted_route;
    const float* sorted_w;
    const int32_t* block_expert;
    const int32_t* num_valid;
    const int32_t* expert_block0;   // [E+1] first block of each expert, then the used blocks
    int M, topk, N, K;         // N, K of one expert's weight matrix
    int64_t cap;               // rows of the sorted fragment-layout operands
    uint8_t* a2q;              // stage 1 outputs
    uint8_t* a2s;
    uint16_t* h_dbg;
    uint16_t* partial;         // stage 2 output [M*topk][N]
    uint64_t* clk;             // optional kernel span (stage 1)
};

// The per-wave source pointers of one stage's five loads; every load is a
// contiguous run (1 KiB of codes or 256 B of scales per wave).
struct StageSrc {
    const uint8_t* a_code[2];  // this lane's 16 B of A slices 2w, 2w+1 at kt = 0
    const uint8_t* b_code[2];  // this lane's 16 B of B pieces 2w, 2w+1 at kt = 0
    const uint8_t* scale;      // waves 0-3: A scale word of row 64w+lane; 4-7: B scale word
    int64_t scale_step;        // bytes per K tile of `scale`
};

// buf: LDS address of the stage buffer; wave: wave-uniform wave index.
__device__ __forceinline__ void issue_stage(const StageSrc& s, int kt, uint32_t buf, int wave)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) dma16(s.a_code[h] + int64_t(kt) * 1024, buf + (2 * wave + h) * 1024);
#pragma unroll
    for (int h = 0; h < 2; ++h) dma16(s.b_code[h] + int64_t(kt) * 4096, buf + kOffB + (2 * wave + h) * 1024);
    if (wave < 4) dma4(s.scale + kt * s.scale_step, buf + kOffAS + wave * 256);
    else dma4(s.scale + kt * s.scale_step, buf + kOffBS + (wave - 4) * 256);
}

// acc[mt][nt] += A[256 x K] . W[e][tile columns]^T over the whole K.
__device__ __forceinline__ void tile_mainloop(const StageSrc& src, int KT, uint8_t* lds,
                                              v16f acc[2][4])
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int wave_m = wave >> 1, wave_n = wave & 1;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(lds));
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < KT) issue_stage(src, s, lds0 + s * kStageBytes, wave);

    for (int kt = 0; kt < KT; ++kt) {
        // stage kt has landed once at most `ahead` later stages are pending
        const int ahead = min(KT - 1 - kt, kStages - 2);
        if (ahead >= 3) wait_barrier<3 * kLoadsPerStage>();
        else if (ahead == 2) wait_barrier<2 * kLoadsPerStage>();
        else if (ahead == 1) wait_barrier<kLoadsPerStage>();
        else wait_barrier<0>();
        if (kt + kStages - 1 < KT)
            issue_stage(src, kt + kStages - 1, lds0 + ((kt + kStages - 1) % kStages) * kStageBytes, wave);

        const uint8_t* buf = lds + (kt % kStages) * kStageBytes;
        uint32_t sa_word[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            sa_word[mt] = *reinterpret_cast<const uint32_t*>(buf + kOffAS + (wave_m * 64 + mt * 32 + (lane & 31)) * 4);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = 2 * jj + (lane >> 5);
            uint4 af[2], bf[4];
            uint32_t sb[4];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                af[mt] = *reinterpret_cast<const uint4*>(buf + tile_off(wave_m * 64 + mt * 32 + (lane & 31), c));
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int prow = wave_n * 128 + nt * 32 + (lane & 31);
                bf[nt] = *reinterpret_cast<const uint4*>(buf + kOffB + tile_off(prow, c));
                sb[nt] = buf[kOffBS + (prow >> 6) * 256 + (c * 16 + (prow & 15)) * 4 + ((prow >> 4) & 3)];
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint32_t sa = (sa_word[mt] >> (8 * c)) & 0xFFu;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = mfma_fp4_32x32x64(af[mt], bf[nt], acc[mt][nt], sa, sb[nt]);
            }
        }
    }
}

__device__ __forceinline__ void zero_acc(v16f acc[2][4])
{
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;
}

// B sources of this wave: pieces 2w, 2w+1 (1 KiB each) of the four 64-row
// groups n64 = ntile*4 + piece/4 at K tile 0; B scale word of group w-4.
__device__ __forceinline__ void b_sources(const TileArgs& p, int e, int ntile, StageSrc& s)
{
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int KT = p.K / 128;
    const uint8_t* wexp = p.wp + int64_t(e) * p.N * (p.K / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int piece = 2 * wave + h;
        s.b_code[h] = wexp + int64_t(ntile * 4 + piece / 4) * KT * 4096 + (piece % 4) * 1024 + lane * 16;
    }
    if (wave >= 4) {
        s.scale = p.wsp + int64_t(e) * p.N * (p.K / 32) + int64_t(ntile * 4 + wave - 4) * KT * 256 + lane * 4;
        s.scale_step = 256;
    }
}

// A sources of this wave: 16-row slices 2w, 2w+1 of the block's 256 sorted
// rows; A scale words of rows 64w .. 64w+63 (waves 0-3).
__device__ __forceinline__ void a_sources(const TileArgs& p, int blk, StageSrc& s)
{
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int KT = p.K / 128;
    const int64_t row0 = int64_t(blk) * kTM;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        s.a_code[h] = p.a + frag_code_off(row0 + (2 * wave + h) * 16, 0, 0, KT) + lane * 16;
    if (wave < 4) {
        s.scale = p.as + frag_scale_off(row0 + wave * 64 + lane, 0, p.cap);
        s.scale_step = p.cap * 4;
    }
}

// Tile order.  The dispatcher deals workgroups to the XCDs round-robin by id
// and each XCD has its own L2, so workgroup w runs on XCD w % 8 as that
// XCD's (w / 8)-th.  Each XCD takes an equal contiguous share of the used
// tiles, ordered expert by expert and, inside an expert, column tile by
// column tile across the expert's row blocks: the workgroups resident on
// one XCD at a time share an expert's weight tiles and activation blocks
// in their L2 instead of every XCD fetching every block.  The grid is
// rounded up to a multiple of 8 (tile_grid), so every share fits.

// Column tile, block and expert of this workgroup; false past the used tiles.
__device__ __forceinline__ bool tile_of(const TileArgs& p, int n_tiles, int& ntile, int& blk,
                                        int& e)
{
    const int w = blockIdx.x;
    const int xcd = w % kXcds, j = w / kXcds;
    const int64_t used = int64_t(n_tiles) * (p.num_valid[0] / kTM);
    const int64_t lo = used * xcd / kXcds, hi = used * (xcd + 1) / kXcds;
    const int64_t t = lo + j;
    if (t >= hi) return false;
    e = p.block_expert[t / n_tiles];
    const int first = p.expert_block0[e];
    const int nb = p.expert_block0[e + 1] - first;
    const int local = int(t - int64_t(n_tiles) * first);
    ntile = local / nb;
    blk = first + local % nb;
    return true;
}

// ------------------------------------------------------------ stage 1 ----

__global__ void __launch_bounds__(kTThreads, 1)
gemm1_tile_kernel(TileArgs p, int I)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    span_begin(p.clk);
    int ntile, blk, e;
    if (!tile_of(p, p.N / kTN, ntile, blk, e)) {
        span_end(p.clk);
        return;
    }
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wave_m = wave >> 1, wave_n = wave & 1;

    // A: the sorted, fragment-layout copy of the activations (gather kernel)
    StageSrc src;
    a_sources(p, blk, src);
    b_sources(p, e, ntile, src);

    v16f acc[2][4];
    zero_acc(acc);
    tile_mainloop(src, p.K / 128, lds, acc);

    // Epilogue: the wave's N tiles are (gate, up) of h groups hg0 and hg0 + 1
    // (prepared 64-row group = 32 gate rows then 32 up rows).
    const int hg0 = ntile * 4 + wave_n * 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            const int hg = hg0 + gi;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = wave_m * 64 + mt * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                const int64_t srow = int64_t(blk) * kTM + row;
                const uint32_t h = f32_to_bf16_rne(silu_fast(acc[mt][2 * gi][i]) * acc[mt][2 * gi + 1][i]);
                if (p.h_dbg) p.h_dbg[srow * I + hg * 32 + (lane & 31)] = uint16_t(h);
                // MXFP4 group: the 32 columns of this row held by one half-wave
                // (DPP rows 0-1 or 2-3); the two row maxima meet via readlane
                const uint32_t rmax = row16_max(h & 0x7FFFu);
                const uint32_t m01 = max(uint32_t(__builtin_amdgcn_readlane(int(rmax), 0)),
                                         uint32_t(__builtin_amdgcn_readlane(int(rmax), 16)));
                const uint32_t m23 = max(uint32_t(__builtin_amdgcn_readlane(int(rmax), 32)),
                                         uint32_t(__builtin_amdgcn_readlane(int(rmax), 48)));
                const uint32_t s = mx_scale_from_amax(lane < 32 ? m01 : m23);
                const uint32_t p4 = pack8_codes(mx_code(h, s));
                if ((lane & 7) == 0)
                    *reinterpret_cast<uint32_t*>(p.a2q + frag_code_off(srow, hg / 4, hg % 4, I / 128) +
                                                 ((lane & 31) >> 3) * 4) = p4;
                if ((lane & 31) == 0) p.a2s[frag_scale_off(srow, hg / 4, p.cap) + hg % 4] = uint8_t(s);
            }
        }
    }
    span_end(p.clk);
}

// ------------------------------------------------------------ stage 2 ----

__global__ void __launch_bounds__(kTThreads, 1)
gemm2_tile_kernel(TileArgs p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int32_t s_route[kTM];
    __shared__ float s_w[kTM];
    int ntile, blk, e;
    if (!tile_of(p, p.N / kTN, ntile, blk, e)) return;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wave_m = wave >> 1, wave_n = wave & 1;
    const int R = p.M * p.topk;
    const int D = p.N;
    if (tid < kTM) {
        s_route[tid] = p.sorted_route[blk * kTM + tid];
        s_w[tid] = p.sorted_w[blk * kTM + tid];
    }
    __syncthreads();
    StageSrc src;
    a_sources(p, blk, src);
    b_sources(p, e, ntile, src);

    v16f acc[2][4];
    zero_acc(acc);
    tile_mainloop(src, p.K / 128, lds, acc);

#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = wave_m * 64 + mt * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
            const int sr = s_route[row];
            const float w = s_w[row];
            uint16_t* dst = p.partial + int64_t(sr) * D + ntile * kTN + wave_n * 128 + (lane & 31);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                // columns lane%32 and lane%32 + 1 as one dword from the even lane
                const uint32_t v = f32_to_bf16_rne(w * acc[mt][nt][i]);
                const uint32_t pair = v | (dpp<kDppXor1>(v) << 16);
                if (sr < R && (lane & 1) == 0) *reinterpret_cast<uint32_t*>(dst + nt * 32) = pair;
            }
        }
    }
}

hipError_t tile_allow_lds()
{
    const int bytes = int(tile_lds_bytes());
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm1_tile_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm2_tile_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_gemm1_tile(const Gemm1Args& a, hipStream_t stream, const KernelEvents& ev)
{
    if (a.nb_cap == 0) return hipSuccess;
    if (a.block_m != kTM || (2 * a.I) % kTN != 0) return hipErrorInvalidValue;
    if (!a.expert_block0) return hipErrorInvalidValue;
    TileArgs p{a.a1f, a.a1fs, a.w13p, a.w13sp, a.sorted_route, nullptr, a.block_expert,
               a.num_valid, a.expert_block0, a.M, a.topk, 2 * a.I, a.D, a.cap, a.a2q, a.a2s,
               a.h_dbg, nullptr, a.clk};
    MOE_LAUNCH(gemm1_tile_kernel, dim3(tile_grid(2 * a.I / kTN, a.nb_cap)), dim3(kTThreads),
               uint32_t(tile_lds_bytes()), stream, ev, p, a.I);
    return hipGetLastError();
}

hipError_t launch_gemm2_tile(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev)
{
    if (a.nb_cap == 0) return hipSuccess;
    if (a.block_m != kTM || a.D % kTN != 0) return hipErrorInvalidValue;
    if (!a.expert_block0) return hipErrorInvalidValue;
    TileArgs p{a.a2q, a.a2s, a.w2p, a.w2sp, a.sorted_route, a.sorted_w, a.block_expert,
               a.num_valid, a.expert_block0, a.M, a.topk, a.D, a.I, a.cap, nullptr, nullptr,
               nullptr, a.partial, nullptr};
    MOE_LAUNCH(gemm2_tile_kernel, dim3(tile_grid(a.D / kTN, a.nb_cap)), dim3(kTThreads),
               uint32_t(tile_lds_bytes()), stream, ev, p);
    return hipGetLastError();
}

}  // namespace moe
