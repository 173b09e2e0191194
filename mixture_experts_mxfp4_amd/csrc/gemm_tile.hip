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
//                   by direct global->LDS loads (global_load_lds) issued three
//                   stages ahead, without staging registers;
//   schedule        each stage's loads, LDS fragment reads and barrier sit
//                   between its MFMAs in a fixed order (tile_step), so the
//                   matrix cores are never left waiting on them;
//   LDS layout      codes as [16-row slice][32-element chunk][row%16][16 B]:
//                   a quarter-wave reads 256 contiguous bytes per fragment (no
//                   bank conflicts), and the prepared weight fragments already
//                   have this order, so B is copied verbatim.
// Per stage a wave issues 16 MFMAs of 32x32x64 (512 cycles) against 6 KiB of
// LDS fragment reads; the workgroup fetches 34 KiB per stage, 2 x 256 x 256 x
// 128 / 34 KiB = 480 FLOP per byte of L2 traffic.
#include <algorithm>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kTThreads = 512;
constexpr int kTM = 256;                 // rows per tile (= block_m of this path)
constexpr int kTN = 256;                 // columns per tile
constexpr int kStages = 4;
constexpr int kOffB = kTM * 64;          // A codes 16 KiB, then B codes 16 KiB
constexpr int kOffAS = kOffB + kTN * 64; // A scales: [row][4 B]
constexpr int kOffBS = kOffAS + kTM * 4; // B scales: [n64 group][lane][4 slices]
constexpr int kStageBytes = kOffBS + kTN * 4;
constexpr int kLoadsPerStage = 5;        // global_load_lds per wave per stage
// MFMAs of a step's second half issued before its barrier: they use only
// fragments read in the first half (the compiler waits for just the ones each
// needs), and keep the matrix cores busy while the waves meet; the reads of
// the next stage come after the barrier.  Two measured best (0-4 tried).
constexpr int kPreMfma = 2;
// Stage-2 epilogue staging in the (then idle) ring: rows padded by 16 B so
// that consecutive rows start 4 banks apart.
constexpr int kPStride = kTN * 2 + 16;   // 256 bf16 output columns per row
static_assert(kTM * kPStride <= kStages * kStageBytes, "epilogue staging must fit in the ring");

size_t tile_lds_bytes() { return size_t(kStages) * kStageBytes; }

__device__ __forceinline__ uint32_t lds_address(const uint8_t* p)
{
    return uint32_t(uintptr_t((__attribute__((address_space(3))) const uint8_t*)(p)));
}

// A wave-uniform pointer as the compiler's uniform value (SGPR pair).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return reinterpret_cast<const uint8_t*>((uint64_t(hi) << 32) | lo);
}

// Direct global->LDS loads from a wave-uniform 64-bit base (SGPRs) plus a
// 32-bit per-lane byte offset.  Lane l's 16 (or 4) bytes land at LDS address
// m0 + l*16 (l*4); `lds_addr` must be wave-uniform.  They are issued from
// inline assembly so that the compiler does not treat them as LDS writes and
// drain the whole prefetch pipeline (s_waitcnt vmcnt(0)) before every LDS
// read; completion is tracked explicitly with wait_barrier<N>() instead.  m0
// is saved and restored around the load.
__device__ __forceinline__ void dma16s(const uint8_t* base, uint32_t off, uint32_t lds_addr)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(off), "s"(base), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4s(const uint8_t* base, uint32_t off, uint32_t lds_addr)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(off), "s"(base), "s"(lds_addr) : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding,
// then join the workgroup barrier (no other counters, no cache fences).
template <int N>
__device__ __forceinline__ void wait_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Block-scaled FP4 MFMA whose scale bytes are picked from 32-bit words by the
// instruction's byte selects (SA, SB: byte 0..3 of sa, sb).
template <int SA, int SB>
__device__ __forceinline__ v16f mfma_fp4_sel(uint4 a, uint4 b, v16f c, uint32_t sa, uint32_t sb)
{
    v8i A = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
    v8i B = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, SA, int(sa), SB, int(sb));
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
    const int32_t* num_valid;
    const int4* block_info;    // per used block: expert, its first block, block count, routes
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
// Wave-uniform 64-bit bases (held in SGPRs) and 32-bit per-lane offsets.
struct StageSrc {
    const uint8_t* a_base;     // the block's A codes
    const uint8_t* b_base;     // the expert's prepared weight codes
    const uint8_t* s_base;     // waves 0-3: the block's A scale words; 4-7: B scale words
    uint32_t a_off[2];         // this lane's 16 B of A slices 2w, 2w+1 at kt = 0
    uint32_t b_off[2];         // this lane's 16 B of B pieces 2w, 2w+1 at kt = 0
    uint32_t s_off;            // this lane's scale word at kt = 0
    uint32_t s_step;           // bytes per K tile of the scale words
    uint32_t scale_lds;        // byte offset of this wave's scale words in a stage buffer
};

// Load d (0-4) of this wave for K tile kt into the stage buffer at LDS address
// `buf`; wave: wave-uniform wave index.
__device__ __forceinline__ void issue_load(const StageSrc& s, int kt, int d, uint32_t buf, int wave)
{
    if (d < 2) dma16s(s.a_base, s.a_off[d] + uint32_t(kt) * 1024u, buf + (2 * wave + d) * 1024);
    else if (d < 4) dma16s(s.b_base, s.b_off[d - 2] + uint32_t(kt) * 4096u, buf + kOffB + (2 * wave + d - 2) * 1024);
    else dma4s(uniform_ptr(s.s_base), s.s_off + uint32_t(kt) * s.s_step,
               __builtin_amdgcn_readfirstlane(buf + s.scale_lds));
}

// MFMA operands of one 64-deep K half for a wave's 64 x 128 tile.
struct HalfFrags {
    uint4 a[2], b[4];
};

// Fragment i (0-1: A tile i, 2-5: B tile i-2) of K half jj from stage buffer buf.
__device__ __forceinline__ void read_frag(const uint8_t* buf, int jj, int wave_m, int wave_n, int lane,
                                          HalfFrags& f, int i)
{
    const int c = 2 * jj + (lane >> 5);
    if (i < 2) f.a[i] = *reinterpret_cast<const uint4*>(buf + tile_off(wave_m * 64 + i * 32 + (lane & 31), c));
    else f.b[i - 2] = *reinterpret_cast<const uint4*>(buf + kOffB + tile_off(wave_n * 128 + (i - 2) * 32 + (lane & 31), c));
}

// Scale words.  A: the four chunk scales of row wave_m*64 + mt*32 + lane%32 (byte c
// = chunk).  B: the prepared word of group wave_n*2 + g for chunk 2jj + lane/32 and
// row lane%16, which holds the scales of the group's four 16-row slices; MFMA tile nt
// of this lane uses slice 2(nt%2) + (lane/16)%2 of group wave_n*2 + nt/2.
__device__ __forceinline__ uint32_t read_sa(const uint8_t* buf, int wave_m, int lane, int mt)
{
    return *reinterpret_cast<const uint32_t*>(buf + kOffAS + (wave_m * 64 + mt * 32 + (lane & 31)) * 4);
}
__device__ __forceinline__ uint32_t read_sb(const uint8_t* buf, int wave_n, int lane, int jj, int g)
{
    const int c = 2 * jj + (lane >> 5);
    return *reinterpret_cast<const uint32_t*>(buf + kOffBS + (wave_n * 2 + g) * 256 + (c * 16 + (lane & 15)) * 4);
}

// acc[mt][nt] += A[256 x K] . W[e][tile columns]^T over the whole K.
//
// One K tile (stage) per step, in two halves of eight MFMAs.  The instruction
// stream of a step is fixed (sched_barrier fences): between the MFMAs of half 0
// the wave issues its five loads of stage kt+3 (whose ring slot was last read
// before the previous step's barrier) and reads half 1's fragments; it issues
// the first kPreMfma MFMAs of half 1, waits for its LDS reads and for its loads
// of stage kt+1, and joins the barrier; between the remaining MFMAs of half 1
// it reads half 0 of stage kt+1.  So the matrix cores always have the next
// MFMA queued while loads, LDS reads and the barrier are in flight.  The scale
// words are shifted once per stage to this lane's byte pair and the MFMA byte
// selects pick chunk and slice.
template <bool kLoad, bool kSwap>
__device__ __forceinline__ void tile_step(const StageSrc& src, int KT, int kt, uint8_t* lds,
                                          uint32_t lds0, int wave, int lane, v16f acc[2][4],
                                          HalfFrags& f0, HalfFrags& f1, uint32_t sa[2],
                                          uint32_t sb0[2])
{
    const int wave_m = wave >> 1, wave_n = wave & 1;
    const uint8_t* cur = lds + (kt % kStages) * kStageBytes;
    const uint8_t* nxt = lds + ((kt + 1) % kStages) * kStageBytes;
    const uint32_t load_buf = lds0 + ((kt + kStages - 1) % kStages) * kStageBytes;
    uint32_t sb1[2], sa_next[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) sa[m] >>= 8 * (lane >> 5);
#pragma unroll
    for (int g = 0; g < 2; ++g) sb0[g] >>= 8 * ((lane >> 4) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int mt = i >> 2, nt = i & 3;
        if constexpr (kSwap)
            acc[mt][nt] = (nt & 1) ? mfma_fp4_sel<2, 0>(f0.b[nt], f0.a[mt], acc[mt][nt], sb0[nt >> 1], sa[mt])
                                   : mfma_fp4_sel<0, 0>(f0.b[nt], f0.a[mt], acc[mt][nt], sb0[nt >> 1], sa[mt]);
        else
            acc[mt][nt] = (nt & 1) ? mfma_fp4_sel<0, 2>(f0.a[mt], f0.b[nt], acc[mt][nt], sa[mt], sb0[nt >> 1])
                                   : mfma_fp4_sel<0, 0>(f0.a[mt], f0.b[nt], acc[mt][nt], sa[mt], sb0[nt >> 1]);
        if (kLoad && i < kLoadsPerStage) issue_load(src, kt + kStages - 1, i, load_buf, wave);
        if (i == 0) {
            sb1[0] = read_sb(cur, wave_n, lane, 1, 0);
            sb1[1] = read_sb(cur, wave_n, lane, 1, 1);
        }
        if (i >= 1 && i < 7) read_frag(cur, 1, wave_m, wave_n, lane, f1, i - 1);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) sb1[g] >>= 8 * ((lane >> 4) & 1);
    auto mfma1 = [&](int i) {
        const int mt = i >> 2, nt = i & 3;
        if constexpr (kSwap)
            acc[mt][nt] = (nt & 1) ? mfma_fp4_sel<2, 2>(f1.b[nt], f1.a[mt], acc[mt][nt], sb1[nt >> 1], sa[mt])
                                   : mfma_fp4_sel<0, 2>(f1.b[nt], f1.a[mt], acc[mt][nt], sb1[nt >> 1], sa[mt]);
        else
            acc[mt][nt] = (nt & 1) ? mfma_fp4_sel<2, 2>(f1.a[mt], f1.b[nt], acc[mt][nt], sa[mt], sb1[nt >> 1])
                                   : mfma_fp4_sel<2, 0>(f1.a[mt], f1.b[nt], acc[mt][nt], sa[mt], sb1[nt >> 1]);
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPreMfma; ++i) {
        mfma1(i);
        __builtin_amdgcn_sched_barrier(0);
    }
    // this wave's LDS reads of stage kt are done, and its loads of stage kt+1
    // have landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (kLoad) {
        wait_barrier<2 * kLoadsPerStage>();          // stages kt+2, kt+3 may be in flight
    } else if (kt + 2 < KT) {
        wait_barrier<kLoadsPerStage>();              // stage kt+2 may be in flight
    } else {
        wait_barrier<0>();
    }
    __builtin_amdgcn_sched_barrier(0);
    // the remaining MFMAs carry the reads of stage kt+1 (scale words first,
    // so they have landed when the next step shifts them); after the last
    // stage these read a ring slot whose contents go unused
    constexpr int kSlots = 8 - kPreMfma;
    static_assert(kSlots >= 3, "two scale-word slots and at least one fragment slot");
#pragma unroll
    for (int i = kPreMfma; i < 8; ++i) {
        mfma1(i);
        const int slot = i - kPreMfma;          // A scale words, B scale words, then fragments
        if (slot == 0) {
            sa_next[0] = read_sa(nxt, wave_m, lane, 0);
            sa_next[1] = read_sa(nxt, wave_m, lane, 1);
        }
        if (slot == 1) {
            sb0[0] = read_sb(nxt, wave_n, lane, 0, 0);
            sb0[1] = read_sb(nxt, wave_n, lane, 0, 1);
        }
#pragma unroll
        for (int j = 0; j < 6; ++j)
            if (slot >= 2 && 2 + j * (kSlots - 2) / 6 == slot) read_frag(nxt, 0, wave_m, wave_n, lane, f0, j);
        __builtin_amdgcn_sched_barrier(0);
    }
    sa[0] = sa_next[0];
    sa[1] = sa_next[1];
}

// kSwap: the weights are the MFMA's first operand, so acc[mt][nt] holds the
// transposed 32x32 tile (lane: row mt*32 + lane%32 of the wave's rows,
// element i: column (i/4)*8 + (lane/32)*4 + i%4 of N tile nt).
template <bool kSwap>
__device__ __forceinline__ void tile_mainloop(const StageSrc& src, int KT, uint8_t* lds,
                                              v16f acc[2][4])
{
    static_assert(kStages == 4, "the waits below assume three stages in flight");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int wave_m = wave >> 1, wave_n = wave & 1;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(lds));
    const int pre = min(KT, kStages - 1);
    for (int s = 0; s < pre; ++s)
        for (int d = 0; d < kLoadsPerStage; ++d) issue_load(src, s, d, lds0 + s * kStageBytes, wave);
    // stage 0 has landed once at most pre - 1 later stages are pending
    if (pre == 3) wait_barrier<2 * kLoadsPerStage>();
    else if (pre == 2) wait_barrier<kLoadsPerStage>();
    else wait_barrier<0>();

    HalfFrags f0, f1;
    uint32_t sa[2], sb0[2];
#pragma unroll
    for (int i = 0; i < 6; ++i) read_frag(lds, 0, wave_m, wave_n, lane, f0, i);
    sa[0] = read_sa(lds, wave_m, lane, 0);
    sa[1] = read_sa(lds, wave_m, lane, 1);
    sb0[0] = read_sb(lds, wave_n, lane, 0, 0);
    sb0[1] = read_sb(lds, wave_n, lane, 0, 1);

    int kt = 0;
#pragma unroll 1
    for (; kt + kStages - 1 < KT; ++kt)
        tile_step<true, kSwap>(src, KT, kt, lds, lds0, wave, lane, acc, f0, f1, sa, sb0);
#pragma unroll 1
    for (; kt < KT; ++kt)
        tile_step<false, kSwap>(src, KT, kt, lds, lds0, wave, lane, acc, f0, f1, sa, sb0);
}

// Main loop of a wave whose 64 rows are all padding (an expert's routes come
// first in its segment, so a block's padding rows are its last ones).  It
// still issues its share of the B-tile and scale loads (its A slices are
// rows of its own padding group) and joins every barrier, but reads no
// fragments and issues no MFMAs, leaving its SIMD's matrix core to the
// other wave there.  Its sums stay zero.
constexpr int kIdleLoads = kLoadsPerStage - 2;     // loads 2..4 of issue_load
__device__ __forceinline__ void tile_mainloop_idle(const StageSrc& src, int KT, uint8_t* lds)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(lds));
    const int pre = min(KT, kStages - 1);
    for (int s = 0; s < pre; ++s)
        for (int d = 2; d < kLoadsPerStage; ++d) issue_load(src, s, d, lds0 + s * kStageBytes, wave);
    if (pre == 3) wait_barrier<2 * kIdleLoads>();
    else if (pre == 2) wait_barrier<kIdleLoads>();
    else wait_barrier<0>();
#pragma unroll 1
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + kStages - 1 < KT) {
            const uint32_t buf = lds0 + ((kt + kStages - 1) % kStages) * kStageBytes;
            for (int d = 2; d < kLoadsPerStage; ++d) issue_load(src, kt + kStages - 1, d, buf, wave);
            wait_barrier<2 * kIdleLoads>();
        } else if (kt + 2 < KT) {
            wait_barrier<kIdleLoads>();
        } else {
            wait_barrier<0>();
        }
    }
}

// Whether this wave's 64 rows of a block with `valid` routes hold any route
// (an expert's routes fill its segment first, padding comes last).
__device__ __forceinline__ bool rows_in_use(int valid, int wave_m) { return valid > wave_m * 64; }

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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int KT = p.K / 128;
    s.b_base = uniform_ptr(p.wp + int64_t(e) * p.N * (p.K / 2));   // < 2^31 bytes per expert
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int piece = 2 * wave + h;
        s.b_off[h] = uint32_t((ntile * 4 + piece / 4) * KT * 4096 + (piece % 4) * 1024 + lane * 16);
    }
    if (wave >= 4) {
        s.s_base = uniform_ptr(p.wsp + int64_t(e) * p.N * (p.K / 32) + int64_t(ntile * 4 + wave - 4) * KT * 256);
        s.s_off = uint32_t(lane * 4);
        s.s_step = 256;
        s.scale_lds = uint32_t(kOffBS + (wave - 4) * 256);
    }
}

// A sources of this wave: 16-row slices 2w, 2w+1 of the block's 256 sorted
// rows; A scale words of rows 64w .. 64w+63 (waves 0-3).
__device__ __forceinline__ void a_sources(const TileArgs& p, int blk, StageSrc& s)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int KT = p.K / 128;
    const int64_t row0 = int64_t(blk) * kTM;
    s.a_base = uniform_ptr(p.a + frag_code_off(row0, 0, 0, KT));   // the block: 256 * K/2 bytes
#pragma unroll
    for (int h = 0; h < 2; ++h)
        s.a_off[h] = uint32_t(frag_code_off((2 * wave + h) * 16, 0, 0, KT) + lane * 16);
    if (wave < 4) {
        s.s_base = uniform_ptr(p.as + frag_scale_off(row0, 0, p.cap));
        s.s_off = uint32_t((wave * 64 + lane) * 4);
        s.s_step = uint32_t(p.cap * 4);
        s.scale_lds = uint32_t(kOffAS + wave * 256);
    }
}

// Tile order.  The dispatcher deals workgroups to the XCDs round-robin by id
// and each XCD has its own L2, so workgroup w runs on XCD w % 8 as that
// XCD's (w / 8)-th.  Each XCD takes an equal contiguous share of the used
// tiles, ordered expert by expert and, inside an expert, column tile by
// column tile across the expert's row blocks: the workgroups resident on
// one XCD at a time share an expert's weight tiles and activation blocks
// in their L2 instead of every XCD fetching every block.  Both kernels are
// persistent: one workgroup per CU (tile_persistent_grid, a multiple of 8)
// walks its XCD's share with a stride of the XCD's workgroup count, so the
// workgroups resident on an XCD at a time take consecutive tiles; a new
// tile's ring fill then follows the previous tile's epilogue on the same CU
// without a workgroup launch in between.

// This workgroup's XCD share [lo, hi) of the used tiles and its index j in
// that XCD.
__device__ __forceinline__ void xcd_share(const TileArgs& p, int n_tiles, int64_t& lo, int64_t& hi,
                                          int& j)
{
    const int w = blockIdx.x;
    const int xcd = w % kXcds;
    j = w / kXcds;
    const int64_t used = int64_t(n_tiles) * (p.num_valid[0] / kTM);
    lo = used * xcd / kXcds;
    hi = used * (xcd + 1) / kXcds;
}

// One 16-byte record of the sort at a wave-uniform address, through the
// scalar cache and waited for inside the asm block.  A vector load here
// would make the compiler wait for every older vector-memory operation of the
// wave (s_waitcnt vmcnt(0)), a persistent workgroup's previous stores
// included.
__device__ __forceinline__ int4 load_record(const int4* rec)
{
    typedef int v4i_t __attribute__((ext_vector_type(4)));
    // both halves as unsigned 32-bit words (uniform_ptr): readfirstlane
    // returns int, which would sign-extend the low word into the high one
    const uint8_t* au = uniform_ptr(reinterpret_cast<const uint8_t*>(rec));
    v4i_t v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(au) : "memory");
    return make_int4(v.x, v.y, v.z, v.w);
}

// Column tile, block, expert and the block's number of routes for tile t of
// the order above: one 16-byte record of the sort (tiles t of an expert's
// n_tiles * nb run lie within its blocks' records).
__device__ __forceinline__ void tile_at(const TileArgs& p, int n_tiles, int64_t t, int& ntile,
                                        int& blk, int& e, int& valid)
{
    const int4 bi = load_record(p.block_info + t / n_tiles);
    e = bi.x;
    const int first = bi.y, nb = bi.z;
    const int local = int(t - int64_t(n_tiles) * first);
    ntile = local / nb;
    blk = first + local % nb;
    valid = min(kTM, bi.w - (blk - first) * kTM);
}

// ------------------------------------------------------------ stage 1 ----

__global__ void __launch_bounds__(kTThreads, 1)
gemm1_tile_kernel(TileArgs p, int I)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    span_begin(p.clk);
    const int n_tiles = p.N / kTN;
    int64_t lo, hi;
    int jx;                                  // this workgroup's index in its XCD
    xcd_share(p, n_tiles, lo, hi, jx);
    const int per_xcd = int(gridDim.x) / kXcds;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wave_m = wave >> 1, wave_n = wave & 1;
#pragma unroll 1
    for (int64_t t = lo + jx; t < hi; t += per_xcd) {
        int ntile, blk, e, valid;
        tile_at(p, n_tiles, t, ntile, blk, e, valid);

        // A: the sorted, fragment-layout copy of the activations (gather kernel)
        StageSrc src;
        a_sources(p, blk, src);
        b_sources(p, e, ntile, src);

        v16f acc[2][4];
        zero_acc(acc);
        if (rows_in_use(valid, wave_m)) tile_mainloop<true>(src, p.K / 128, lds, acc);
        else tile_mainloop_idle(src, p.K / 128, lds);

        // Epilogue.  The wave's N tiles are (gate, up) of h groups wave_n*2 and
        // wave_n*2 + 1 of the tile (prepared 64-row group = 32 gate rows then 32 up
        // rows: gate and up of an h column sit at the same place of tiles 2gi and
        // 2gi+1); the tile's 128 h columns are K tile `ntile` of stage 2.  With the
        // swapped product a lane holds, for row mt*32 + lane%32, 16 of the 32
        // columns of an MXFP4 block (columns (i/4)*8 + (lane/32)*4 + i%4) and lane
        // lane^32 the other 16: the block maximum takes one exchange, and after a
        // second each half stores 8 contiguous code bytes of the row's 16-byte chunk
        // (lanes < 32 bytes 0-7, lanes >= 32 bytes 8-15).
        const bool upper = lane >= 32;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int64_t srow = int64_t(blk) * kTM + wave_m * 64 + mt * 32 + (lane & 31);
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                const int c = wave_n * 2 + gi;               // 32-column chunk in K tile `ntile`
                // h of element pairs (2j, 2j+1) as packed bf16; block maximum on
                // the 15-bit magnitudes, two per packed 16-bit max
                typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
                uint32_t hp[8];
                u16x2_t m2 = {0, 0};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    hp[j] = f32x2_to_bf16x2(silu_fast(acc[mt][2 * gi][2 * j]) * acc[mt][2 * gi + 1][2 * j],
                                            silu_fast(acc[mt][2 * gi][2 * j + 1]) * acc[mt][2 * gi + 1][2 * j + 1]);
                    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, hp[j] & 0x7FFF7FFFu));
                }
                uint32_t amax = max(uint32_t(m2.x), uint32_t(m2.y));
                amax = max(amax, uint32_t(__shfl_xor(int(amax), 32)));
                const uint32_t s = mx_scale_from_amax(amax);
                const float so = mx_scale_operand(s);
                // element pair j of this lane's 16 -> chunk byte (j/2)*4 + (lane/32)*2 + j%2:
                // bytes of pairs 0-3 in `lo`, of pairs 4-7 in `hi`
                uint32_t lo = 0, hi = 0;
                lo = mx_code_pair<0>(lo, hp[0], so);
                lo = mx_code_pair<1>(lo, hp[1], so);
                lo = mx_code_pair<2>(lo, hp[2], so);
                lo = mx_code_pair<3>(lo, hp[3], so);
                hi = mx_code_pair<0>(hi, hp[4], so);
                hi = mx_code_pair<1>(hi, hp[5], so);
                hi = mx_code_pair<2>(hi, hp[6], so);
                hi = mx_code_pair<3>(hi, hp[7], so);
                // lanes < 32 hold chunk bytes {0,1,4,5} and {8,9,12,13}, lanes >= 32
                // {2,3,6,7} and {10,11,14,15}
                const uint32_t recv = uint32_t(__shfl_xor(int(upper ? lo : hi), 32));
                uint2 out;
                if (!upper) {
                    out.x = (lo & 0xFFFFu) | (recv << 16);
                    out.y = (lo >> 16) | (recv & 0xFFFF0000u);
                } else {
                    out.x = (recv & 0xFFFFu) | (hi << 16);
                    out.y = (recv >> 16) | (hi & 0xFFFF0000u);
                }
                *reinterpret_cast<uint2*>(p.a2q + frag_code_off(srow, ntile, c, I / 128) + (upper ? 8 : 0)) = out;
                if (!upper) p.a2s[frag_scale_off(srow, ntile, p.cap) + c] = uint8_t(s);
                if (p.h_dbg) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        p.h_dbg[srow * I + ntile * 128 + c * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3)] =
                            uint16_t(hp[i >> 1] >> (16 * (i & 1)));
                }
            }
        }
        // the next tile's loads overwrite the ring: every wave is past this
        // tile's LDS reads (the stores stay in flight)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    span_end(p.clk);
}

// ------------------------------------------------------------ stage 2 ----

// Persistent: one workgroup per CU walks its XCD's share of the tiles with a
// stride of the XCD's workgroup count, so the workgroups resident on an XCD
// at a time still take consecutive tiles.  The partial-row stores of a tile
// are issued before the next tile's first loads and are not waited for: the
// next tile's ring waits (s_waitcnt vmcnt(N)) only need its own loads, which
// complete in issue order after the older stores.  With one tile per
// workgroup, every workgroup drained its 256 KiB of stores before the CU
// could start the next tile (58 us of the kernel's time at 4,096 tokens).
__global__ void __launch_bounds__(kTThreads, 1)
gemm2_tile_kernel(TileArgs p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int32_t s_route[kTM];
    __shared__ float s_w[kTM];
    span_begin(p.clk);
    const int n_tiles = p.N / kTN;
    int64_t lo, hi;
    int jx;                                  // this workgroup's index in its XCD
    xcd_share(p, n_tiles, lo, hi, jx);
    const int per_xcd = int(gridDim.x) / kXcds;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wave_m = wave >> 1, wave_n = wave & 1;
    const int R = p.M * p.topk;
    const int D = p.N;
#pragma unroll 1
    for (int64_t t = lo + jx; t < hi; t += per_xcd) {
        int ntile, blk, e, valid;
        tile_at(p, n_tiles, t, ntile, blk, e, valid);
        // the rows' routes (waves 0-3) and weights (waves 4-7) go straight to
        // LDS ahead of the first K stages; the main loop's waits cover them
        {
            const int q = wave & 3;
            const uint8_t* base = wave < 4 ? reinterpret_cast<const uint8_t*>(p.sorted_route)
                                           : reinterpret_cast<const uint8_t*>(p.sorted_w);
            const uint8_t* dst = wave < 4 ? reinterpret_cast<const uint8_t*>(s_route)
                                          : reinterpret_cast<const uint8_t*>(s_w);
            dma4s(uniform_ptr(base + (int64_t(blk) * kTM + q * kWave) * 4), uint32_t(lane * 4),
                  __builtin_amdgcn_readfirstlane(lds_address(dst) + q * kWave * 4));
        }
        StageSrc src;
        a_sources(p, blk, src);
        b_sources(p, e, ntile, src);

        v16f acc[2][4];
        zero_acc(acc);
        if (rows_in_use(valid, wave_m)) tile_mainloop<true>(src, p.K / 128, lds, acc);
        else tile_mainloop_idle(src, p.K / 128, lds);

        // Epilogue: the routing weight times the sum, rounded to bf16, goes
        // through LDS as the 256 x 256 tile; then each half-wave stores one
        // row's 512 contiguous bytes into its route's partial row (padding rows
        // are skipped).  With the swapped product a lane holds one row (mt*32 +
        // lane%32 of the wave's 64) and, per group of four elements, four
        // consecutive columns: one routing weight per row tile and 8-byte LDS
        // writes.
        uint8_t* ps = lds;                                   // [256 rows][kPStride]
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int row = wave_m * 64 + mt * 32 + (lane & 31);
            const float w = s_w[row];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = wave_n * 128 + nt * 32 + q * 8 + (lane >> 5) * 4;
                    uint2 v;
                    v.x = f32x2_to_bf16x2(w * acc[mt][nt][4 * q], w * acc[mt][nt][4 * q + 1]);
                    v.y = f32x2_to_bf16x2(w * acc[mt][nt][4 * q + 2], w * acc[mt][nt][4 * q + 3]);
                    *reinterpret_cast<uint2*>(ps + row * kPStride + col * 2) = v;
                }
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < kTM / 16; ++k) {
            const int row = wave * (kTM / 8) + 2 * k + (lane >> 5);
            const int sr = s_route[row];
            const uint4 v = *reinterpret_cast<const uint4*>(ps + row * kPStride + (lane & 31) * 16);
            if (sr < R)
                *reinterpret_cast<uint4*>(p.partial + int64_t(sr) * D + ntile * kTN + (lane & 31) * 8) = v;
        }
        // the next tile's loads overwrite the ring and s_route: every wave's
        // LDS reads of this tile are done (the stores stay in flight)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    span_end(p.clk);
}

unsigned tile_persistent_grid(int n_tiles, int nb_cap, int n_cu)
{
    const unsigned g = tile_grid(n_tiles, nb_cap);
    return n_cu >= kXcds ? std::min(g, unsigned(n_cu / kXcds * kXcds)) : g;
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
    if (!a.block_info) return hipErrorInvalidValue;
    TileArgs p{a.a1f, a.a1fs, a.w13p, a.w13sp, a.sorted_route, nullptr, a.num_valid,
               reinterpret_cast<const int4*>(a.block_info), a.M, a.topk, 2 * a.I, a.D, a.cap, a.a2q, a.a2s,
               a.h_dbg, nullptr, a.clk};
    MOE_LAUNCH(gemm1_tile_kernel, dim3(tile_persistent_grid(2 * a.I / kTN, a.nb_cap, a.n_cu)),
               dim3(kTThreads), uint32_t(tile_lds_bytes()), stream, ev, p, a.I);
    return hipGetLastError();
}

hipError_t launch_gemm2_tile(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev)
{
    if (a.nb_cap == 0) return hipSuccess;
    if (a.block_m != kTM || a.D % kTN != 0) return hipErrorInvalidValue;
    if (!a.block_info) return hipErrorInvalidValue;
    TileArgs p{a.a2q, a.a2s, a.w2p, a.w2sp, a.sorted_route, a.sorted_w, a.num_valid,
               reinterpret_cast<const int4*>(a.block_info), a.M, a.topk, a.D, a.I, a.cap, nullptr, nullptr,
               nullptr, a.partial, a.clk};
    MOE_LAUNCH(gemm2_tile_kernel, dim3(tile_persistent_grid(a.D / kTN, a.nb_cap, a.n_cu)),
               dim3(kTThreads), uint32_t(tile_lds_bytes()), stream, ev, p);
    return hipGetLastError();
}

}  // namespace moe
