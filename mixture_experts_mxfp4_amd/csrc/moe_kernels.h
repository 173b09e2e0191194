// Host-side launchers of the gfx950 kernels (internal to libmoe_mxfp4.so).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Optional timestamps of one forward launch: events attached to the kernel's
// own dispatch (hipExtLaunchKernel), so they time the kernel and nothing else
// (an event record between two kernels adds microseconds of idle time).
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

#define MOE_LAUNCH(kernel, grid, block, shmem, stream, ev, ...)                                   \
    do {                                                                                        \
        if ((ev).start || (ev).stop)                                                            \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (ev).start, (ev).stop, 0, \
                                  __VA_ARGS__);                                                 \
        else                                                                                    \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                \
    } while (0)

size_t route_lds_bytes(int E);
hipError_t route_allow_lds(int bytes);   // lift the 64 KiB dynamic-LDS default
hipError_t launch_route_sort(const int32_t* ids, const float* tw, int M, int topk, int E, int bm,
                             int nb_cap, int32_t* sorted_route, float* sorted_w,
                             int32_t* block_expert, int32_t* num_valid, hipStream_t stream);

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                             uint8_t* scales, int n_cu, hipStream_t stream);

// Route sort + activation quantization in one launch: the first workgroup
// (short lists) or the first route_chunks workgroups (long lists) sort, the
// others quantize.
struct PrologueArgs {
    const int32_t* ids;
    const float* tw;
    int M, topk, E, bm, nb_cap;
    int32_t *sorted_route;
    float* sorted_w;
    int32_t *block_expert, *num_valid;
    const uint16_t* hidden;
    int D;
    uint8_t *a1q, *a1s;
    // [nb_cap][4], per used block: its expert, the expert's first block, its
    // number of blocks and its number of routes (tiled kernels; may be null)
    int32_t* block_info;
};
// Chunks (workgroups) of the route sort for this many routes (0: a short
// list, sorted by one wave).
int route_chunks(int M, int topk);
hipError_t launch_prologue(const PrologueArgs& a, int n_cu, hipStream_t stream,
                           const KernelEvents& ev = {});

hipError_t launch_prepare(const uint8_t* src_codes, const uint8_t* src_scales, uint8_t* dst_codes,
                          uint8_t* dst_scales, int E, int N, int K, int gate_up_I, int inverse,
                          int n_cu, hipStream_t stream);

// Gather the token-major activations a1 into sorted-row fragment layout
// (tiled path); padding rows are not written (no kernel uses them).
hipError_t launch_gather_a1(const uint8_t* a1q, const uint8_t* a1s, const int32_t* sorted_route,
                            const int32_t* num_valid, int M, int D, int topk, int64_t cap,
                            uint8_t* a1f, uint8_t* a1fs, int n_cu, hipStream_t stream,
                            const KernelEvents& ev = {});

// a2 (fragment layout) -> canonical row-major codes [cap][I/2] and scales [cap][I/32].
hipError_t launch_a2_to_canonical(const uint8_t* a2q, const uint8_t* a2s, int64_t cap, int I,
                                  uint8_t* codes, uint8_t* scales, hipStream_t stream);

struct Gemm1Args {
    const uint8_t *a1q, *a1s;      // token-major activations (streaming kernels)
    const uint8_t *a1f, *a1fs;     // sorted fragment-layout activations (tiled kernels)
    const uint8_t *w13p, *w13sp;
    const int32_t *sorted_route, *block_expert, *num_valid;
    uint8_t *a2q, *a2s;            // h in fragment layout, rows = cap
    uint16_t* h_dbg;
    int M, D, I, topk, block_m, nb_cap;
    int64_t cap;
    uint64_t* clk = nullptr;       // optional kernel span (span_begin / span_end)
    const int32_t* block_info = nullptr;   // [nb_cap][4] (paired blocks, tiled kernels)
    int n_cu = 0;                  // compute units: the tiled kernel's persistent grid
    bool pair_blocks = false;      // block_m 32: pairs of an expert's blocks as 64-row units
};
hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t stream, const KernelEvents& ev = {});
// 64-row gate_up groups per workgroup of the streaming stage 1 (grid: I/32 /
// groups x blocks).  Two groups halve the activation rows each weight byte
// pays for; at 16-row blocks the gather is small and the wider grid wins.
// I is a multiple of 256, so I/32 divides by 2.
constexpr int stream_stage1_groups(int block_m)
{
    return block_m == 64 || block_m == 32 ? 2 : 1;
}


struct Gemm2Args {
    const uint8_t *a2q, *a2s, *w2p, *w2sp;
    const int32_t* sorted_route;
    const float* sorted_w;
    const int32_t *block_expert, *num_valid;
    uint16_t* partial;          // bf16 [M*topk][D], weighted contribution per route
    int M, D, I, topk, block_m, nb_cap;
    int64_t cap;
    const int32_t* block_info = nullptr;   // [nb_cap][4] (paired blocks, tiled kernels)
    uint64_t* clk = nullptr;       // optional workgroup spans (tiled kernel)
    int n_cu = 0;                  // compute units: the tiled kernel's persistent grid
    bool pair_blocks = false;      // block_m 32: pairs of an expert's blocks as 64-row units
};
hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev = {});

// LDS-tiled variants for block_m = 256.  Their grids are one-dimensional:
// n_tiles column tiles x nb_cap blocks, rounded up to whole rounds of the 8 XCDs.
constexpr int kXcds = 8;
inline unsigned tile_grid(int n_tiles, int nb_cap)
{
    return unsigned((int64_t(n_tiles) * nb_cap + kXcds - 1) / kXcds * kXcds);
}
// Unit (x, block) of workgroup blockIdx.x in a grid of tile_grid(X,
// nb_cap) for the streaming GEMMs: the dispatcher deals workgroups to the
// XCDs round-robin, so workgroup w runs on XCD w % 8 as its (w / 8)-th; each
// XCD takes a contiguous equal share of the U = X * nb_used units ordered
// x-major, then block.  An expert's blocks at one x (one weight slice) then
// run side by side on one XCD and share that slice in its L2, instead of
// every XCD fetching it.  False past the used units.
__device__ __forceinline__ bool xcd_unit(int X, int nb_used, int& x, int& blk)
{
    const int w = blockIdx.x, k = w % kXcds, j = w / kXcds;
    const int64_t U = int64_t(X) * nb_used;
    const int64_t lo = U * k / kXcds, hi = U * (k + 1) / kXcds;
    if (lo + j >= hi) return false;
    const int64_t u = lo + j;
    x = int(u / nb_used);
    blk = int(u % nb_used);
    return true;
}
// Streaming kernels at block_m 32 with pair_blocks: the blocks 2j, 2j+1 of an
// expert with at most kPairMaxBlocks blocks form a 64-row unit (block_info
// record bi: expert, first block, block count, routes), which the two blocks'
// workgroups split by columns; a last odd block stays a 32-row unit.
constexpr int kPairMaxBlocks = 4;
__device__ __forceinline__ bool paired_block(int4 bi, int blk)
{
    return bi.z <= kPairMaxBlocks && ((blk - bi.y) ^ 1) < bi.z;
}
hipError_t tile_allow_lds();   // lift the dynamic-LDS limit of the tiled kernels
// Workgroups of a persistent tiled launch: one per CU (a multiple of the XCD
// count), fewer when there are fewer tiles; n_cu < 8: one per tile.
unsigned tile_persistent_grid(int n_tiles, int nb_cap, int n_cu);
hipError_t launch_gemm1_tile(const Gemm1Args& a, hipStream_t stream, const KernelEvents& ev = {});
hipError_t launch_gemm2_tile(const Gemm2Args& a, hipStream_t stream, const KernelEvents& ev = {});

// Route-indexed path (small batches): no route sort, no quantization or
// reduction pass; a2 rows and h rows are indexed by the route r = t*topk + s.
constexpr int kDirectMaxTokens = 32;
constexpr int kMaxTopkDirect = 16;
constexpr int kDirectMaxRoutes = 1024;
constexpr int kDirectMaxE = 1024;
// 64-row gate_up groups per stage-1 workgroup of the route-indexed path, and
// the stage-1 grid's x extent (2I/64 groups; I is a multiple of 256)
constexpr int kDirectGroups = 2;
__host__ __device__ inline int direct_stage1_x(int I) { return I / (32 * kDirectGroups); }
// expert slots: min(E, M*topk), an upper bound of the active experts
__host__ __device__ inline int direct_slots(int M, int E, int topk)
{
    return M * topk < E ? M * topk : E;
}
struct DirectArgs {
    const uint16_t* hidden;
    const uint8_t *w13p, *w13sp, *w2p, *w2sp;
    const int32_t* ids;
    const float* tw;
    uint8_t *a2q, *a2s;            // [M*topk][I/2], [M*topk][I/32]
    int32_t* slot_expert;          // [slots] expert of slot y (descending ids), or -1
    int32_t* slot_layers;          // [slots] layers of slot y's token -> route table
    int32_t* route_of;             // [topk][slots][M] route of token t to slot y's expert, or -1
    int32_t* n_active;             // [1] number of active experts
    uint16_t* out;                 // bf16 [M][D]
    uint16_t* h_dbg;
    int M, D, I, E, topk;
    uint64_t* clk = nullptr;       // optional stage-1 span (span_begin / span_end)
    // A16W4 mode when set: bf16 activations, no quantization; h is kept bf16
    // here, [M*topk][I] (a2q / a2s unused)
    uint16_t* h16 = nullptr;
    int h_lds = 0;                 // stage 2: bytes of h it stages in LDS (set by its launcher)
    // split-K stage 1 (ks_parts > 1): each unit's K in ks_parts parts on as
    // many workgroups, fp32 partial sums in `part` ([ks_parts][M*topk][2I]),
    // merged by the last part to finish, counted in split_ctr
    // ([slots][stage-1 x extent], zero before the first call, zero again after)
    int ks_parts = 1;
    float* part = nullptr;
    uint32_t* split_ctr = nullptr;
};
hipError_t direct_allow_lds();     // lift the dynamic-LDS limit of the stage-2 kernels
hipError_t launch_gemm1_direct(const DirectArgs& a, hipStream_t stream, const KernelEvents& ev = {});
hipError_t launch_gemm2_direct(const DirectArgs& a, hipStream_t stream, const KernelEvents& ev = {});
hipError_t launch_direct_rows(const int32_t* ids, int R, int E, int32_t* row_route,
                              int32_t* num_valid, hipStream_t stream);

// Single persistent launch of the route-indexed forward (decode_fused.hip):
// stage 1, a grid barrier on bar[0..1] (zero before the first call, zero
// again after each completed call; bar[2] becomes nonzero if a wait timed
// out), stage 2.  MXFP4 activations only (a.h16 must be null).
hipError_t fused_allow_lds();      // LDS limits and per-CU occupancy, once per device
int fused_grid(int M, int n_cu);   // workgroups of the launch (0 before fused_allow_lds)
hipError_t launch_zero_fill(uint8_t* p, size_t bytes, int n_cu, hipStream_t stream);
hipError_t launch_decode_fused(const DirectArgs& a, uint32_t* bar, int n_cu, uint64_t timeout_ticks,
                               hipStream_t stream, const KernelEvents& ev = {});

hipError_t launch_reduce_slots(const uint16_t* partial, const int32_t* ids, int M, int D, int E,
                               int topk, uint16_t* out, int n_cu, hipStream_t stream,
                               const KernelEvents& ev = {});

}  // namespace moe
