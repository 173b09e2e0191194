// Forward prologue: the route sort and the dynamic MXFP4 quantization of the
// hidden states, in ONE launch (the first workgroups sort the routes, the
// others quantize; neither depends on the other).
//
// Route sort.  What it computes follows the sorting workspace of kernelindex
// submission 754773 (sorted ids / sorted weights / per-block expert ids /
// num_valid, each expert's segment padded to a multiple of block_m) and the
// routing kernels of submission 723815 (histogram over experts, exclusive
// scan, scatter; expert ids outside [0, E) are ignored).  A route is
// r = t*topk + s.  Design (one 1024-thread workgroup):
//   pass 1  every wave walks its own contiguous range of routes, 64 at a time;
//           lanes holding the same expert are found with ballots over the bits
//           of the expert id, and the lowest such lane adds their count to the
//           wave's private LDS histogram row (no atomics, no contention);
//   scan    per expert: padded count, workgroup-wide exclusive scan -> expert
//           base; per (wave, expert) start = base + counts of earlier waves;
//   pass 2  the same walk again; each route lands at start + rank among equal
//           lanes, so every expert's list is in ascending route order and the
//           output is deterministic.
// Short route lists (M*topk <= 4096, decode) are sorted by a single wave
// instead (route_sort_wave): a kernel that one workgroup runs once is bound by
// barriers, instruction fetch and memory latency, not by arithmetic.  Long
// lists are split into chunks of kRouteChunk routes, one workgroup each, with
// a 4x unrolled walk that keeps more loads in flight; every chunk workgroup
// also counts the other chunks' routes (plain LDS atomics: counts need no
// order), so the whole sort is one launch with no workgroup waiting on
// another (9,216 routes: 16.4 us with the quantization, against 8.2 + 13.4 us
// for a counting launch followed by a scattering one; 36,864 routes: 20.4
// against 15.1 + 13.0 us).
//
// Activation quantization (OCP MX v1.0; the FP4 branch of 754773 quantizes
// the hidden states per 32 elements before the gate_up GEMM): four lanes own
// one 32-element block (8 bf16 = 16 bytes each); the block maximum is reduced
// across the four lanes, each lane writes 4 code bytes and the first lane the
// scale byte.
#include <algorithm>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kPrologueThreads = 1024;
constexpr int kRouteWaves = kPrologueThreads / kWave;
constexpr int kRouteChunk = 2 * kPrologueThreads;   // routes per workgroup of the chunked sort

// Lanes of this wave whose (valid) expert id equals mine.
__device__ __forceinline__ uint64_t same_expert_lanes(int id, bool valid, int nbits)
{
    uint64_t peers = __ballot(valid);
#pragma unroll 1
    for (int b = 0; b < nbits; ++b) {
        bool bit = (id >> b) & 1;
        uint64_t set = __ballot(valid && bit);
        peers &= bit ? set : ~set;
    }
    return peers;
}

// Every slot of the route list starts as padding (route M*topk, weight 0) and
// every block as unused (expert -1); the sort then only stores the real
// routes and the used blocks' experts (the padding is never written per
// expert, one slot at a time).  `part`/`parts` split the fill among the
// workgroups of a launch; the fill is ordered before the sort's own stores
// by a barrier (one workgroup) or by the launch boundary (chunked sort).
__device__ __forceinline__ void fill_padding(int R, int bm, int nb_cap,
                                             int32_t* __restrict__ sorted_route,
                                             float* __restrict__ sorted_w,
                                             int32_t* __restrict__ block_expert, int part = 0,
                                             int parts = 1)
{
    const int64_t cap = int64_t(nb_cap) * bm;
    const int64_t p0 = cap * part / parts, p1 = cap * (part + 1) / parts;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += kPrologueThreads) {
        sorted_route[p] = R;
        sorted_w[p] = 0.0f;
    }
    const int b0 = int(int64_t(nb_cap) * part / parts), b1 = int(int64_t(nb_cap) * (part + 1) / parts);
    for (int b = b0 + threadIdx.x; b < b1; b += kPrologueThreads) block_expert[b] = -1;
}

// Each wave of a workgroup takes a contiguous sub-range [w_begin, w_end) of
// the routes [c0, c1), kWave * U routes per batch; the first batch is loaded
// by the caller ahead of the work that can overlap its latency.
__device__ __forceinline__ void wave_range(int c0, int c1, int& w_begin, int& w_end)
{
    const int per_wave = (c1 - c0 + kRouteWaves - 1) / kRouteWaves;
    w_begin = min(c1, c0 + int(threadIdx.x / kWave) * per_wave);
    w_end = min(c1, w_begin + per_wave);
}

template <int U>
__device__ __forceinline__ void load_batch(const int32_t* __restrict__ ids, int base, int w_end,
                                           int (&id)[U])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = base + u * kWave + int(threadIdx.x % kWave);
        id[u] = r < w_end ? ids[r] : -1;
    }
}

// Per-wave histograms of the wave's routes: lanes holding the same expert are
// found with ballots over the bits of the id, and the lowest such lane adds
// their number to the wave's row cnt[wave * E + id] (no atomics).  id0 holds
// the first batch.
template <int U>
__device__ __forceinline__ void wave_histograms(const int32_t* __restrict__ ids, int w_begin,
                                                int w_end, const int (&id0)[U], int E, int nbits,
                                                int32_t* cnt)
{
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll 1
    for (int base = w_begin; base < w_end; base += kWave * U) {
        int id[U];
        if (base == w_begin) {
#pragma unroll
            for (int u = 0; u < U; ++u) id[u] = id0[u];
        } else {
            load_batch<U>(ids, base, w_end, id);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = id[u] >= 0 && id[u] < E;
            const uint64_t peers = same_expert_lanes(id[u], valid, nbits);
            if (valid && (peers & lanes_below) == 0) cnt[wave * E + id[u]] += __popcll(peers);
        }
    }
}

// Counts of the routes outside the chunk [c0, c1): out[e] those before it,
// out[E + e] those after it, with one LDS atomic per route (the counts are
// order-free; only the chunk's own ranks need the ballot walk).  Outside
// route i (i < R - (c1 - c0)) is route i before the chunk and i + (c1 - c0)
// after it; batch b holds routes b * kOutsideBatch + u * threads + tid.  When
// one batch holds them all, the caller loads it ahead of its own work (9,216
// routes: 20.1 -> 16.4 us with the quantization); with more batches that
// measured slower (36,864 routes: 20.9 -> 22.1 us).
constexpr int kOutsideU = 8;
constexpr int kOutsideBatch = kOutsideU * kPrologueThreads;

__device__ __forceinline__ void outside_load(const int32_t* __restrict__ ids, int R, int c0, int c1,
                                             int i0, int (&id)[kOutsideU])
{
    const int n_out = R - (c1 - c0);
#pragma unroll
    for (int u = 0; u < kOutsideU; ++u) {
        const int i = i0 + u * kPrologueThreads + int(threadIdx.x);
        id[u] = i < n_out ? ids[i < c0 ? i : i + (c1 - c0)] : -1;
    }
}

__device__ void outside_histogram(const int32_t* __restrict__ ids, int R, int c0, int c1, int E,
                                  bool preloaded, const int (&first)[kOutsideU], int32_t* out)
{
    const int n_out = R - (c1 - c0);
    int id[kOutsideU];
#pragma unroll
    for (int u = 0; u < kOutsideU; ++u) id[u] = first[u];
#pragma unroll 1
    for (int i0 = 0; i0 < n_out; i0 += kOutsideBatch) {
        if (i0 > 0 || !preloaded) outside_load(ids, R, c0, c1, i0, id);
#pragma unroll
        for (int u = 0; u < kOutsideU; ++u) {
            const int i = i0 + u * kPrologueThreads + int(threadIdx.x);
            if (id[u] >= 0 && id[u] < E) atomicAdd(&out[(i < c0 ? 0 : E) + id[u]], 1);
        }
    }
}

// Sorts the routes [c0, c1) (one chunk of the list, or all of it) into their
// final places.  With G > 1 chunks, the chunk's workgroup also counts every
// other chunk's routes (outside_histogram): the expert segments' bases come
// from the totals and this chunk's routes go after those of the chunks before
// it, so the G workgroups of one launch never wait for each other; each then
// writes the padding rows of experts g, g + G, ... and its part of the rows
// past the used blocks.  Chunk 0 (or the only one) writes block_expert,
// num_valid and, when given, block_info (per used block: expert, the expert's
// first block, its block count, its route count).  The order inside an
// expert's segment is ascending route: chunk, then wave, then lane order.
template <int U>
__device__ void route_sort_body(const int32_t* __restrict__ ids, const float* __restrict__ tw,
                                int M, int topk, int E, int bm, int nb_cap,
                                int32_t* __restrict__ sorted_route, float* __restrict__ sorted_w,
                                int32_t* __restrict__ block_expert,
                                int32_t* __restrict__ num_valid,
                                int32_t* __restrict__ block_info, int32_t* lds,
                                int c0 = 0, int c1 = -1, int G = 1, int g = 0)
{
    int32_t* cnt = lds;                                   // [waves][E]
    int32_t* wave_sum = lds + kRouteWaves * E;            // [2][waves] scan scratch
    // chunked sort: the routes before / after the chunk per expert, then each
    // expert's padding rows [start, end)
    int32_t* outside = wave_sum + 2 * kRouteWaves;        // [2][E]
    const bool chunked = G > 1;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int R = M * topk;
    if (c1 < 0) c1 = R;
    const int nbits = E > 1 ? 32 - __builtin_clz(unsigned(E - 1)) : 0;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // The wave's first batch of routes (the whole range of a chunk) and this
    // thread's per-chunk counts are loaded up front, so that both passes and
    // the scan wait on one round of memory latency.
    int w_begin, w_end;
    wave_range(c0, c1, w_begin, w_end);
    int id0[U];
    float wt0[U];
    load_batch<U>(ids, w_begin, w_end, id0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = w_begin + u * kWave + lane;
        wt0[u] = r < w_end ? tw[r] : 0.0f;
    }

    int oid[kOutsideU] = {};              // the other chunks' ids, when one batch
    const bool preload = chunked && R - (c1 - c0) <= kOutsideBatch;
    if (preload) outside_load(ids, R, c0, c1, 0, oid);
    for (int i = tid; i < kRouteWaves * E; i += kPrologueThreads) cnt[i] = 0;
    if (chunked)
        for (int i = tid; i < 2 * E; i += kPrologueThreads) outside[i] = 0;
    else
        fill_padding(R, bm, nb_cap, sorted_route, sorted_w, block_expert);
    __syncthreads();

    // pass 1: per-wave histogram of this chunk (and the counts of every other
    // chunk's routes)
    wave_histograms<U>(ids, w_begin, w_end, id0, E, nbits, cnt);
    if (chunked) outside_histogram(ids, R, c0, c1, E, preload, oid, outside);
    __syncthreads();

    // scan over experts of the padded totals (one expert per thread per round)
    int carry = 0, valid_total = 0;
#pragma unroll 1
    for (int e0 = 0; e0 < E; e0 += kPrologueThreads) {
        const int e = e0 + tid;
        int total = 0, earlier = 0;       // all routes of e; those of chunks before this one
        if (e < E) {
#pragma unroll 1
            for (int w = 0; w < kRouteWaves; ++w) total += cnt[w * E + e];
            if (chunked) {
                earlier = outside[e];
                total += outside[e] + outside[E + e];
            }
        }
        const int padded = (total + bm - 1) / bm * bm;
        int inc = padded, vinc = total;               // inclusive scans within the wave
#pragma unroll 1
        for (int off = 1; off < kWave; off <<= 1) {
            int a = __shfl_up(inc, off), b = __shfl_up(vinc, off);
            if (lane >= off) { inc += a; vinc += b; }
        }
        if (lane == kWave - 1) { wave_sum[wave] = inc; wave_sum[kRouteWaves + wave] = vinc; }
        __syncthreads();
        int before = 0, all = 0, vall = 0;
#pragma unroll 1
        for (int w = 0; w < kRouteWaves; ++w) {
            const int s = wave_sum[w];
            before += (w < wave) ? s : 0;
            all += s;
            vall += wave_sum[kRouteWaves + w];
        }
        const int base_e = carry + before + inc - padded;
        if (e < E) {
            int run = base_e + earlier;
#pragma unroll 1
            for (int w = 0; w < kRouteWaves; ++w) {
                int c = cnt[w * E + e];
                cnt[w * E + e] = run;
                run += c;
            }
            if (chunked) {             // this expert's padding rows, written below
                outside[e] = base_e + total;
                outside[E + e] = base_e + padded;
            }
            if (g == 0) {
#pragma unroll 1
                for (int b = base_e / bm; b < (base_e + padded) / bm; ++b) {
                    block_expert[b] = e;
                    if (block_info)
                        *reinterpret_cast<int4*>(block_info + 4 * b) =
                            make_int4(e, base_e / bm, padded / bm, total);
                }
            }
        }
        carry += all;
        valid_total += vall;
        __syncthreads();
    }
    if (tid == 0 && g == 0) {
        num_valid[0] = carry;
        num_valid[1] = valid_total;
    }
    if (chunked) {
        // padding: chunk g writes the padding rows of experts g, g + G, ...
        // (rows no chunk scatters to), part g of the rows past the used
        // blocks, and marks part g of the unused blocks
        // (at most bm - 1 rows each: with bm <= 64, one expert per wave at a
        // time across its lanes, else one at a time across the workgroup)
        if (bm <= kWave) {
#pragma unroll 1
            for (int e = g + G * wave; e < E; e += G * kRouteWaves)
                for (int p = outside[e] + lane; p < outside[E + e]; p += kWave) {
                    sorted_route[p] = R;
                    sorted_w[p] = 0.0f;
                }
        } else {
#pragma unroll 1
            for (int e = g; e < E; e += G)
                for (int p = outside[e] + tid; p < outside[E + e]; p += kPrologueThreads) {
                    sorted_route[p] = R;
                    sorted_w[p] = 0.0f;
                }
        }
        const int64_t cap = int64_t(nb_cap) * bm, tail = cap - carry;
        for (int64_t p = carry + tail * g / G + tid; p < carry + tail * (g + 1) / G;
             p += kPrologueThreads) {
            sorted_route[p] = R;
            sorted_w[p] = 0.0f;
        }
        const int nb_used = carry / bm, nb_tail = nb_cap - nb_used;
        for (int b = nb_used + int(int64_t(nb_tail) * g / G) + tid;
             b < nb_used + int(int64_t(nb_tail) * (g + 1) / G); b += kPrologueThreads)
            block_expert[b] = -1;
    }

    // pass 2: stable scatter (each wave only touches its own histogram row)
#pragma unroll 1
    for (int base = w_begin; base < w_end; base += kWave * U) {
        int id[U];
        float wt[U];
        if (base == w_begin) {
#pragma unroll
            for (int u = 0; u < U; ++u) { id[u] = id0[u]; wt[u] = wt0[u]; }
        } else {
            load_batch<U>(ids, base, w_end, id);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = base + u * kWave + lane;
                wt[u] = r < w_end ? tw[r] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * kWave + lane;
            const bool valid = id[u] >= 0 && id[u] < E;
            const uint64_t peers = same_expert_lanes(id[u], valid, nbits);
            const int start = valid ? cnt[wave * E + id[u]] : 0;
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                const int pos = start + __popcll(peers & lanes_below);
                sorted_route[pos] = r;
                sorted_w[pos] = wt[u];
                if ((peers & lanes_below) == 0) cnt[wave * E + id[u]] = start + __popcll(peers);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// The same route sort for short route lists: the workgroup stages topk_ids /
// topk_w in LDS with one coalesced load and counts them with LDS atomics, then
// ONE wave scans (DPP wave scans), writes each expert's blocks and padding
// rows, and scatters from LDS (no further barriers).  Nothing is filled
// beforehand: every row is written once, by the scatter or as padding.  The
// output order is identical to route_sort_body's (ascending route per expert).
// Its scatter walks the list 64 routes at a time in that one wave, so longer
// lists go to the workgroup sort (route_sort_body), whose waves scatter side
// by side.  Measured (sort plus the activation quantization, one launch):
// 576 routes at E=33 7.7 against 10.5 us; 900 routes at E=33 10.8 against
// 10.0; 1,152 routes at E=257 18.7 against 14.3; 2,700 routes at E=257 39.0
// against 17.1.
constexpr int kShortList = 768;

__device__ void route_sort_wave(const int32_t* __restrict__ ids_g, const float* __restrict__ tw_g,
                                int M, int topk, int E, int bm, int nb_cap,
                                int32_t* __restrict__ sorted_route, float* __restrict__ sorted_w,
                                int32_t* __restrict__ block_expert,
                                int32_t* __restrict__ num_valid,
                                int32_t* __restrict__ block_info, int32_t* lds)
{
    int32_t* ids = lds;                                          // [R]
    float* tw = reinterpret_cast<float*>(lds + kShortList);      // [R]
    int32_t* cnt = lds + 2 * kShortList;                         // [E]
    const int R = M * topk;
    for (int e = threadIdx.x; e < E; e += kPrologueThreads) cnt[e] = 0;
    __syncthreads();
    // pass 1: the whole workgroup stages the list in LDS and counts it (order-
    // free LDS atomics; only the scatter below needs the ordered walk)
    for (int r = threadIdx.x; r < R; r += kPrologueThreads) {
        const int id = ids_g[r];
        ids[r] = id;
        tw[r] = tw_g[r];
        if (id >= 0 && id < E) atomicAdd(&cnt[id], 1);
    }
    __syncthreads();
    if (threadIdx.x >= kWave) return;
    const int lane = threadIdx.x;
    const int nbits = E > 1 ? 32 - __builtin_clz(unsigned(E - 1)) : 0;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // scan of padded counts; cnt[e] becomes the expert's first row.  The
    // lane of expert e also writes its blocks' records and its padding rows
    // (no other store touches those rows, so nothing is filled beforehand).
    int carry = 0, vcarry = 0;
#pragma unroll 1
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        const int total = e < E ? cnt[e] : 0;
        const int padded = (total + bm - 1) / bm * bm;
        const int inc = wave_inclusive_scan(padded);
        const int vinc = wave_inclusive_scan(total);
        const int base_e = carry + inc - padded;
        if (e < E) {
            cnt[e] = base_e;
#pragma unroll 1
            for (int b = base_e / bm; b < (base_e + padded) / bm; ++b) {
                block_expert[b] = e;
                if (block_info)
                    *reinterpret_cast<int4*>(block_info + 4 * b) =
                        make_int4(e, base_e / bm, padded / bm, total);
            }
#pragma unroll 1
            for (int p = base_e + total; p < base_e + padded; ++p) {
                sorted_route[p] = R;
                sorted_w[p] = 0.0f;
            }
        }
        carry += __builtin_amdgcn_readlane(inc, kWave - 1);
        vcarry += __builtin_amdgcn_readlane(vinc, kWave - 1);
        __builtin_amdgcn_wave_barrier();
    }
    // rows past the used blocks are padding, blocks past them unused
    for (int64_t p = carry + lane; p < int64_t(nb_cap) * bm; p += kWave) {
        sorted_route[p] = R;
        sorted_w[p] = 0.0f;
    }
    for (int b = carry / bm + lane; b < nb_cap; b += kWave) block_expert[b] = -1;
    if (lane == 0) {
        num_valid[0] = carry;
        num_valid[1] = vcarry;
    }
    // pass 2: stable scatter
#pragma unroll 1
    for (int base = 0; base < R; base += kWave) {
        const int r = base + lane;
        const int id = r < R ? ids[r] : -1;
        const float wt = r < R ? tw[r] : 0.0f;
        const bool valid = id >= 0 && id < E;
        const uint64_t peers = same_expert_lanes(id, valid, nbits);
        const int start = valid ? cnt[id] : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            const int pos = start + __popcll(peers & lanes_below);
            sorted_route[pos] = r;
            sorted_w[pos] = wt;
            if ((peers & lanes_below) == 0) cnt[id] = start + __popcll(peers);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// MXFP4 quantization of rows of bf16 (grid-stride over 8-element chunks, four
// lanes per 32-element block): codes [rows][cols/2], scales [rows][cols/32].
__device__ void quant_rows_body(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                int64_t block, int64_t nblocks, int nthreads)
{
    const int64_t chunks_per_row = cols / 8;
    const int64_t n_chunks = rows * chunks_per_row;
    const int64_t stride = nblocks * nthreads;
    for (int64_t i0 = block * nthreads; i0 < n_chunks; i0 += stride) {
        const int64_t i = i0 + threadIdx.x;
        const bool in = i < n_chunks;          // whole 4-lane groups are in or out
        uint4 v = in ? *reinterpret_cast<const uint4*>(x + i * 8) : make_uint4(0, 0, 0, 0);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            amax = max(amax, w[j] & 0x7FFFu);
            amax = max(amax, (w[j] >> 16) & 0x7FFFu);
        }
        amax = max(amax, dpp<kDppXor1>(amax));      // the block's four lanes
        amax = max(amax, dpp<kDppXor2>(amax));
        const uint32_t s = mx_scale_from_amax(amax);
        const uint32_t packed = mx_pack8(w[0], w[1], w[2], w[3], s);
        if (in) {
            reinterpret_cast<uint32_t*>(codes)[i] = packed;
            if ((i & 3) == 0) {
                scales[i / 4] = uint8_t(s);        // block index = chunk index / 4
            }
        }
    }
}

// U = 0: single-wave sort (short lists); otherwise the workgroup sort.
template <int U>
__global__ void __launch_bounds__(kPrologueThreads)
route_sort_kernel(const int32_t* __restrict__ ids, const float* __restrict__ tw, int M,
                  int topk, int E, int bm, int nb_cap, int32_t* __restrict__ sorted_route,
                  float* __restrict__ sorted_w, int32_t* __restrict__ block_expert,
                  int32_t* __restrict__ num_valid)
{
    extern __shared__ int32_t lds[];
    if constexpr (U == 0) {
        route_sort_wave(ids, tw, M, topk, E, bm, nb_cap, sorted_route, sorted_w, block_expert,
                        num_valid, nullptr, lds);
    } else {
        route_sort_body<U>(ids, tw, M, topk, E, bm, nb_cap, sorted_route, sorted_w,
                           block_expert, num_valid, nullptr, lds);
    }
}

__global__ void __launch_bounds__(kPrologueThreads)
quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    quant_rows_body(x, rows, cols, codes, scales, blockIdx.x, gridDim.x, kPrologueThreads);
}

// Short route lists (at most kShortList routes): workgroup 0 sorts with one
// wave, the others quantize the activations.
__global__ void __launch_bounds__(kPrologueThreads)
prologue_kernel(PrologueArgs a)
{
    extern __shared__ int32_t lds[];
    if (blockIdx.x == 0) {
        route_sort_wave(a.ids, a.tw, a.M, a.topk, a.E, a.bm, a.nb_cap, a.sorted_route, a.sorted_w,
                        a.block_expert, a.num_valid, a.block_info, lds);
    } else {
        quant_rows_body(a.hidden, a.M, a.D, a.a1q, a.a1s, blockIdx.x - 1, gridDim.x - 1,
                        kPrologueThreads);
    }
}

// Long route lists in ONE launch: workgroup g < G sorts chunk g of
// kRouteChunk routes; it counts every other chunk's routes itself (each
// chunk workgroup reads the whole id list, a few hundred KiB at most), so no
// workgroup waits for another.  The others quantize the activations.
__global__ void __launch_bounds__(kPrologueThreads)
prologue_sort_kernel(PrologueArgs a, int G)
{
    extern __shared__ int32_t lds[];
    const int g = blockIdx.x;
    if (g < G) {
        const int R = a.M * a.topk;
        route_sort_body<4>(a.ids, a.tw, a.M, a.topk, a.E, a.bm, a.nb_cap, a.sorted_route,
                           a.sorted_w, a.block_expert, a.num_valid, a.block_info, lds,
                           g * kRouteChunk, min(R, (g + 1) * kRouteChunk), G, g);
    } else {
        quant_rows_body(a.hidden, a.M, a.D, a.a1q, a.a1s, blockIdx.x - G, gridDim.x - G,
                        kPrologueThreads);
    }
}

// Sorted-row fragment copy of the quantized activations for the tiled
// kernels.  A workgroup copies one 16-row slice at a time: the slice's codes
// are one contiguous run of KT KiB in the fragment layout ([K tile][32-element
// chunk][row][16 B]), so thread i of the slice writes 16-byte piece i of that
// run (a wave stores 1 KiB contiguous per instruction) and reads it from its
// row, 16 rows x 64 contiguous bytes per wave instruction; the scale words go
// the same way (64 contiguous bytes per K tile).  Only rows holding a route
// are written: padding rows (and rows past num_valid[0]) are left as they are.
// Stage 1 never reads the rows of an all-padding 64-row group, and a padding
// row it does read only decides that row of the product (an MFMA output row
// depends on its own A row and scale alone), whose h and stage-2 result are
// never stored to a route.
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 8;       // 16-byte pieces in flight per thread

__global__ void __launch_bounds__(kGatherThreads)
gather_a1_kernel(const uint8_t* __restrict__ a1q, const uint8_t* __restrict__ a1s,
                 const int32_t* __restrict__ sorted_route, const int32_t* __restrict__ num_valid,
                 int M, int D, int topk, int64_t cap, uint8_t* __restrict__ a1f,
                 uint8_t* __restrict__ a1fs)
{
    const int KT = D / 128;
    const int64_t slices = num_valid[0] / 16;
    const int R = M * topk;
    const int r = threadIdx.x % 16;            // this thread's row of every slice
    const int pieces = KT * 64;                // 16-byte code pieces per slice
#pragma unroll 1
    for (int64_t sl = blockIdx.x; sl < slices; sl += gridDim.x) {
        const int64_t row = sl * 16 + r;
        const int sr = sorted_route[row];
        if (sr >= R) continue;                 // a padding row: nothing to copy
        const uint8_t* src = a1q + int64_t(sr / topk) * (D / 2);
        uint8_t* dst = a1f + frag_code_off(sl * 16, 0, 0, KT);
        // piece i = (kt, chunk c, row r): i = (kt * 4 + c) * 16 + r
#pragma unroll 1
        for (int i0 = threadIdx.x; i0 < pieces; i0 += kGatherThreads * kGatherUnroll) {
            uint4 v[kGatherUnroll];
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) {
                const int i = i0 + u * kGatherThreads;
                if (i < pieces) v[u] = ld16(src + (i >> 4) * 16);   // (kt * 4 + c) * 16 bytes
            }
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) {
                const int i = i0 + u * kGatherThreads;
                if (i < pieces) *reinterpret_cast<uint4*>(dst + int64_t(i) * 16) = v[u];
            }
        }
        // scale words: (kt, r) for kt = threadIdx.x / 16, + 16, ...
        const uint8_t* ssrc = a1s + int64_t(sr / topk) * (D / 32);
#pragma unroll 1
        for (int kt = threadIdx.x / 16; kt < KT; kt += kGatherThreads / 16)
            *reinterpret_cast<uint32_t*>(a1fs + frag_scale_off(row, kt, cap)) =
                *reinterpret_cast<const uint32_t*>(ssrc + kt * 4);
    }
}

hipError_t launch_gather_a1(const uint8_t* a1q, const uint8_t* a1s, const int32_t* sorted_route,
                            const int32_t* num_valid, int M, int D, int topk, int64_t cap,
                            uint8_t* a1f, uint8_t* a1fs, int n_cu, hipStream_t stream,
                            const KernelEvents& ev)
{
    const int64_t slices = cap / 16;
    if (slices == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>(slices, int64_t(n_cu) * 8);
    MOE_LAUNCH(gather_a1_kernel, dim3(unsigned(blocks)), dim3(kGatherThreads), 0, stream, ev, a1q,
               a1s, sorted_route, num_valid, M, D, topk, cap, a1f, a1fs);
    return hipGetLastError();
}

size_t route_lds_bytes(int E)
{
    const size_t wg = size_t(kRouteWaves) * E + 2 * kRouteWaves + 2 * size_t(E);   // workgroup sort
    const size_t wave = 2 * size_t(kShortList) + E;                  // single-wave sort
    return sizeof(int32_t) * (wg > wave ? wg : wave);
}

static bool long_list(int M, int topk) { return int64_t(M) * topk > kShortList; }

int route_chunks(int M, int topk)
{
    return long_list(M, topk) ? int((int64_t(M) * topk + kRouteChunk - 1) / kRouteChunk) : 0;
}

hipError_t route_allow_lds(int bytes)
{
    const void* k[] = {reinterpret_cast<const void*>(&route_sort_kernel<0>),
                       reinterpret_cast<const void*>(&route_sort_kernel<4>),
                       reinterpret_cast<const void*>(&prologue_kernel),
                       reinterpret_cast<const void*>(&prologue_sort_kernel)};
    for (const void* f : k) {
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_route_sort(const int32_t* ids, const float* tw, int M, int topk, int E, int bm,
                             int nb_cap, int32_t* sorted_route, float* sorted_w,
                             int32_t* block_expert, int32_t* num_valid, hipStream_t stream)
{
    if (long_list(M, topk))
        hipLaunchKernelGGL(route_sort_kernel<4>, dim3(1), dim3(kPrologueThreads),
                           route_lds_bytes(E), stream, ids, tw, M, topk, E, bm, nb_cap,
                           sorted_route, sorted_w, block_expert, num_valid);
    else
        hipLaunchKernelGGL(route_sort_kernel<0>, dim3(1), dim3(kPrologueThreads),
                           route_lds_bytes(E), stream, ids, tw, M, topk, E, bm, nb_cap,
                           sorted_route, sorted_w, block_expert, num_valid);
    return hipGetLastError();
}

static int64_t quant_blocks(int64_t rows, int64_t cols, int n_cu)
{
    const int64_t n_chunks = rows * (cols / 8);
    int64_t blocks = (n_chunks + kPrologueThreads - 1) / kPrologueThreads;
    return blocks > int64_t(n_cu) * 4 ? int64_t(n_cu) * 4 : blocks;
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                             uint8_t* scales, int n_cu, hipStream_t stream)
{
    const int64_t blocks = quant_blocks(rows, cols, n_cu);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_rows_kernel, dim3(unsigned(blocks)), dim3(kPrologueThreads), 0,
                       stream, x, rows, cols, codes, scales);
    return hipGetLastError();
}

hipError_t launch_prologue(const PrologueArgs& a, int n_cu, hipStream_t stream,
                           const KernelEvents& ev)
{
    const uint32_t lds_bytes = uint32_t(route_lds_bytes(a.E));
    const int G = route_chunks(a.M, a.topk);
    if (G > 0) {
        const int64_t blocks = G + quant_blocks(a.M, a.D, n_cu);
        MOE_LAUNCH(prologue_sort_kernel, dim3(unsigned(blocks)), dim3(kPrologueThreads), lds_bytes,
                   stream, ev, a, G);
        return hipGetLastError();
    }
    // a short list: one launch (the chunked sort above takes every long list;
    // a single workgroup sorting 9,216 routes measured 28 us against 20 us for
    // the two chunked launches, 36,864 routes 86 against 30 us)
    const int64_t blocks = 1 + quant_blocks(a.M, a.D, n_cu);
    MOE_LAUNCH(prologue_kernel, dim3(unsigned(blocks)), dim3(kPrologueThreads), lds_bytes, stream, ev,
               a);
    return hipGetLastError();
}

}  // namespace moe
