// Route sort: expert-sorted, block_m-padded route lists (one workgroup).
//
// What it computes follows the sorting workspace of kernelindex submission
// 754773 (sorted ids / sorted weights / per-block expert ids / num_valid, with
// each expert's segment padded to a multiple of block_m) and the routing
// kernels of submission 723815 (histogram over experts, exclusive scan,
// scatter; expert ids outside [0, E) are ignored).  A route is r = t*topk + s.
//
// Design (gfx950, one 1024-thread workgroup):
//   pass 1  every wave walks its own contiguous range of routes, 64 at a time;
//           lanes holding the same expert are found with ballots over the bits
//           of the expert id, and the lowest such lane adds their count to the
//           wave's private LDS histogram row (no atomics, no contention);
//   scan    per expert: padded count, workgroup-wide exclusive scan -> expert
//           base; per (wave, expert) start = base + counts of earlier waves;
//   pass 2  the same walk again; each route lands at start + rank among equal
//           lanes, so every expert's list is in ascending route order and the
//           output is deterministic.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRouteUnroll = 8;

// Lanes of this wave whose (valid) expert id equals mine.
__device__ __forceinline__ uint64_t same_expert_lanes(int id, bool valid, int nbits)
{
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (id >> b) & 1;
        uint64_t set = __ballot(valid && bit);
        peers &= bit ? set : ~set;
    }
    return peers;
}

__global__ void __launch_bounds__(kRouteThreads)
route_sort_kernel(const int32_t* __restrict__ ids, const float* __restrict__ tw, int M,
                  int topk, int E, int bm, int nb_cap, int32_t* __restrict__ sorted_route,
                  float* __restrict__ sorted_w, int32_t* __restrict__ block_expert,
                  int32_t* __restrict__ num_valid)
{
    extern __shared__ int32_t lds[];
    int32_t* cnt = lds;                                   // [waves][E]
    int32_t* wave_sum = lds + kRouteWaves * E;            // [waves] scan scratch
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int R = M * topk;
    const int nbits = E > 1 ? 32 - __builtin_clz(unsigned(E - 1)) : 0;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) cnt[i] = 0;
    __syncthreads();

    const int per_wave = (R + kRouteWaves - 1) / kRouteWaves;
    const int w_begin = min(R, wave * per_wave), w_end = min(R, w_begin + per_wave);

    // pass 1: per-wave histogram
    for (int base = w_begin; base < w_end; base += kWave * kRouteUnroll) {
        int id[kRouteUnroll];
#pragma unroll
        for (int u = 0; u < kRouteUnroll; ++u) {
            int r = base + u * kWave + lane;
            id[u] = r < w_end ? ids[r] : -1;
        }
#pragma unroll
        for (int u = 0; u < kRouteUnroll; ++u) {
            bool valid = id[u] >= 0 && id[u] < E;
            uint64_t peers = same_expert_lanes(id[u], valid, nbits);
            if (valid && (peers & lanes_below) == 0) cnt[wave * E + id[u]] += __popcll(peers);
        }
    }
    __syncthreads();

    // scan over experts of the padded counts (one expert per thread per round)
    int carry = 0, valid_total = 0;
    for (int e0 = 0; e0 < E; e0 += kRouteThreads) {
        int e = e0 + tid;
        int total = 0;
        if (e < E)
            for (int w = 0; w < kRouteWaves; ++w) total += cnt[w * E + e];
        int padded = (total + bm - 1) / bm * bm;
        // inclusive scan of `padded` (and of `total`) across the workgroup
        int inc = padded, vinc = total;
        for (int off = 1; off < kWave; off <<= 1) {
            int a = __shfl_up(inc, off), b = __shfl_up(vinc, off);
            if (lane >= off) { inc += a; vinc += b; }
        }
        if (lane == kWave - 1) { wave_sum[wave] = inc; wave_sum[kRouteWaves + wave] = vinc; }
        __syncthreads();
        int before = 0, all = 0, vall = 0;
        for (int w = 0; w < kRouteWaves; ++w) {
            int s = wave_sum[w], vs = wave_sum[kRouteWaves + w];
            if (w < wave) before += s;
            all += s;
            vall += vs;
        }
        int base_e = carry + before + inc - padded;
        if (e < E) {
            int run = base_e;
            for (int w = 0; w < kRouteWaves; ++w) {
                int c = cnt[w * E + e];
                cnt[w * E + e] = run;
                run += c;
            }
            for (int p = base_e + total; p < base_e + padded; ++p) {
                sorted_route[p] = R;
                sorted_w[p] = 0.0f;
            }
            for (int b = base_e / bm; b < (base_e + padded) / bm; ++b) block_expert[b] = e;
        }
        carry += all;
        valid_total += vall;
        __syncthreads();
    }
    for (int b = carry / bm + tid; b < nb_cap; b += kRouteThreads) block_expert[b] = -1;
    if (tid == 0) {
        num_valid[0] = carry;
        num_valid[1] = valid_total;
    }
    __syncthreads();

    // pass 2: stable scatter
    for (int base = w_begin; base < w_end; base += kWave * kRouteUnroll) {
        int id[kRouteUnroll];
        float wt[kRouteUnroll];
#pragma unroll
        for (int u = 0; u < kRouteUnroll; ++u) {
            int r = base + u * kWave + lane;
            id[u] = r < w_end ? ids[r] : -1;
            wt[u] = r < w_end ? tw[r] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kRouteUnroll; ++u) {
            int r = base + u * kWave + lane;
            bool valid = id[u] >= 0 && id[u] < E;
            uint64_t peers = same_expert_lanes(id[u], valid, nbits);
            int start = valid ? cnt[wave * E + id[u]] : 0;
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                int pos = start + __popcll(peers & lanes_below);
                sorted_route[pos] = r;
                sorted_w[pos] = wt[u];
                if ((peers & lanes_below) == 0) cnt[wave * E + id[u]] = start + __popcll(peers);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

hipError_t route_allow_lds(int bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&route_sort_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

size_t route_lds_bytes(int E) { return sizeof(int32_t) * (size_t(kRouteWaves) * E + 2 * kRouteWaves); }

hipError_t launch_route_sort(const int32_t* ids, const float* tw, int M, int topk, int E, int bm,
                             int nb_cap, int32_t* sorted_route, float* sorted_w,
                             int32_t* block_expert, int32_t* num_valid, hipStream_t stream)
{
    hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(kRouteThreads), route_lds_bytes(E),
                       stream, ids, tw, M, topk, E, bm, nb_cap, sorted_route, sorted_w,
                       block_expert, num_valid);
    return hipGetLastError();
}

}  // namespace moe
