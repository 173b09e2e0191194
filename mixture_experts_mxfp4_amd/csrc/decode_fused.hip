// Single persistent launch of the route-indexed (decode) forward.
//
// The two-launch forward (direct.hip) ends stage 1, drains the GPU and starts
// stage 2 from an idle chip: the CUs that finish their stage-1 share early
// (one unit against two elsewhere) wait with the memory system half used,
// and stage 2 then ramps up its weight stream from nothing.  This kernel runs
// both stages in ONE launch of persistent workgroups (the prior-art design of
// the CuTeDSL W4A16 fused MoE kernel: FC1, a grid barrier, FC2 with the top-k
// sum folded into its epilogue):
//
//   phase 1  each workgroup of four waves runs stage-1 units (stage1_unit,
//            direct_common.h: route scan, in-register activation quant,
//            gate_up GEMM, SwiGLU, requant of h by route) in a fixed
//            round-robin order;
//   phase 2  each workgroup builds its stage-2 tables itself (active experts
//            in descending id order, the token -> route table, the routing
//            weights: nothing here depends on stage 1), then issues the
//            weight loads of its first stage-2 step, and only then waits at
//            the grid barrier: its first weights stream in while the slower
//            CUs finish stage 1;
//   barrier  an arrival counter and a generation word in the caller's
//            workspace (zero before the first call, zero again after every
//            completed call); every wait is bounded by a wall-clock limit;
//   stage 2  each workgroup's four waves compute a 16-column output slice
//            for all tokens (as gemm2_direct_kernel does for 32 columns with
//            sixteen waves: each wave takes every fourth active expert, three
//            of them per step (two with 17-32 tokens), with the next step's
//            weights loaded before the current step's MFMAs) and write it once, as bf16, with the
//            per-token sum over experts in fp32.  The workgroups without a
//            stage-1 unit take the first slices.
//
// Stage 1 takes ~250 VGPRs per lane, so a CU holds two of these workgroups;
// the grid is exactly what the CUs hold at once (the occupancy the runtime
// reports for this kernel, times the CUs), which the barrier needs: every
// workgroup is resident at once when the GPU runs nothing else.
// If a workgroup waits longer than the limit (another kernel holding CUs),
// it gives up: it fills the output slices it owns with NaN, sets the error
// word, and exits; the barrier state must then be reset (init) before the
// next call.
#include <atomic>

#include "direct_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedNS = 1;                 // 16-column slices per stage-2 unit
constexpr int kFusedMaxSlots = kDirectMaxTokens * kMaxTopkDirect;
// 64-row gate_up groups per stage-1 unit, as in the two-launch kernel (one
// group per unit halves the weight bytes each wave keeps in flight).
constexpr int kFusedGroups = kDirectGroups;
// Arrival groups of the grid barrier: workgroup w arrives on counter w % 8,
// the last arrival of each group on the grid counter.
constexpr int kBarrierGroups = 8;

template <int RT>
struct FusedStage2Lds {
    int32_t s_e[kFusedMaxSlots];                 // slot -> expert (descending ids)
    int16_t e2y[kDirectMaxE];                    // expert -> slot
    int32_t s_route[kFusedMaxSlots * 16 * RT];   // [slot][token]: first route, or a large value
    float s_tw[kFusedMaxSlots];                  // topk_w by route
    uint32_t bitmap[kDirectMaxE / 32];
    int32_t active;
    int32_t ok;
    float red[kFusedWaves][kFusedNS][RT][4][kWave];
};

template <int RT>
union FusedLds {
    Stage1Lds<kFusedGroups> p1;
    FusedStage2Lds<RT> p2;
};

// Stage-2 tables of this workgroup, from the routing alone: slot y of the
// active experts in descending id order (as stage 1 numbers them), token t's
// first route to slot y's expert, the routing weights.  Run by all threads.
template <int RT>
__device__ __forceinline__ void fused_tables(const DirectArgs& a, FusedStage2Lds<RT>& L)
{
    const int R = a.M * a.topk;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int words = (a.E + 31) / 32;
    for (int i = threadIdx.x; i < words; i += kFusedThreads) L.bitmap[i] = 0u;
    for (int i = threadIdx.x; i < kFusedMaxSlots * 16 * RT; i += kFusedThreads) L.s_route[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int r = threadIdx.x; r < R; r += kFusedThreads) {
        const int e = a.ids[r];
        if (e >= 0 && e < a.E) atomicOr(&L.bitmap[e / 32], 1u << (e % 32));
        L.s_tw[r] = a.tw[r];
    }
    __syncthreads();
    if (wave == 0) {
        // word w on lane words-1-w: the highest ids first
        const int wi = words - 1 - lane;
        uint32_t w = lane < words ? L.bitmap[wi] : 0u;
        const int pc = __popc(w);
        const int inc = wave_inclusive_scan(pc);
        int y = inc - pc;
        while (w) {
            const int b = 31 - __builtin_clz(w);
            const int e = wi * 32 + b;
            L.s_e[y] = e;
            L.e2y[e] = int16_t(y);
            ++y;
            w &= ~(1u << b);
        }
        if (lane == kWave - 1) L.active = inc;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < R; r += kFusedThreads) {
        const int e = a.ids[r];
        if (e >= 0 && e < a.E) {
            const int y = L.e2y[e];
            atomicMin(&L.s_route[y * 16 * RT + r / a.topk], r);
        }
    }
    __syncthreads();
}

// Grid barrier of the persistent workgroups.  bar[0] is the generation
// (read by every workgroup at its start as `gen`), bar[1] the sticky error
// word, bar[4 + 32 * j] (one 128-byte line each) the arrival count of group j
// (workgroups w with w % 8 == j) and bar[4 + 32 * 8] that of the groups.
// The last arrival of a group resets its count and arrives on the grid
// count; the last of those resets it and advances the generation.  The
// others wait for the generation to move, polling with relaxed loads (an
// acquiring load would invalidate the caches at every poll) for at most
// `timeout_ticks` of the constant-rate clock.  One thread per workgroup makes
// the workgroup's stores visible device-wide before arriving (agent-scope
// release) and, once the generation moved, invalidates the workgroup's
// caches (agent-scope acquire).  Returns false on a timeout.
__device__ __forceinline__ uint32_t* barrier_count(uint32_t* bar, int j) { return bar + 4 + 32 * j; }

__device__ __forceinline__ bool grid_barrier(uint32_t* bar, uint32_t gen, uint32_t nwg,
                                             uint64_t timeout_ticks, int32_t* ok_lds)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t j = blockIdx.x % kBarrierGroups;
        const uint32_t in_group = (nwg - j + kBarrierGroups - 1) / kBarrierGroups;
        const uint32_t groups = nwg < kBarrierGroups ? nwg : kBarrierGroups;
        bool last = false;
        if (__hip_atomic_fetch_add(barrier_count(bar, j), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == in_group - 1) {
            __hip_atomic_store(barrier_count(bar, j), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = __hip_atomic_fetch_add(barrier_count(bar, kBarrierGroups), 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == groups - 1;
        }
        int ok = 1;
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(barrier_count(bar, kBarrierGroups), 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&bar[0], gen + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const uint64_t t0 = wall_clock64();
            while (__hip_atomic_load(&bar[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                if (wall_clock64() - t0 > timeout_ticks) {
                    ok = 0;
                    __hip_atomic_store(&bar[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        *ok_lds = ok;
    }
    __syncthreads();
    return *ok_lds != 0;
}

// Weight fragments of one stage-2 step of a wave: G slots x 2 K tiles x NS
// slices (16 bytes each) and the slots' scale words.
template <int G>
struct W2Step {
    uint4 b[G][2][kFusedNS];
    uint32_t sw[G][2];
};

template <int G>
__device__ __forceinline__ void load_w2_step(const DirectArgs& a, const int32_t* s_e, int active,
                                             int y0, int kt, const uint8_t* wcol,
                                             const uint8_t* scol, W2Step<G>& w)
{
    const int64_t w_stride = int64_t(a.D) * (a.I / 2), s_stride = int64_t(a.D) * (a.I / 32);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int y = y0 + g * kFusedWaves;
        const bool on = y < active;
        const int64_t e = on ? s_e[y] : 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int sl = 0; sl < kFusedNS; ++sl)
                w.b[g][h][sl] = on ? ld16_nt(wcol + e * w_stride + int64_t(kt + h) * 4096 + sl * 1024)
                                   : make_uint4(0, 0, 0, 0);
            w.sw[g][h] = on ? *reinterpret_cast<const uint32_t*>(scol + e * s_stride + (kt + h) * 256) : 0u;
        }
    }
}

template <int RT, int G>
__global__ void __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(2)))
decode_fused_kernel(DirectArgs a, uint32_t* bar, uint64_t timeout_ticks)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    FusedLds<RT>& L = *reinterpret_cast<FusedLds<RT>*>(lds_raw);
    span_begin(a.clk);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int nwg = gridDim.x;
    __shared__ uint32_t gen_lds;
    if (threadIdx.x == 0) gen_lds = __hip_atomic_load(&bar[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t gen = gen_lds;

    // ---- phase 1: stage-1 units u = blockIdx.x + k * nwg (expert slot u / X,
    // group pair u % X), while u names an active slot.  The first unit is
    // straight-line code: inside the loop the unit needs more registers than
    // the 256 a lane has here and spills, and at decode (fewer units than
    // workgroups) the loop never runs.
    {
        const int X = a.I / (32 * kFusedGroups);
        const int slots = direct_slots(a.M, a.E, a.topk);
        int limit = slots * X;
        if (int(blockIdx.x) < limit)
            limit = X * stage1_unit<kG1Unroll, kFusedGroups, false>(
                            a, blockIdx.x % X, blockIdx.x / X, wave, L.p1, [] { __syncthreads(); });
#pragma unroll 1
        for (int u = blockIdx.x + nwg; u < limit; u += nwg)
            stage1_unit<kG1Unroll, kFusedGroups, false>(a, u % X, u / X, wave, L.p1,
                                                        [] { __syncthreads(); });
    }
    __syncthreads();

    // ---- phase 2: local tables, first weights, grid barrier, stage 2
    FusedStage2Lds<RT>& S = L.p2;
    fused_tables<RT>(a, S);
    const int active = S.active;
    const int M = a.M, D = a.D, I = a.I;
    const int KT = I / 128;                     // even
    const int n_slices = D / (16 * kFusedNS);
    const int row = lane % 16, kq = lane / 16;
    int s = nwg - 1 - int(blockIdx.x);          // workgroups with less stage-1 work first

    auto slice_cols = [&](int sl_unit, const uint8_t*& wcol, const uint8_t*& scol) {
        const int n16_0 = sl_unit * kFusedNS, n64 = n16_0 / 4, q0 = n16_0 % 4;
        wcol = a.w2p + (int64_t(n64) * KT * 4 + q0) * 1024 + lane * 16;
        scol = a.w2sp + int64_t(n64) * KT * 256 + lane * 4;
    };
    W2Step<G> cur;
    const uint8_t *wcol = nullptr, *scol = nullptr;
    if (s < n_slices) {
        slice_cols(s, wcol, scol);
        load_w2_step<G>(a, S.s_e, active, wave, 0, wcol, scol, cur);
    }
    const bool ok = grid_barrier(bar, gen, uint32_t(nwg), timeout_ticks, &S.ok);

    for (; s < n_slices; s += nwg) {
        const int n16_0 = s * kFusedNS, q0 = n16_0 % 4;
        if (!ok) {                                // timed out: this slice is NaN
            for (int o = threadIdx.x; o < M * 16 * kFusedNS; o += kFusedThreads)
                a.out[int64_t(o / (16 * kFusedNS)) * D + n16_0 * 16 + o % (16 * kFusedNS)] = 0x7FC0;
            continue;
        }
        if (wcol == nullptr) {
            slice_cols(s, wcol, scol);
            load_w2_step<G>(a, S.s_e, active, wave, 0, wcol, scol, cur);
        }
        v4f acc[kFusedNS][RT];
#pragma unroll
        for (int sl = 0; sl < kFusedNS; ++sl)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[sl][rt] = v4f{0.f, 0.f, 0.f, 0.f};
        // steps: (y0, kt) for y0 = wave, wave + 8G, ... and kt = 0, 2, ..
#pragma unroll 1
        for (int y0 = wave; y0 < active; y0 += kFusedWaves * G) {
            v4f tmp[G][kFusedNS][RT];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int sl = 0; sl < kFusedNS; ++sl)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) tmp[g][sl][rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int kt = 0; kt < KT; kt += 2) {
                HFrag<false> av[G][2][RT];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int y = y0 + g * kFusedWaves;
                    const bool on = y < active;
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const int t = rt * 16 + row;
                        const int r0 = (on && t < M) ? S.s_route[y * 16 * RT + t] : 0x7FFFFFFF;
                        const int r = r0 == 0x7FFFFFFF ? -1 : r0;
#pragma unroll
                        for (int h = 0; h < 2; ++h) av[g][h][rt] = load_hfrag<false>(a, r, kt + h, kq, nullptr);
                    }
                }
                // the next step's weights (same slots at kt + 2, or the next slots)
                W2Step<G> nxt;
                const bool more_kt = kt + 2 < KT;
                const int ny0 = more_kt ? y0 : y0 + kFusedWaves * G;
                const bool have_next = more_kt || ny0 < active;
                if (have_next) load_w2_step<G>(a, S.s_e, active, ny0, more_kt ? kt + 2 : 0, wcol, scol, nxt);
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int sl = 0; sl < kFusedNS; ++sl)
                            mfma_hfrag<false, RT>(av[g][h], cur.b[g][h][sl],
                                                  (cur.sw[g][h] >> (8 * (q0 + sl))) & 0xFFu, tmp[g][sl]);
                if (have_next) cur = nxt;
            }
            // weight each token's row by its routing weight and accumulate
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int y = y0 + g * kFusedWaves;
                if (y >= active) break;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = rt * 16 + 4 * kq + i;
                        const int r = t < M ? S.s_route[y * 16 * RT + t] : 0x7FFFFFFF;
                        const float w = r != 0x7FFFFFFF ? S.s_tw[r] : 0.0f;
#pragma unroll
                        for (int sl = 0; sl < kFusedNS; ++sl) acc[sl][rt][i] += w * tmp[g][sl][rt][i];
                    }
            }
        }

        // further layers (a token naming one expert in several slots): rare,
        // one slot and K tile at a time, routes from the tables stage 1 published
        const int slots = direct_slots(M, a.E, a.topk);
#pragma unroll 1
        for (int y = wave; y < active; y += kFusedWaves) {
            const int layers = a.slot_layers[y];
            const int64_t e = S.s_e[y];
#pragma unroll 1
            for (int l = 1; l < layers; ++l) {
                const int32_t* tab = a.route_of + (int64_t(l) * slots + y) * M;
                v4f tmp[kFusedNS][RT];
#pragma unroll
                for (int sl = 0; sl < kFusedNS; ++sl)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) tmp[sl][rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
                for (int kt = 0; kt < KT; ++kt) {
                    const uint32_t sw = *reinterpret_cast<const uint32_t*>(
                        scol + e * int64_t(D) * (I / 32) + kt * 256);
                    HFrag<false> av[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const int t = rt * 16 + row;
                        av[rt] = load_hfrag<false>(a, t < M ? tab[t] : -1, kt, kq, nullptr);
                    }
#pragma unroll
                    for (int sl = 0; sl < kFusedNS; ++sl) {
                        const uint4 b = ld16(wcol + e * int64_t(D) * (I / 2) + int64_t(kt) * 4096 + sl * 1024);
                        mfma_hfrag<false, RT>(av, b, (sw >> (8 * (q0 + sl))) & 0xFFu, tmp[sl]);
                    }
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = rt * 16 + 4 * kq + i;
                        const int r = t < M ? tab[t] : -1;
                        const float w = r >= 0 ? S.s_tw[r] : 0.0f;
#pragma unroll
                        for (int sl = 0; sl < kFusedNS; ++sl) acc[sl][rt][i] += w * tmp[sl][rt][i];
                    }
            }
        }

        // the waves' sums, in wave order; one bf16 rounding
#pragma unroll
        for (int sl = 0; sl < kFusedNS; ++sl)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) S.red[wave][sl][rt][i][lane] = acc[sl][rt][i];
        __syncthreads();
        for (int o = threadIdx.x; o < M * 16 * kFusedNS; o += kFusedThreads) {
            const int t = o / (16 * kFusedNS), c = o % (16 * kFusedNS);
            const int sl = c / 16, col = c % 16;
            const int rt = t / 16, tt = t % 16;
            const int Ln = col + 16 * (tt / 4), i = tt % 4;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < kFusedWaves; ++w) sum += S.red[w][sl][rt][i][Ln];
            a.out[int64_t(t) * D + n16_0 * 16 + c] = uint16_t(f32_to_bf16_rne(sum));
        }
        __syncthreads();                          // red is rewritten by the next slice
        wcol = nullptr;
    }
    span_end(a.clk);
}

// Zero fill of a buffer (a multiple of 16 bytes, 16-byte aligned): plain
// vector stores, so that it may be captured in a graph.
__global__ void zero_fill_kernel(uint4* p, int64_t n16)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

static size_t fused_lds_bytes(int M)
{
    return M <= 16 ? sizeof(FusedLds<1>) : sizeof(FusedLds<2>);
}

// Workgroups of each instance that one CU holds at once, found once per
// process (every device the library runs on is a gfx950 with the same limits).
static std::atomic<int> g_fused_per_cu[2];

hipError_t fused_allow_lds()
{
    const void* k[2] = {reinterpret_cast<const void*>(&decode_fused_kernel<1, 3>),
                        reinterpret_cast<const void*>(&decode_fused_kernel<2, 2>)};
    const size_t bytes[2] = {sizeof(FusedLds<1>), sizeof(FusedLds<2>)};
    for (int i = 0; i < 2; ++i) {
        hipError_t e = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                           int(bytes[i]));
        if (e != hipSuccess) return e;
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k[i], kFusedThreads, bytes[i]);
        if (e != hipSuccess) return e;
        g_fused_per_cu[i].store(per_cu, std::memory_order_relaxed);
    }
    return hipSuccess;
}

int fused_grid(int M, int n_cu)
{
    return g_fused_per_cu[M <= 16 ? 0 : 1].load(std::memory_order_relaxed) * n_cu;
}

hipError_t launch_zero_fill(uint8_t* p, size_t bytes, int n_cu, hipStream_t stream)
{
    const int64_t n16 = int64_t(bytes / 16);
    if (n16 == 0) return hipSuccess;
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > int64_t(n_cu) * 8) blocks = int64_t(n_cu) * 8;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(p), n16);
    return hipGetLastError();
}

hipError_t launch_decode_fused(const DirectArgs& a, uint32_t* bar, int n_cu, uint64_t timeout_ticks,
                               hipStream_t stream, const KernelEvents& ev)
{
    if (a.M == 0) return hipSuccess;
    if (a.M > kDirectMaxTokens || a.topk > kMaxTopkDirect ||
        int64_t(a.M) * a.topk > kDirectMaxRoutes || a.E > kDirectMaxE || a.h16)
        return hipErrorInvalidValue;
    const uint32_t lds = uint32_t(fused_lds_bytes(a.M));
    const int inst = a.M <= 16 ? 0 : 1;
    const int nwg = fused_grid(a.M, n_cu);
    if (nwg < 1) return hipErrorInvalidConfiguration;
    const dim3 grid{unsigned(nwg)};
    if (inst == 0)
        MOE_LAUNCH((decode_fused_kernel<1, 3>), grid, dim3(kFusedThreads), lds, stream, ev, a, bar,
                   timeout_ticks);
    else
        MOE_LAUNCH((decode_fused_kernel<2, 2>), grid, dim3(kFusedThreads), lds, stream, ev, a, bar,
                   timeout_ticks);
    return hipGetLastError();
}

}  // namespace moe
