// Route-indexed path for small batches (decode): the two grouped GEMMs of the
// forward without a route sort, a sorted route list, an activation-quant pass
// or a reduction pass.
//
// Same semantics as the sorted path (gemm1.hip and gemm2.hip hold them and the
// passages of the pages they follow).  What changes is the bookkeeping: with a
// few hundred routes the sort, the padding and the separate passes are pure
// launch and latency overhead (each dependent launch costs a few microseconds
// of a ~60 us forward), so the forward is two kernels:
//
// Stage 1, workgroup (c, y): one 64-row group c of the gate_up weight of the
//   y-th active expert in descending id order (grid.y runs to min(E, M*topk),
//   an upper bound of the active experts; surplus workgroups leave at once).
//   Its first wave marks the active experts in an LDS bitmap, picks its own
//   and collects that expert's routes r = t*topk + s (ascending) in LDS.  It
//   quantizes the activations itself: in the 16x16x128 MFMA layout a lane's A
//   operand is one whole 32-element MX block of one row, so the block
//   maximum, e8m0 scale and E2M1 codes come from the lane's registers (same
//   rule and helpers as the standalone quantization kernel, identical codes).
//   h is stored MXFP4 at its route index: a2 [M*topk][I/2] codes +
//   [M*topk][I/32] scales.  The workgroups (0, y) publish slot y's expert and
//   a token -> route table (one layer per repeat of the expert in a token's
//   slots; almost always a single layer).
//
// Stage 2, workgroup n16: one 16-column slice of the output for all tokens.
//   Its waves split the active experts; for each expert a wave streams the
//   slice's down-projection fragments (1 KiB per K tile), gathers the MXFP4 h
//   rows of the expert's tokens into the MFMA rows of those tokens, and adds
//   topk_w * result to fp32 accumulators that stay in registers for the whole
//   kernel; the waves' sums meet in LDS and the slice is written once, as
//   bf16.  Every weight byte is read once, nothing is written per route and
//   no workgroup depends on another; the per-token sum runs over the
//   experts in descending id order (deterministic) with one rounding.
//
// Descending id order: a shared expert is conventionally the last id and has
// a route from every token, the heaviest stage-1 work; its workgroups then
// run first instead of forming the tail.
#include <atomic>
#include <type_traits>

#include "direct_common.h"

namespace moe {

constexpr int kDirThreads = 256;

// ---------------------------------------------------------------- stage 1 --
//
// Workgroup (x, y) of four waves runs stage-1 unit (x % X, y) (stage1_unit,
// direct_common.h; X = direct_stage1_x(I)), K part x / X of KS.
template <int U, int NG, bool A16, int KS = 1>
__global__ void __launch_bounds__(kDirThreads) __attribute__((amdgpu_waves_per_eu(2)))
gemm1_direct_kernel(DirectArgs a)
{
    __shared__ Stage1Lds<NG> L;
    span_begin(a.clk);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int X = direct_stage1_x(a.I);
    stage1_unit<U, NG, A16, KS>(a, blockIdx.x % X, blockIdx.y, wave, L, [] { __syncthreads(); },
                                blockIdx.x / X);
    span_end(a.clk);
}

// ---------------------------------------------------------------- stage 2 --
//
// Workgroup x: output columns x*16*NS .. +16*NS (NS adjacent 16-row slices
// of one 64-row group of the prepared down weight) for every token; RT row
// tiles of 16 tokens.  Its 16 waves split the active slots (wave w takes
// slots w, w + 16, ...); per slot and K tile a wave loads the NS slices'
// weight fragments (NS x 1 KiB, contiguous), one scale word (the slices'
// scale bytes) and, for MFMA row t, the h fragment of token t's route to the
// slot's expert (zero when there is none), shared by the NS slices.  G slots
// x 2 K tiles are loaded before their MFMAs: G x 2 x NS KiB of weights in
// flight per wave, 16 waves per CU (one workgroup per CU, 128 VGPRs each).
//
// A16W4 (a.h16 set): the h fragment of a row is 32 bf16 (64 bytes) of its
// route's bf16 h row, and each weight fragment is widened to bf16 once per
// slot and K tile and shared by the row tiles (mfma_a16w4_block).
constexpr int kOsSlotsInFlight = 2;       // slots loaded before their MFMAs (MXFP4 h)
constexpr int kOsA16SlotsInFlight = 1;    // the same with bf16 h (64-byte fragments)
constexpr int kOsThreads = 1024;
constexpr int kOsWaves = kOsThreads / kWave;
constexpr int kOsSlices = 2;
constexpr int kOsMaxSlots = kDirectMaxTokens * kMaxTopkDirect;
template <int RT, int G, int NS, bool A16, int KH = 2>
__global__ void __launch_bounds__(kOsThreads)
gemm2_direct_kernel(DirectArgs a)
{
    __shared__ int32_t s_e[kOsMaxSlots];
    __shared__ int32_t s_layers[kOsMaxSlots];
    __shared__ int16_t s_route[kOsMaxSlots * 16 * RT];     // layer 0: [slot][token]
    __shared__ float s_tw[kOsMaxSlots];                    // topk_w by route
    __shared__ float red[kOsWaves][NS][RT][4][kWave];
    __shared__ int32_t s_active;
    extern __shared__ __attribute__((aligned(16))) uint8_t hbuf[];   // a.h_lds bytes
    const int n16_0 = blockIdx.x * NS;          // first slice; NS | 4, so one 64-row group
    const int n64 = n16_0 / 4, q0 = n16_0 % 4;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int M = a.M, D = a.D, I = a.I, topk = a.topk;
    const int R = M * topk;
    const int slots = direct_slots(M, a.E, topk);
    const int KT = I / 128;                   // even: KH (1 or 2) K tiles per step

    if (threadIdx.x == 0) s_active = *a.n_active;
    for (int y = threadIdx.x; y < slots; y += kOsThreads) {
        s_e[y] = a.slot_expert[y];
        s_layers[y] = a.slot_layers[y];
    }
    for (int i = threadIdx.x; i < slots * M; i += kOsThreads) {
        const int y = i / M, t = i % M;
        s_route[y * 16 * RT + t] = int16_t(a.route_of[i]);
    }
    for (int r = threadIdx.x; r < R; r += kOsThreads) s_tw[r] = a.tw[r];
    // bf16 h of every route (A16W4, when it fits): staged once, the slots
    // below gather their rows from LDS instead of the L2
    const uint8_t* hl = nullptr;
    if (a.h_lds > 0) {
        const int64_t code_bytes = A16 ? int64_t(R) * I * 2 : int64_t(R) * (I / 2);
        const uint8_t* src = A16 ? reinterpret_cast<const uint8_t*>(a.h16) : a.a2q;
        for (int64_t i = int64_t(threadIdx.x) * 16; i < code_bytes; i += int64_t(kOsThreads) * 16)
            *reinterpret_cast<uint4*>(hbuf + i) = ld16(src + i);
        if constexpr (!A16) {
            const int64_t scale_bytes = int64_t(R) * (I / 32);          // a multiple of 8
            for (int64_t i = int64_t(threadIdx.x) * 8; i < scale_bytes; i += int64_t(kOsThreads) * 8)
                *reinterpret_cast<uint2*>(hbuf + code_bytes + i) =
                    *reinterpret_cast<const uint2*>(a.a2s + i);
        }
        hl = hbuf;
    }
    __syncthreads();
    const int active = s_active;

    const int64_t w_stride = int64_t(D) * (I / 2), s_stride = int64_t(D) * (I / 32);
    // slice s of K tile kt of expert e: wcol + e*w_stride + kt*4096 + s*1024
    const uint8_t* wcol = a.w2p + (int64_t(n64) * KT * 4 + q0) * 1024 + lane * 16;
    const uint8_t* scol = a.w2sp + int64_t(n64) * KT * 256 + lane * 4;      // + e*s_stride + kt*256
    const int row = lane % 16, kq = lane / 16;

    v4f acc[NS][RT];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[sl][rt] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
    for (int y0 = wave; y0 < active; y0 += kOsWaves * G) {
        v4f tmp[G][NS][RT];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int sl = 0; sl < NS; ++sl)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) tmp[g][sl][rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int kt = 0; kt < KT; kt += KH) {
            uint4 b[G][KH][NS];
            HFrag<A16> av[G][KH][RT];
            uint32_t sw[G][KH];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int y = y0 + g * kOsWaves;
                const bool on = y < active;
                const int64_t e = on ? s_e[y] : 0;
#pragma unroll
                for (int h = 0; h < KH; ++h) {
#pragma unroll
                    for (int sl = 0; sl < NS; ++sl)
                        b[g][h][sl] = on ? ld16_nt(wcol + e * w_stride + int64_t(kt + h) * 4096 + sl * 1024)
                                         : make_uint4(0, 0, 0, 0);
                    sw[g][h] = on ? *reinterpret_cast<const uint32_t*>(scol + e * s_stride +
                                                                       (kt + h) * 256)
                                  : 0u;
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const int t = rt * 16 + row;
                    const int r = (on && t < M) ? s_route[y * 16 * RT + t] : -1;
#pragma unroll
                    for (int h = 0; h < KH; ++h) av[g][h][rt] = load_hfrag<A16>(a, r, kt + h, kq, hl);
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int h = 0; h < KH; ++h)
#pragma unroll
                    for (int sl = 0; sl < NS; ++sl)
                        mfma_hfrag<A16, RT>(av[g][h], b[g][h][sl], (sw[g][h] >> (8 * (q0 + sl))) & 0xFFu,
                                            tmp[g][sl]);
        }
        // weight each token's row by its routing weight and accumulate
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int y = y0 + g * kOsWaves;
            if (y >= active) break;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = rt * 16 + 4 * kq + i;
                    const int r = t < M ? s_route[y * 16 * RT + t] : -1;
                    const float w = r >= 0 ? s_tw[r] : 0.0f;
#pragma unroll
                    for (int sl = 0; sl < NS; ++sl) acc[sl][rt][i] += w * tmp[g][sl][rt][i];
                }
        }
    }

    // further layers (a token naming one expert in several slots): rare,
    // one slot and K tile at a time, routes from the global table
#pragma unroll 1
    for (int y = wave; y < active; y += kOsWaves) {
        const int layers = s_layers[y];
        const int64_t e = s_e[y];
#pragma unroll 1
        for (int l = 1; l < layers; ++l) {
            const int32_t* tab = a.route_of + (int64_t(l) * slots + y) * M;
            v4f tmp[NS][RT];
#pragma unroll
            for (int sl = 0; sl < NS; ++sl)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) tmp[sl][rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int kt = 0; kt < KT; ++kt) {
                const uint32_t sw = *reinterpret_cast<const uint32_t*>(scol + e * s_stride + kt * 256);
                HFrag<A16> av[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const int t = rt * 16 + row;
                    av[rt] = load_hfrag<A16>(a, t < M ? tab[t] : -1, kt, kq, hl);
                }
#pragma unroll
                for (int sl = 0; sl < NS; ++sl) {
                    const uint4 b = ld16(wcol + e * w_stride + int64_t(kt) * 4096 + sl * 1024);
                    mfma_hfrag<A16, RT>(av, b, (sw >> (8 * (q0 + sl))) & 0xFFu, tmp[sl]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = rt * 16 + 4 * kq + i;
                    const int r = t < M ? tab[t] : -1;
                    const float w = r >= 0 ? s_tw[r] : 0.0f;
#pragma unroll
                    for (int sl = 0; sl < NS; ++sl) acc[sl][rt][i] += w * tmp[sl][rt][i];
                }
        }
    }

    // the waves' sums, in wave order; one bf16 rounding
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][sl][rt][i][lane] = acc[sl][rt][i];
    __syncthreads();
    for (int o = threadIdx.x; o < M * 16 * NS; o += kOsThreads) {
        const int t = o / (16 * NS), c = o % (16 * NS);
        const int sl = c / 16, col = c % 16;
        const int rt = t / 16, tt = t % 16;
        const int L = col + 16 * (tt / 4), i = tt % 4;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kOsWaves; ++w) sum += red[w][sl][rt][i][L];
        a.out[int64_t(t) * D + n16_0 * 16 + c] = uint16_t(f32_to_bf16_rne(sum));
    }
}

static bool direct_shape_ok(const DirectArgs& a)
{
    return a.M <= kDirectMaxTokens && a.topk <= kMaxTopkDirect &&
           int64_t(a.M) * a.topk <= kDirectMaxRoutes && a.E <= kDirectMaxE;
}

hipError_t launch_gemm1_direct(const DirectArgs& a, hipStream_t stream, const KernelEvents& ev)
{
    if (!direct_shape_ok(a)) return hipErrorInvalidValue;
    if (a.M == 0) return hipSuccess;
    if (a.ks_parts != 1 && (a.ks_parts != 2 || a.h16 || !a.part || !a.split_ctr))
        return hipErrorInvalidValue;
    const dim3 grid(direct_stage1_x(a.I) * a.ks_parts, direct_slots(a.M, a.E, a.topk));
    if (a.h16)
        MOE_LAUNCH((gemm1_direct_kernel<kG1Unroll, kDirectGroups, true>), grid,
                   dim3(kDirThreads), 0, stream, ev, a);
    else if (a.ks_parts == 2)
        MOE_LAUNCH((gemm1_direct_kernel<kG1Unroll, kDirectGroups, false, 2>), grid,
                   dim3(kDirThreads), 0, stream, ev, a);
    else
        MOE_LAUNCH((gemm1_direct_kernel<kG1Unroll, kDirectGroups, false>), grid,
                   dim3(kDirThreads), 0, stream, ev, a);
    return hipGetLastError();
}

// The four stage-2 instances, and the LDS each can take for h beyond its
// static arrays (the CU's 160 KiB less those), found once per process.
static const void* const kG2Direct[4] = {
    reinterpret_cast<const void*>(&gemm2_direct_kernel<1, kOsA16SlotsInFlight, kOsSlices, true>),
    reinterpret_cast<const void*>(&gemm2_direct_kernel<2, 1, kOsSlices, true, 1>),
    reinterpret_cast<const void*>(&gemm2_direct_kernel<1, kOsSlotsInFlight, kOsSlices, false>),
    reinterpret_cast<const void*>(&gemm2_direct_kernel<2, 1, kOsSlices, false>)};
static std::atomic<int> g_h_lds_max[4];   // written once per device set-up (same values)
constexpr int kCuLds = 160 * 1024;

hipError_t direct_allow_lds()
{
    for (int i = 0; i < 4; ++i) {
        hipFuncAttributes attr;
        hipError_t e = hipFuncGetAttributes(&attr, kG2Direct[i]);
        if (e != hipSuccess) return e;
        const int avail = kCuLds - int(attr.sharedSizeBytes);
        if (avail <= 0) continue;
        e = hipFuncSetAttribute(kG2Direct[i], hipFuncAttributeMaxDynamicSharedMemorySize, avail);
        if (e != hipSuccess) return e;
        g_h_lds_max[i].store(avail, std::memory_order_relaxed);
    }
    return hipSuccess;
}

hipError_t launch_gemm2_direct(const DirectArgs& a0, hipStream_t stream, const KernelEvents& ev)
{
    if (!direct_shape_ok(a0)) return hipErrorInvalidValue;
    if (a0.M == 0) return hipSuccess;
    const dim3 grid(a0.D / (16 * kOsSlices));
    const int inst = (a0.h16 ? 0 : 2) + (a0.M <= 16 ? 0 : 1);
    const int64_t R = int64_t(a0.M) * a0.topk;
    const int64_t hbytes = a0.h16 ? R * a0.I * 2 : R * (a0.I / 2 + a0.I / 32);
    DirectArgs a = a0;
    // bf16 h (A16W4) is four times the MXFP4 codes: staging it pays for its copy
    // (decode stage 2 24.5 -> 23.4 us); the MXFP4 h gathers from the L2 cost less
    // than copying it (21.5 -> 22.3 us when staged), so those stay global
    a.h_lds = a0.h16 && hbytes <= g_h_lds_max[inst].load(std::memory_order_relaxed) ? int(hbytes) : 0;
    const uint32_t dyn = uint32_t(a.h_lds);
    switch (inst) {
    case 0:
        MOE_LAUNCH((gemm2_direct_kernel<1, kOsA16SlotsInFlight, kOsSlices, true>), grid,
                   dim3(kOsThreads), dyn, stream, ev, a);
        break;
    case 1:
        MOE_LAUNCH((gemm2_direct_kernel<2, 1, kOsSlices, true, 1>), grid, dim3(kOsThreads), dyn,
                   stream, ev, a);
        break;
    case 2:
        MOE_LAUNCH((gemm2_direct_kernel<1, kOsSlotsInFlight, kOsSlices, false>), grid,
                   dim3(kOsThreads), dyn, stream, ev, a);
        break;
    default:
        MOE_LAUNCH((gemm2_direct_kernel<2, 1, kOsSlices, false>), grid, dim3(kOsThreads), dyn,
                   stream, ev, a);
        break;
    }
    return hipGetLastError();
}

// Debug view of the route-indexed rows: row r holds route r when its id is
// valid, else the sentinel M*topk; num_valid = {M*topk, valid routes}.
__global__ void direct_rows_kernel(const int32_t* __restrict__ ids, int R, int E,
                                   int32_t* __restrict__ row_route, int32_t* __restrict__ num_valid)
{
    __shared__ int32_t count;
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    int mine = 0;
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
        const bool v = ids[r] >= 0 && ids[r] < E;
        if (row_route) row_route[r] = v ? r : R;
        mine += v;
    }
    atomicAdd(&count, mine);
    __syncthreads();
    if (threadIdx.x == 0 && num_valid) {
        num_valid[0] = R;
        num_valid[1] = count;
    }
}

hipError_t launch_direct_rows(const int32_t* ids, int R, int E, int32_t* row_route,
                              int32_t* num_valid, hipStream_t stream)
{
    hipLaunchKernelGGL(direct_rows_kernel, dim3(1), dim3(256), 0, stream, ids, R, E, row_route,
                       num_valid);
    return hipGetLastError();
}

}  // namespace moe
