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

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kDirThreads = 256;
constexpr int kG1Unroll = 1;     // K tiles per double-buffered chunk (x NG x 4 KiB of weights)

// Picks this workgroup's expert and its routes; run by one whole wave.
// Pass 1 marks the experts that have a route in an LDS bitmap; the y-th
// marked expert in descending id order is this workgroup's, or none
// (*e_out = -1) when fewer than y + 1 experts are active (*active_out = the
// number of active experts).  Pass 2 (the ids again, now in the L1 cache)
// collects that expert's routes r = t*topk + s, ascending, into list[] and
// their number into *n_out.  Ids outside [0, E) are skipped.
__device__ __forceinline__ void active_expert_routes(const int32_t* __restrict__ ids, int R, int E,
                                                     int y, uint32_t* bitmap, int32_t* list,
                                                     int& n_out, int& e_out, int& active_out)
{
    const int lane = threadIdx.x % kWave;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int words = (E + 31) / 32;
    if (lane < words) bitmap[lane] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll 1
    for (int base = 0; base < R; base += 4 * kWave) {
        int id[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = base + u * kWave + lane;
            id[u] = r < R ? ids[r] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (id[u] >= 0 && id[u] < E) atomicOr(&bitmap[id[u] / 32], 1u << (id[u] % 32));
    }
    __builtin_amdgcn_wave_barrier();
    // word w of the bitmap on lane words-1-w (highest expert ids first); the
    // y-th set bit in descending order
    const int wi = words - 1 - lane;
    uint32_t w = lane < words ? bitmap[wi] : 0u;
    const int pc = __popc(w);
    const int inc = wave_inclusive_scan(pc);
    const bool mine = y >= inc - pc && y < inc;
    int e = -1;
    if (mine) {
        for (int k = y - (inc - pc); k > 0; --k) w &= ~(0x80000000u >> __builtin_clz(w));  // drop the upper set bits
        e = wi * 32 + 31 - __builtin_clz(w);
    }
    const uint64_t who = __ballot(mine);
    e = who ? __builtin_amdgcn_readlane(e, __builtin_ctzll(who)) : -1;
    int n = 0;
    if (e >= 0) {
#pragma unroll 1
        for (int base = 0; base < R; base += 4 * kWave) {
            int id[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = base + u * kWave + lane;
                id[u] = r < R ? ids[r] : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool hit = id[u] == e;
                const uint64_t m = __ballot(hit);
                if (hit) list[n + __popcll(m & below)] = base + u * kWave + lane;
                n += __popcll(m);
            }
        }
    }
    n_out = n;
    e_out = e;
    active_out = __builtin_amdgcn_readlane(inc, kWave - 1);
}

// Raw buffer loads: a wave-uniform base and size in a buffer resource
// (SGPRs), a 32-bit per-lane offset, a uniform offset and an immediate, so a
// wave keeps one address register per stream instead of one 64-bit address
// per load in flight; offsets at or past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                             0x00020000);
}
constexpr int kCacheStream = 2;            // non-temporal (single-use weight streams)
template <int IMM, int AUX = 0>
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(voff + IMM), int(soff), AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), int(soff), 0);
}

// One 32-element MX block held by one lane as 64 bytes of bf16 (x[0] =
// elements 0..7, ...): returns its 16 code bytes (byte b = elements 2b, 2b+1)
// and the e8m0 scale byte.
__device__ __forceinline__ uint4 mx_quant_lane_block(const uint4 (&x)[4], uint32_t& scale)
{
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = {0, 0};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t w[4] = {x[p].x, x[p].y, x[p].z, x[p].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
    }
    const uint32_t s = mx_scale_from_amax(max(uint32_t(m.x), uint32_t(m.y)));
    scale = s;
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) out[p] = mx_pack8(x[p].x, x[p].y, x[p].z, x[p].w, s);
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Slot y's entry for stage 2 (wave 0 of workgroup (0, y), after the route
// scan): the expert (or -1), the number of layers L (the most routes any one
// token has to this expert, 0 if none) and the token -> route table of each
// layer l < L: route_of[(l*slots + y)*M + t] = the l-th route of token t to
// this expert, or -1.  Layer 0 is written for every slot, so stage 2 can
// read all of it without knowing which slots are active.  A token's routes to
// one expert are adjacent in the ascending list; lane t finds them by binary
// search.  Workgroup (0, 0) also stores the number of active experts.
__device__ __forceinline__ void publish_slot(const DirectArgs& a, int y, const int32_t* list, int n,
                                             int e, int active)
{
    const int lane = threadIdx.x % kWave;
    const int slots = direct_slots(a.M, a.E, a.topk);
    int first = 0, cnt = 0;
    if (e >= 0 && lane < a.M) {
        const int lo_key = lane * a.topk, hi_key = lo_key + a.topk;
        int lo = 0, hi = n;
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (list[mid] < lo_key) lo = mid + 1; else hi = mid;
        }
        first = lo;
        hi = n;
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (list[mid] < hi_key) lo = mid + 1; else hi = mid;
        }
        cnt = lo - first;
    }
    int layers = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) layers = max(layers, __shfl_xor(layers, off));
    if (lane == 0) {
        a.slot_expert[y] = e;
        a.slot_layers[y] = layers;
        if (y == 0) *a.n_active = active;
    }
    for (int l = 0; l < max(layers, 1); ++l)
        if (lane < a.M)
            a.route_of[(int64_t(l) * slots + y) * a.M + lane] = l < cnt ? list[first + l] : -1;
}

// ---------------------------------------------------------------- stage 1 --
//
// Workgroup (x, y): NG consecutive 64-row groups c = x*NG + j of the prepared
// gate_up weight of the y-th active expert e (gate columns c*32..+31 and the
// matching up columns), all K = D, four waves splitting K as in the sorted
// streaming kernel.  The NG groups share the route scan and each K tile's
// activation fragment (loaded as bf16 and quantized once).
//
// A16W4 (a.h16 set): the bf16 activations go to the bf16 matrix cores as
// they are and each weight fragment is widened to bf16 in registers
// (mfma_a16w4_block); h stays bf16, stored at its route in a.h16.
template <int U, int NG, bool A16>
__global__ void __launch_bounds__(kDirThreads)
gemm1_direct_kernel(DirectArgs a)
{
    __shared__ int32_t list[kDirectMaxRoutes];
    __shared__ uint32_t bitmap[kDirectMaxE / 32];
    __shared__ int32_t n_list, e_sel;
    __shared__ float red[4][NG][4][4][kWave];      // [wave][group][slice][i][lane]
    const int x = blockIdx.x, y = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int R = a.M * a.topk;
    const int D = a.D, I = a.I;
    span_begin(a.clk);
    if (wave == 0) {
        int nw, ew, active;
        active_expert_routes(a.ids, R, a.E, y, bitmap, list, nw, ew, active);
        if (lane == 0) {
            n_list = nw;
            e_sel = ew;
        }
        if (x == 0) publish_slot(a, y, list, nw, ew, active);
    }
    __syncthreads();
    const int n = n_list, e = e_sel;
    if (e < 0) {
        span_end(a.clk);
        return;
    }

    const int KT = D / 128;
    const uint32_t gstride = uint32_t(KT) * 4096, sgstride = uint32_t(KT) * 256;   // per 64-row group
    // this workgroup's NG groups of codes and scales, and the hidden rows
    const auto wres = buffer_rsrc(a.w13p + int64_t(e) * I * D + int64_t(x) * NG * gstride,
                                  NG * gstride);
    const auto sres = buffer_rsrc(a.w13sp + int64_t(e) * I * D / 16 + int64_t(x) * NG * sgstride,
                                  NG * sgstride);
    const uint32_t hbytes = uint32_t(a.M) * D * 2;
    const auto hres = buffer_rsrc(a.hidden, hbytes);
    const int kt_begin = wave * KT / 4, kt_end = (wave + 1) * KT / 4;

#pragma unroll 1
    for (int t0 = 0; t0 < n; t0 += 16) {
        const int j = t0 + lane % 16;
        // this lane's 32 bf16 of its row at K tile kt: 64 bytes at hoff + kt*256
        // (rows past the expert's routes read as zero)
        const uint32_t hoff = j < n ? uint32_t(list[j] / a.topk) * D * 2 + (lane / 16) * 64 : hbytes;

        v4f acc[NG][4];
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[g][q] = v4f{0.f, 0.f, 0.f, 0.f};

        // chunks of U K tiles; the loads of the next chunk are issued before
        // the quantization and MFMAs of the current one (register double
        // buffering); tiles past the wave's K range load nothing and add zero
        uint4 b0[U][NG][4], b1[U][NG][4], x0[U][4], x1[U][4];
        uint32_t s0[U][NG], s1[U][NG];
        auto load = [&](uint4 (&b)[U][NG][4], uint4 (&xa)[U][4], uint32_t (&sw)[U][NG], int kt0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kt = kt0 + u;
                const bool in = kt < kt_end;
                const uint32_t wo = in ? lane * 16 + uint32_t(kt) * 4096 : NG * gstride;
                const uint32_t so = in ? lane * 4 + uint32_t(kt) * 256 : NG * sgstride;
                const uint32_t ho = in ? hoff + uint32_t(kt) * 256 : hbytes;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    sw[u][g] = bld4(sres, so, g * sgstride);
                    b[u][g][0] = bld16<0, kCacheStream>(wres, wo, g * gstride);
                    b[u][g][1] = bld16<1024, kCacheStream>(wres, wo, g * gstride);
                    b[u][g][2] = bld16<2048, kCacheStream>(wres, wo, g * gstride);
                    b[u][g][3] = bld16<3072, kCacheStream>(wres, wo, g * gstride);
                }
                xa[u][0] = bld16<0>(hres, ho, 0);
                xa[u][1] = bld16<16>(hres, ho, 0);
                xa[u][2] = bld16<32>(hres, ho, 0);
                xa[u][3] = bld16<48>(hres, ho, 0);
            }
        };
        auto compute = [&](const uint4 (&b)[U][NG][4], const uint4 (&xa)[U][4],
                           const uint32_t (&sw)[U][NG]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (A16) {
#pragma unroll
                    for (int g = 0; g < NG; ++g)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            uint4 w[4];
                            fp4_block_to_bf16(b[u][g][q], (sw[u][g] >> (8 * q)) & 0xFFu, w);
                            acc[g][q] = mfma_a16w4_block(xa[u], w, acc[g][q]);
                        }
                } else {
                    uint32_t sa;
                    const uint4 av = mx_quant_lane_block(xa[u], sa);
#pragma unroll
                    for (int g = 0; g < NG; ++g)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[g][q] = mfma_fp4_16x16x128(av, b[u][g][q], acc[g][q], sa,
                                                           (sw[u][g] >> (8 * q)) & 0xFFu);
                }
            }
        };
        const int nchunks = (kt_end - kt_begin + U - 1) / U;
        if (nchunks > 0) load(b0, x0, s0, kt_begin);
        for (int ci = 0; ci < nchunks; ci += 2) {
            if (ci + 1 < nchunks) load(b1, x1, s1, kt_begin + (ci + 1) * U);
            compute(b0, x0, s0);
            if (ci + 1 >= nchunks) break;
            if (ci + 2 < nchunks) load(b0, x0, s0, kt_begin + (ci + 2) * U);
            compute(b1, x1, s1);
        }

#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wave][g][q][i][lane] = acc[g][q][i];
        __syncthreads();

        // wave w finishes element i = w of every lane: row 4*(lane/16) + w of the tile
        const int i = wave;
        const int jr = t0 + 4 * (lane / 16) + i;
        const bool row_ok = jr < n;
        const int64_t r = row_ok ? list[jr] : 0;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int c = x * NG + g;
            float s4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                s4[q] = red[0][g][q][i][lane] + red[1][g][q][i][lane] + red[2][g][q][i][lane] +
                        red[3][g][q][i][lane];
            // slices 0,1 = gate columns c*32 + lane%16 (+16), slices 2,3 = up
            const uint32_t h0 = f32_to_bf16_rne(silu_fast(s4[0]) * s4[2]);
            const uint32_t h1 = f32_to_bf16_rne(silu_fast(s4[1]) * s4[3]);
            if (a.h_dbg && row_ok) {
                a.h_dbg[r * I + c * 32 + lane % 16] = uint16_t(h0);
                a.h_dbg[r * I + c * 32 + 16 + lane % 16] = uint16_t(h1);
            }
            if constexpr (A16) {
                if (row_ok) {
                    a.h16[r * I + c * 32 + lane % 16] = uint16_t(h0);
                    a.h16[r * I + c * 32 + 16 + lane % 16] = uint16_t(h1);
                }
                continue;
            }
            // the row's MXFP4 group = columns c*32..+31, held by the 16 lanes of a DPP row
            const uint32_t s = mx_scale_from_amax(row16_max(max(h0 & 0x7FFFu, h1 & 0x7FFFu)));
            const uint32_t qlo = pack8_codes(mx_code(h0, s));   // bytes 0-3 on lane%16 == 0
            const uint32_t qhi = pack8_codes(mx_code(h1, s));   // bytes 8-11
            const uint32_t d1 = from_lane_plus<8>(qlo);         // bytes 4-7
            const uint32_t d3 = from_lane_plus<8>(qhi);         // bytes 12-15
            if (row_ok && lane % 16 == 0) {
                *reinterpret_cast<uint4*>(a.a2q + r * (I / 2) + c * 16) = make_uint4(qlo, d1, qhi, d3);
                a.a2s[r * (I / 32) + c] = uint8_t(s);
            }
        }
        __syncthreads();          // red is rewritten by the next row tile
    }
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

// One row's stage-2 operand at K tile kt for route r (r < 0: none, zeros):
// MXFP4 (16 code bytes + scale byte of 32-block kq) or, A16W4, 32 bf16.
template <bool A16>
struct HFrag {
    uint4 v[A16 ? 4 : 1];
    uint32_t s;
};
// hl: h staged in LDS (A16W4: [M*topk][I] bf16; else the codes [M*topk][I/2]
// followed by the scales [M*topk][I/32]), or null to read the global copy.
template <bool A16>
__device__ __forceinline__ HFrag<A16> load_hfrag(const DirectArgs& a, int r, int kt, int kq,
                                                 const uint8_t* hl)
{
    HFrag<A16> f;
    const int I = a.I;
    if constexpr (A16) {
        f.s = 0u;
        const int64_t off = (int64_t(r) * I + kt * 128 + kq * 32) * 2;
        if (hl) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f.v[j] = r >= 0 ? *reinterpret_cast<const uint4*>(hl + off + 16 * j) : make_uint4(0, 0, 0, 0);
        } else {
            const uint8_t* p = reinterpret_cast<const uint8_t*>(a.h16) + off;
#pragma unroll
            for (int j = 0; j < 4; ++j) f.v[j] = r >= 0 ? ld16(p + 16 * j) : make_uint4(0, 0, 0, 0);
        }
    } else {
        const int64_t off = int64_t(r) * (I / 2) + kt * 64 + kq * 16;
        const int64_t soff = int64_t(r) * (I / 32) + kt * 4 + kq;
        if (hl) {
            const int64_t codes = int64_t(a.M) * a.topk * (I / 2);
            f.v[0] = r >= 0 ? *reinterpret_cast<const uint4*>(hl + off) : make_uint4(0, 0, 0, 0);
            f.s = r >= 0 ? hl[codes + soff] : 0u;
        } else {
            f.v[0] = r >= 0 ? ld16(a.a2q + off) : make_uint4(0, 0, 0, 0);
            f.s = r >= 0 ? a.a2s[soff] : 0u;
        }
    }
    return f;
}
// acc[rt] += product of the rows' fragments f[rt] with one weight fragment
// (16 code bytes, scale byte sb) over K tile kt
template <bool A16, int RT>
__device__ __forceinline__ void mfma_hfrag(const HFrag<A16> (&f)[RT], uint4 b, uint32_t sb,
                                           v4f (&acc)[RT])
{
    if constexpr (A16) {
        uint4 w[4];
        fp4_block_to_bf16(b, sb, w);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma_a16w4_block(f[rt].v, w, acc[rt]);
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma_fp4_16x16x128(f[rt].v[0], b, acc[rt], f[rt].s, sb);
    }
}

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
    const dim3 grid(direct_stage1_x(a.I), direct_slots(a.M, a.E, a.topk));
    if (a.h16)
        MOE_LAUNCH((gemm1_direct_kernel<kG1Unroll, kDirectGroups, true>), grid,
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
