// Device helpers of the route-indexed (decode) kernels, shared by the
// two-launch kernels (direct.hip) and the single persistent launch
// (decode_fused.hip): the route scan, raw buffer loads, the in-register
// activation quantizer, the stage-2 table publication and the stage-2
// operand fragments.
#pragma once

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {
constexpr int kG1Unroll = 1;     // K tiles per double-buffered chunk (x NG x 4 KiB of weights)
}

namespace moe {

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
// One stage-1 unit (x, y): NG consecutive 64-row groups c = x*NG + j of the
// prepared gate_up weight of the y-th active expert e (gate columns
// c*32..+31 and the matching up columns), all K = D, run by four waves
// (`wave` 0..3) that split K as in the sorted streaming kernel.  The NG
// groups share the route scan and each K tile's activation fragment (loaded
// as bf16 and quantized once).  `sync` joins the four waves (a workgroup
// barrier when they are the whole workgroup, a team barrier when several
// teams share one).  The unit with x = 0 publishes slot y's stage-2 tables.
// Returns the number of active experts.
//
// A16W4 (a.h16 set): the bf16 activations go to the bf16 matrix cores as
// they are and each weight fragment is widened to bf16 in registers
// (mfma_a16w4_block); h stays bf16, stored at its route in a.h16.
template <int NG>
struct Stage1Lds {
    int32_t list[kDirectMaxRoutes];
    uint32_t bitmap[kDirectMaxE / 32];
    int32_t n_list, e_sel, n_active, last;
    float red[4][NG][4][4][kWave];      // [wave][group][slice][i][lane]
};

// Split-K partial sums of stage 1 (KS > 1), fp32, by route: for K part k,
// route r, 64-row group c, 16-row slice q and column j of the slice,
// part[((k * R + r) * (I/32) + c) * 64 + q * 16 + j].  They are written and
// read with agent-coherent accesses (write-through; reads from the coherence
// point), which is what lets the merging workgroup on another XCD see them
// without cache maintenance.
__device__ __forceinline__ int64_t split_part_off(int k, int64_t r, int R, int I, int c, int q, int j)
{
    return ((int64_t(k) * R + r) * (I / 32) + c) * 64 + q * 16 + j;
}

// The end of stage 1 for one lane's row of one 64-row group c, from the
// group's four fp32 sums s4 (gate columns c*32 + lane%16 and +16, then the
// matching up columns): h = bf16(silu(gate) * up), then (MXFP4 mode) the
// requant of the 32 h of the row held by the 16 lanes of the DPP row, stored
// by route; A16W4 stores h as bf16.  Every lane of the wave calls it (the
// block maximum is a cross-lane reduction); lanes without a row store nothing.
template <bool A16>
__device__ __forceinline__ void stage1_finish(const DirectArgs& a, int64_t r, bool row_ok, int c,
                                              const float (&s4)[4])
{
    const int lane = threadIdx.x % kWave;
    const int I = a.I;
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
        return;
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

template <int U, int NG, bool A16, int KS = 1, class Sync>
__device__ __forceinline__ int stage1_unit(const DirectArgs& a, int x, int y, int wave,
                                           Stage1Lds<NG>& L, Sync sync, int ks = 0)
{
    int32_t* list = L.list;
    const int lane = threadIdx.x % kWave;
    const int R = a.M * a.topk;
    const int D = a.D, I = a.I;
    if (wave == 0) {
        int nw, ew, active;
        active_expert_routes(a.ids, R, a.E, y, L.bitmap, list, nw, ew, active);
        if (lane == 0) {
            L.n_list = nw;
            L.e_sel = ew;
            L.n_active = active;
        }
        if (x == 0 && ks == 0) publish_slot(a, y, list, nw, ew, active);
    }
    sync();
    const int n = L.n_list, e = L.e_sel, active = L.n_active;
    if (e < 0) return active;

    const int KT = D / 128;
    const uint32_t gstride = uint32_t(KT) * 4096, sgstride = uint32_t(KT) * 256;   // per 64-row group
    // this workgroup's NG groups of codes and scales, and the hidden rows
    const auto wres = buffer_rsrc(a.w13p + int64_t(e) * I * D + int64_t(x) * NG * gstride,
                                  NG * gstride);
    const auto sres = buffer_rsrc(a.w13sp + int64_t(e) * I * D / 16 + int64_t(x) * NG * sgstride,
                                  NG * sgstride);
    const uint32_t hbytes = uint32_t(a.M) * D * 2;
    const auto hres = buffer_rsrc(a.hidden, hbytes);
    // K part ks of KS, split over the four waves
    const int kp0 = ks * KT / KS, kp1 = (ks + 1) * KT / KS;
    const int kt_begin = kp0 + wave * (kp1 - kp0) / 4, kt_end = kp0 + (wave + 1) * (kp1 - kp0) / 4;

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
                for (int i = 0; i < 4; ++i) L.red[wave][g][q][i][lane] = acc[g][q][i];
        sync();

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
                s4[q] = L.red[0][g][q][i][lane] + L.red[1][g][q][i][lane] + L.red[2][g][q][i][lane] +
                        L.red[3][g][q][i][lane];
            if constexpr (KS > 1) {
                // this part's sums, written through for the merging workgroup
                if (row_ok)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        __hip_atomic_store(a.part + split_part_off(ks, r, R, I, c, q, lane % 16), s4[q],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                stage1_finish<A16>(a, r, row_ok, c, s4);
            }
        }
        sync();                   // red is rewritten by the next row tile
    }
    if constexpr (KS > 1) {
        // The last of the unit's KS workgroups to get here merges: every
        // wave waits until its partial stores have completed (written
        // through), then one thread counts this part in; the count returns
        // to zero after the last part, ready for the next call.  The merge
        // adds the parts in part order, so the result does not depend on
        // which workgroup merges.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        sync();
        if (wave == 0 && lane == 0) {
            uint32_t* ctr = a.split_ctr + y * (I / (32 * NG)) + x;
            const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            L.last = old == KS - 1;
            if (old == KS - 1) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        sync();
        if (!L.last) return active;
#pragma unroll 1
        for (int t0 = 0; t0 < n; t0 += 16) {
            const int jr = t0 + 4 * (lane / 16) + wave;
            if (jr >= n) continue;
            const int64_t r = list[jr];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int c = x * NG + g;
                float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < KS; ++k)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        s4[q] += __hip_atomic_load(a.part + split_part_off(k, r, R, I, c, q, lane % 16),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                stage1_finish<A16>(a, r, true, c, s4);
            }
        }
    }
    return active;
}

// ------------------------------------------------------- stage-2 operands --


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

}  // namespace moe
