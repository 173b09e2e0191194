// Device helpers shared by the gfx950 kernels of the MXFP4 MoE forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 ---

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

// float -> bf16 bits, round to nearest even (the gfx950 conversion
// v_cvt_pk_bf16_f32; a NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two floats -> packed bf16 pair (lo in bits 0-15) in one conversion.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, b16x2_t));
}

// ------------------------------------------------------ MXFP4 quantizer ---
//
// OCP MX v1.0 rule for one 32-element block: X = 2^(floor(log2 amax) - 2),
// e8m0 byte = floor(log2 amax) - 2 + 127 clamped to [0, 254] (0 for an all-zero
// block); each element becomes the E2M1 code nearest to |x| / X, ties to the
// even mantissa, saturating at 6, with the sign bit of x.
//
// Inputs are bf16 bit patterns: the block maximum is taken on the 15
// magnitude bits (monotonic for finite values) and the scale byte comes from
// its exponent field.

// e8m0 scale byte from the largest |x| (15-bit magnitude pattern) of a block.
__device__ __forceinline__ uint32_t mx_scale_from_amax(uint32_t amax_mag)
{
    uint32_t ea = amax_mag >> 7;              // biased exponent of amax (0: zero/subnormal)
    return ea >= 2u ? ea - 2u : 0u;           // floor(log2 amax) - 2 + 127, clamped at 0
}

// E2M1 codes under scale byte s with gfx950's scaled conversion
// v_cvt_scalef32_pk_fp4_bf16: it takes two bf16 values as they are stored,
// divides by the power of two 2^(s-127) held in the scale operand's exponent
// field, rounds to nearest even and saturates at 6, keeping the sign, and
// writes the two codes into the selected byte of its destination (the other
// bytes pass through).  For every finite bf16 input with |x| / 2^(s-127) < 8
// (always the case when s comes from the block maximum) and every scale byte
// 0..254 its codes equal the OCP rule above bit for bit (checked exhaustively
// on the device against the rule and against the f32-source form of the same
// conversion; the GPU tests compare the quantizer with the CPU reference).
__device__ __forceinline__ float mx_scale_operand(uint32_t s)
{
    return __builtin_bit_cast(float, s << 23);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// byte `SEL` of `old` <- codes of the bf16 pair `pair` (low half -> low nibble)
template <int SEL>
__device__ __forceinline__ uint32_t mx_code_pair(uint32_t old, uint32_t pair, float scale_op)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2_t, pair),
                                                     scale_op, SEL);
}
// four bf16 pairs (8 consecutive elements) -> one dword of codes
__device__ __forceinline__ uint32_t mx_pack8(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                             uint32_t s)
{
    const float so = mx_scale_operand(s);
    uint32_t d = mx_code_pair<0>(0u, p0, so);
    d = mx_code_pair<1>(d, p1, so);
    d = mx_code_pair<2>(d, p2, so);
    return mx_code_pair<3>(d, p3, so);
}
// two elements -> one byte: x0 in the low nibble, x1 in the high nibble
__device__ __forceinline__ uint32_t mx_code2(uint32_t bits0, uint32_t bits1, uint32_t s)
{
    return mx_code_pair<0>(0u, (bits0 & 0xFFFFu) | (bits1 << 16), mx_scale_operand(s)) & 0xFFu;
}
__device__ __forceinline__ uint32_t mx_code(uint32_t bits16, uint32_t s)
{
    return mx_code2(bits16, bits16, s) & 0xFu;
}

// ------------------------------------------------------- lane exchange ---
//
// DPP moves within rows of 16 lanes (a VALU operand modifier, no LDS round
// trip): quad_perm xor 1 / xor 2, row rotate by 4 / 8, row shift so that
// lane l reads lane l + n of its row (lanes past the row end read 0).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;    // row_ror:4
constexpr int kDppRor8 = 0x128;    // row_ror:8
template <int N>
__device__ __forceinline__ uint32_t from_lane_plus(uint32_t v) { return dpp<0x100 + N>(v); }  // row_shl:N

// Maximum over each row of 16 lanes, returned in every lane of the row.
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    v = max(v, dpp<kDppXor1>(v));
    v = max(v, dpp<kDppXor2>(v));
    v = max(v, dpp<kDppRor4>(v));
    v = max(v, dpp<kDppRor8>(v));
    return v;
}

// Pack the E2M1 codes of 8 consecutive lanes (element = lane) into a dword
// held by lanes l % 8 == 0: element 2b in the low nibble of byte b.
__device__ __forceinline__ uint32_t pack8_codes(uint32_t code)
{
    const uint32_t b = code | (dpp<kDppXor1>(code) << 4);
    const uint32_t p2 = b | (from_lane_plus<2>(b) << 8);
    return p2 | (from_lane_plus<4>(p2) << 16);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts within
// rows of 16, then row broadcasts of lane 15 / lane 31 into later rows).
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// silu(g) = g / (1 + e^-g) on the hardware exp2 and reciprocal (about 1 ulp
// each; the result is rounded to bf16 right after).  Very negative g gives
// e^-g = inf and a zero reciprocal (silu -> -0); very positive g gives g.
__device__ __forceinline__ float silu_fast(float g)
{
    const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------------ kernel span -----
//
// Optional record of one kernel's execution on the device's constant-rate
// real-time clock (wall_clock64, hipDeviceAttributeWallClockRate): workgroup
// w = blockIdx.x + gridDim.x * blockIdx.y stores its start in clk[2w] and,
// once all its waves are done, its end in clk[2w + 1] (plain stores to slots
// of its own: no contention).  The kernel's span is the earliest start to
// the latest end; it times the kernel from inside, without the queue
// packets that events attached to a launch add in front of it.  A null clk
// records nothing (clk is a kernel argument: the branches are uniform).
__device__ __forceinline__ int64_t span_slot()
{
    return 2 * (int64_t(blockIdx.y) * gridDim.x + blockIdx.x);
}
__device__ __forceinline__ void span_begin(uint64_t* clk)
{
    if (clk && threadIdx.x == 0) clk[span_slot()] = uint64_t(wall_clock64());
}
// every thread of the workgroup calls it (it holds a workgroup barrier)
__device__ __forceinline__ void span_end(uint64_t* clk)
{
    if (clk) {
        __syncthreads();
        if (threadIdx.x == 0) clk[span_slot() + 1] = uint64_t(wall_clock64());
    }
}

// ------------------------------------------------------------- MFMA -----
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1 (format code 4).
// Lane L supplies 32 E2M1 values (16 bytes) of A row L%16 / B column L%16 at K
// offsets (L/16)*32 .. +32, and one e8m0 scale byte for that 32-block; lane L
// receives D[4*(L/16) + i][L%16] in element i.
__device__ __forceinline__ v4f mfma_fp4_16x16x128(uint4 a, uint4 b, v4f c, uint32_t sa,
                                                   uint32_t sb)
{
    v8i A = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
    v8i B = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, int(sa), 0,
                                                            int(sb));
}

// ------------------------------------------------ bf16 MFMA (A16W4) ----
//
// Weights stay MXFP4 in memory; with bf16 activations they are widened to
// bf16 in registers and multiplied on the bf16 matrix cores.
//
// gfx950's v_cvt_scalef32_pk_bf16_fp4 turns byte SEL of `codes` (two E2M1
// elements, the low nibble first) into a packed bf16 pair, each element's
// value times 2^(s-127) read from the exponent field of the scale operand
// (mx_scale_operand(s)).  The result is exact for every code and every scale
// byte up to 252, subnormal results included; magnitudes past the bf16 range
// (scale bytes 253..255 with large codes) become +-inf (checked on the device
// against the definition for all 256 code bytes at scale bytes 0..255).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair_to_bf16(uint32_t codes, float scale_op)
{
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale_op, SEL));
}
// 8 consecutive elements (one dword of codes) -> 8 bf16, element 0 in the low
// half of .x
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t codes, float scale_op)
{
    return make_uint4(fp4_pair_to_bf16<0>(codes, scale_op), fp4_pair_to_bf16<1>(codes, scale_op),
                      fp4_pair_to_bf16<2>(codes, scale_op), fp4_pair_to_bf16<3>(codes, scale_op));
}

// v_mfma_f32_16x16x32_bf16: lane L supplies A row L%16 / B column L%16 at K
// elements 8*(L/16) .. +8 (8 bf16, element 0 in the low half of .x); lane L
// receives D[4*(L/16) + i][L%16] in element i (the layout of the FP4 MFMA
// above).
__device__ __forceinline__ v4f mfma_bf16_16x16x32(uint4 a, uint4 b, v4f c)
{
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t av = {a.x, a.y, a.z, a.w}, bv = {b.x, b.y, b.z, b.w};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                    __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
}

// A lane's 32-element MX block of weights (16 code bytes, scale byte
// `scale`) -> 32 bf16 in w[0..3], 8 consecutive elements each.
__device__ __forceinline__ void fp4_block_to_bf16(uint4 codes, uint32_t scale, uint4 (&w)[4])
{
    const float so = mx_scale_operand(scale);
    w[0] = fp4x8_to_bf16x8(codes.x, so);
    w[1] = fp4x8_to_bf16x8(codes.y, so);
    w[2] = fp4x8_to_bf16x8(codes.z, so);
    w[3] = fp4x8_to_bf16x8(codes.w, so);
}
// The A16W4 counterpart of one 16x16x128 FP4 MFMA: lane L holds its row's
// 32 bf16 activations x[0..3] of 32-block L/16 of the K tile and the same
// block of its weight column widened by fp4_block_to_bf16.  Four bf16
// products cover the 128 K values: product j takes elements 8j..+8 of every
// lane's block from both operands (the same K values on both sides; the
// order of a sum over K is free).
__device__ __forceinline__ v4f mfma_a16w4_block(const uint4 (&x)[4], const uint4 (&w)[4], v4f c)
{
    c = mfma_bf16_16x16x32(x[0], w[0], c);
    c = mfma_bf16_16x16x32(x[1], w[1], c);
    c = mfma_bf16_16x16x32(x[2], w[2], c);
    return mfma_bf16_16x16x32(x[3], w[3], c);
}

// ------------------------------------------------------------- loads ----

__device__ __forceinline__ uint4 ld16(const uint8_t* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

// Non-temporal 16-byte load for single-use weight streams.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const uint8_t* p)
{
    v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------- fragment layout -------
//
// Sorted-row MXFP4 operands (the gathered activations of the tiled path and
// the stage-1 output h) are stored so that every wave-load is one contiguous
// run: on gfx950 the vector memory path handles a load whose 64 lane
// addresses are consecutive 16 B (or 4 B) chunks about four times faster than
// one that touches several rows.
//   codes  [rows/16][K/128][4 chunks of 32][16 rows][16 B]
//   scales [K/128][rows][4 B]       (byte j = 32-block kt*4 + j of the row)
// A 16x16x128 or 32x32x64 MFMA operand of 16 rows at K tile kt is then the
// 1 KiB at frag_code_off(row0, kt, 0, KT), lane L holding row L%16, chunk L/16.
__device__ __host__ __forceinline__ int64_t frag_code_off(int64_t row, int kt, int chunk, int KT)
{
    return (((row >> 4) * KT + kt) * 64 + chunk * 16 + (row & 15)) * 16;
}
__device__ __host__ __forceinline__ int64_t frag_scale_off(int64_t row, int kt, int64_t rows)
{
    return (int64_t(kt) * rows + row) * 4;
}

}  // namespace moe
