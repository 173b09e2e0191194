/*
 * moe_mxfp4.h -- C ABI of the MI355X (gfx950) fused MXFP4 Mixture-of-Experts
 * forward: route sort -> dynamic MXFP4 activation quant -> gate_up GEMM with
 * fused SwiGLU (+ MXFP4 requant) -> down GEMM weighted by the routing weights
 * and accumulated per token into bf16.
 *
 * The operation follows the FP4 ("a4w4") pipeline of kernelindex.com
 * amd-moe-mxfp4 submission 754773 (`custom_kernel`, FP4 branch): activations
 * are MXFP4-quantized before stage 1, the bf16 SwiGLU output is re-quantized
 * before stage 2, and the routing weight is applied in stage 2 only.  Weight
 * rows follow submission 723815's `_reference_forward`: rows 0..I-1 of the
 * gate_up weight are the gate projection, rows I..2I-1 the up projection,
 * act = silu(gate) * up.
 *
 * MXFP4 tensor format (both pages): two E2M1 codes per byte, element 2j in the
 * low nibble and 2j+1 in the high nibble; one e8m0 scale byte (value
 * 2^(s-127)) per 32 consecutive elements along the contraction dimension K.
 * Activation quantization (OCP MX v1.0): scale = 2^(floor(log2 amax) - 2)
 * clamped to the e8m0 range, codes = round-to-nearest-even of x / scale,
 * saturating at +-6, sign kept.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device and must
 *    be 16-byte aligned (the forward's workspace 256-byte aligned).  bf16
 *    tensors are passed as uint16_t bit patterns.  16 bytes is the widest
 *    access any kernel makes to a caller's tensor (one 16-byte vector load or
 *    store per lane), so it is all they need; submission 723815 asserts
 *    128-byte alignment of its shuffled scale tensors for its own kernels,
 *    which these do not share.  The workspace is carved into sub-buffers at
 *    256-byte boundaries, hence its stricter rule.
 *  - The caller owns every buffer, including the workspace.  The library keeps
 *    no pointer after a call returns and allocates no device memory.
 *  - Work is enqueued asynchronously on `stream`; nothing synchronizes with the
 *    host.  Device-side faults surface at the caller's next synchronization.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is enqueued and outputs are untouched.
 *  - Return value: one of the MOE_MXFP4_* status codes below.
 *  - Concurrent calls on different streams must use different workspaces and
 *    outputs.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_MXFP4_OK = 0,
    MOE_MXFP4_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, bad size      */
    MOE_MXFP4_ERR_UNSUPPORTED = 2,  /* device is not gfx950, or shape too large */
    MOE_MXFP4_ERR_WORKSPACE = 3,    /* workspace smaller than required           */
    MOE_MXFP4_ERR_HIP = 4           /* a HIP runtime call or launch failed       */
};

/* Kernel paths of the forward (moe_mxfp4_path). */
enum {
    MOE_MXFP4_PATH_DIRECT = 1,      /* few tokens: route-indexed, no route sort  */
    MOE_MXFP4_PATH_STREAM = 2,      /* expert-sorted, weight-streaming kernels   */
    MOE_MXFP4_PATH_TILED = 3        /* expert-sorted, LDS-tiled kernels          */
};

/* Human-readable text of a status code (static storage, never NULL). */
const char* moe_mxfp4_status_string(int status);

/* Limits of this implementation (host-validated):
 *   D, I: multiples of 256, 256 <= D, I <= 65536
 *   1 <= E <= 1024, 1 <= topk <= 32, 0 <= M, M * topk <= 2^24;
 *   on the TILED path (moe_mxfp4_path) also I * D < 2^31 and
 *   max(D, I) / 128 * moe_mxfp4_route_capacity(M, E, topk, 256) * 4 < 2^32
 *   (its kernels address one expert's weights and the sorted operands' scale
 *   words with 32-bit offsets); a shape beyond them is
 *   MOE_MXFP4_ERR_UNSUPPORTED, and the shape queries below return 0 for it. */

/* ---------------------------------------------------------------------------
 * Weight preparation (offline, once per weight set).
 *
 * Passage: both kernelindex.com amd-moe-mxfp4 submissions receive each weight
 * set twice in their input tuple, raw and pre-shuffled for their kernels
 * (the `*_shuffled` gate_up / down weights and scales that `custom_kernel`
 * passes to its fused MoE call, next to the raw ones that the reference
 * `_dequant` / `_reference_forward` of submission 723815 reads).  The
 * shuffle is kernel-specific and the pages do not define it; this call is the
 * equivalent step for this library's kernels: a pure permutation of bytes
 * that leaves every code and scale value unchanged.
 *
 * Permutes raw MXFP4 weights into the kernel layout.  Raw layouts:
 *   w13       u8 [E, 2I, D/2]   gate_up codes (rows 0..I-1 gate, I..2I-1 up)
 *   w13_scale u8 [E, 2I, D/32]  e8m0 scales
 *   w2        u8 [E, D, I/2]    down codes
 *   w2_scale  u8 [E, D, I/32]   e8m0 scales
 * Outputs have exactly the same byte sizes; the mapping is a bijection
 * (moe_mxfp4_unprepare_weights inverts it).  Inputs and outputs must not
 * alias.  Prepared layout, per expert, for a matrix with N rows and K columns
 * (gate_up: N = 2I, K = D; down: N = D, K = I):
 *   codes  [N/64][K/128][4][64][16 B]: 16-row slice q of 64-row group n64,
 *          K tile kt (128 elements); lane L holds row n64*64 + q*16 + L%16,
 *          elements kt*128 + (L/16)*32 .. +32 (the raw 16 bytes).
 *   scales [N/64][K/128][64][4 B]: byte q of lane L's word at K tile kt is
 *          the scale of row n64*64 + q*16 + L%16, 32-block kt*4 + L/16.
 * For gate_up the rows are first interleaved so that each 64-row group holds
 * gate rows c*32..c*32+31 followed by up rows I+c*32..I+c*32+31 (group c).
 * ------------------------------------------------------------------------- */
int moe_mxfp4_prepare_weights(const uint8_t* w13, const uint8_t* w13_scale,
                              const uint8_t* w2, const uint8_t* w2_scale,
                              int E, int D, int I,
                              uint8_t* w13_out, uint8_t* w13_scale_out,
                              uint8_t* w2_out, uint8_t* w2_scale_out,
                              hipStream_t stream);

/* Inverse of moe_mxfp4_prepare_weights (same arguments, prepared -> raw). */
int moe_mxfp4_unprepare_weights(const uint8_t* w13p, const uint8_t* w13p_scale,
                                const uint8_t* w2p, const uint8_t* w2p_scale,
                                int E, int D, int I,
                                uint8_t* w13_out, uint8_t* w13_scale_out,
                                uint8_t* w2_out, uint8_t* w2_scale_out,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Forward.
 *
 * out[t, :] = bf16( sum_{s < topk, 0 <= e < E} topk_w[t, s] *
 *                   W2[e] . Q( bf16( silu(Wg[e] . Q(hidden[t])) * (Wu[e] . Q(hidden[t])) ) ) )
 * with e = topk_ids[t, s], Q = MXFP4 quantization per 32 along K, dot products
 * of MXFP4 operands accumulated in fp32, the per-token sum over slots in fp32
 * and one final rounding to bf16.  The result is deterministic; the order of
 * that sum depends on the path (moe_mxfp4_path): on the sorted paths each
 * weighted contribution is rounded to bf16 and the sum runs in slot order; on
 * the DIRECT path the contributions stay fp32 and the sum runs over the
 * experts in descending id order (partial sums of 16 interleaved subsets,
 * then added in a fixed order).
 *
 *   hidden    bf16 [M, D]            activations
 *   w13..     prepared weights from moe_mxfp4_prepare_weights
 *   topk_ids  i32  [M, topk]          expert per (token, slot); ids outside
 *                                     [0, E) contribute nothing; a repeated
 *                                     id counts once per slot.  A shared
 *                                     expert is an ordinary id.
 *   topk_w    f32  [M, topk]          routing weight per (token, slot)
 *   out       bf16 [M, D]             fully overwritten
 *   workspace device memory of at least moe_mxfp4_workspace_bytes(...) bytes
 * M = 0 is a valid no-op.
 * ------------------------------------------------------------------------- */
size_t moe_mxfp4_workspace_bytes(int M, int D, int I, int E, int topk);

int moe_mxfp4_forward(const uint16_t* hidden,
                      const uint8_t* w13, const uint8_t* w13_scale,
                      const uint8_t* w2, const uint8_t* w2_scale,
                      const int32_t* topk_ids, const float* topk_w,
                      uint16_t* out,
                      int M, int D, int I, int E, int topk,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Forward that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Same arguments and result as moe_mxfp4_forward without the workspace: the
 * library uses a static device array of MOE_MXFP4_NOALLOC_SCRATCH_BYTES
 * instead (each GPU the library runs on holds its own copy, from the first
 * call on that device until the process ends; nothing is allocated per
 * call, and no kernel relies on its contents from a previous call).
 * A shape whose workspace (moe_mxfp4_workspace_bytes) exceeds that size is
 * refused with MOE_MXFP4_ERR_WORKSPACE before anything is enqueued: the
 * decode and small-batch shapes fit (for example M <= 16 with E = 257,
 * I = 256, or M <= 64 with E = 33, I = 2048 at D = 7168), the prefill shapes
 * do not.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one device (different streams, or different host threads
 * without ordering) race and give undefined results; calls on one stream are
 * ordered and safe.
 * ------------------------------------------------------------------------- */
#define MOE_MXFP4_NOALLOC_SCRATCH_BYTES (32u << 20)

int moe_mxfp4_forward_noalloc(const uint16_t* hidden,
                              const uint8_t* w13, const uint8_t* w13_scale,
                              const uint8_t* w2, const uint8_t* w2_scale,
                              const int32_t* topk_ids, const float* topk_w,
                              uint16_t* out,
                              int M, int D, int I, int E, int topk,
                              hipStream_t stream);

/* The kernel path the forward takes for this shape (0 for an invalid or
 * unsupported shape):
 * DIRECT when M <= 32, topk <= 16, E <= 1024 and block_m is 16; else TILED when
 * block_m is 256; else STREAM.  The choice depends on the shape only. */
int moe_mxfp4_path(int M, int D, int I, int E, int topk);

/* The block_m (rows per expert block of the sorted route list; the row tile
 * of the DIRECT path) the forward uses for this shape, and the capacity
 * (rows) of the sorted route list.  With 32 to 37 routes per expert on
 * average and I <= 512 the forward's 32-row blocks run in pairs of an
 * expert's blocks as 64-row units (the route list itself is the plain
 * 32-row one). */
int moe_mxfp4_block_m(int M, int D, int I, int E, int topk);
int64_t moe_mxfp4_route_capacity(int M, int E, int topk, int block_m);

/* Kernel launches moe_mxfp4_forward enqueues for this shape (0 for an invalid
 * shape or M = 0): DIRECT 2 (stage 1, stage 2); STREAM 4 (route sort with the
 * activation quantization, stage 1, stage 2, slot sum); TILED one more than
 * STREAM (the sorted copy of the activations). */
int moe_mxfp4_launch_count(int M, int D, int I, int E, int topk);

/* ---------------------------------------------------------------------------
 * Single stages, canonical layouts (for tests and for quantizing weights).
 * ------------------------------------------------------------------------- */

/* MXFP4-quantize a bf16 matrix [rows, cols] (cols % 32 == 0) per 32 along a
 * row: codes u8 [rows, cols/2], scales u8 [rows, cols/32] (row-major).
 *
 * Passage: the dynamic activation quantization of kernelindex.com
 * amd-moe-mxfp4 submission 754773 (`custom_kernel`, FP4 branch: the hidden
 * states are quantized per 32 elements to E2M1 codes with one e8m0 scale
 * before the gate_up GEMM, "per_1x32"), in the format its weights use (two
 * codes per byte, low nibble first, as submission 723815's `_dequant` reads
 * them).  The page imports that quantizer without showing its rounding; the
 * rule here is the OCP MX v1.0 one stated at the top of this header.  The
 * forward runs this same quantizer inside its prologue; this entry point
 * exposes it alone (tests; quantizing float weights).
 * Arguments: x bf16 device [rows, cols], 16-byte aligned; codes and scales
 * device, caller-owned, codes 4-byte aligned.  rows = 0 is a no-op.
 * Errors: INVALID_ARG for rows < 0, cols <= 0 or not a multiple of 32, a null
 * or misaligned pointer; UNSUPPORTED off gfx950; ERR_HIP if the launch fails. */
int moe_mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* Route sort alone: expert-sorted, block_m-padded route lists.
 *
 * Passage: the sorting workspace of kernelindex.com amd-moe-mxfp4 submission
 * 754773 (sorted token ids, sorted routing weights, one expert id per block
 * of block_m rows and a num_valid pair, sized for M*topk + E*block_m - topk
 * rows, each expert's segment padded to a multiple of block_m, filled by
 * aiter's `moe_sorting_fwd` before stage 1), and the routing kernels of
 * submission 723815 (`kernel_count_tokens`: a histogram of the expert ids,
 * skipping ids outside [0, E); `kernel_prefix_sum`: an exclusive scan;
 * `kernel_scatter_tokens`: each route into its expert's segment).  The
 * forward runs the same sort in its prologue on the sorted paths; this entry
 * point exposes it alone (tests).  Unlike the atomics of 723815, the order
 * inside a segment is fixed (ascending route), so the list is deterministic.
 *
 * A route is r = t*topk + s.  Experts appear in ascending order, each expert's routes in
 * ascending r, padded with the id M*topk (weight 0) to a multiple of block_m.
 *   sorted_route i32 [cap], sorted_w f32 [cap], block_expert i32 [cap/block_m]
 *   (-1 past the last used block), num_valid i32 [2] = {padded rows, valid
 *   routes}; cap = moe_mxfp4_route_capacity(M, E, topk, block_m).
 * block_m must be 16, 32, 64, 128 or 256.
 * Arguments: topk_ids i32 / topk_w f32 device [M, topk]; outputs device,
 * caller-owned, 4-byte aligned, sized from moe_mxfp4_route_capacity.
 * Errors: INVALID_ARG for a bad M / E / topk / block_m or a null or
 * misaligned pointer; UNSUPPORTED for E > 1024 or M*topk > 2^24 and off
 * gfx950; ERR_HIP if the launch fails. */
int moe_mxfp4_route(const int32_t* topk_ids, const float* topk_w,
                    int M, int E, int topk, int block_m,
                    int32_t* sorted_route, float* sorted_w,
                    int32_t* block_expert, int32_t* num_valid,
                    hipStream_t stream);

/* Forward that also exports its intermediates (any pointer may be NULL):
 *   sorted_route i32 [cap], num_valid i32 [2]      the row -> route map it used
 *   h            bf16 [cap, I]  silu(gate)*up per row, before requant
 *   a2_codes     u8   [cap, I/2], a2_scales u8 [cap, I/32]  its MXFP4 form
 * On the sorted paths the rows are the sorted route list (as moe_mxfp4_route
 * with the block_m of moe_mxfp4_block_m); on the DIRECT path row r is route
 * r (sorted_route[r] = r, or M*topk for an invalid id; num_valid = {M*topk,
 * valid routes}).  Rows of padding and of invalid routes are unspecified.
 * cap = moe_mxfp4_route_capacity(M, E, topk, block_m) >= M*topk. */
int moe_mxfp4_forward_debug(const uint16_t* hidden,
                            const uint8_t* w13, const uint8_t* w13_scale,
                            const uint8_t* w2, const uint8_t* w2_scale,
                            const int32_t* topk_ids, const float* topk_w,
                            uint16_t* out,
                            int M, int D, int I, int E, int topk,
                            void* workspace, size_t workspace_bytes,
                            int32_t* sorted_route, int32_t* num_valid,
                            uint16_t* h, uint8_t* a2_codes, uint8_t* a2_scales,
                            hipStream_t stream);

/* Forward that times its own kernels, for benchmarks.
 *
 * kernel_events (array of 8, entries may be NULL, or NULL): caller-created
 * HIP events attached to the dispatches of the forward's launches
 * (hipExtLaunchKernel); kernel_events[2*i] / [2*i+1] = start / stop of
 * launch i:
 *   0  prologue (route sort + activation quant; on the TILED path also the
 *      sorted copy of the activations: start on the first kernel, stop on
 *      the second)
 *   1  stage 1 (gate_up GEMM + SwiGLU + MXFP4 requant; on the DIRECT path
 *      also the route scan and the activation quant)
 *   2  stage 2 (down GEMM x routing weight; on the DIRECT path also the
 *      per-token sum)
 *   3  per-token sum over slots (sorted paths)
 * Events of launches a path does not make are not recorded.  The runtime
 * puts a marker in front of each launch that carries events, which delays
 * that kernel's start by a few microseconds; the spans below have no such
 * effect.
 *
 * stage1_clock (device pointer to 2 * moe_mxfp4_stage1_workgroups(...)
 * uint64, 8-byte aligned, or NULL): stage-1 workgroup w stores its start in
 * [2w] and, when all its waves are done, its end in [2w+1], in ticks of the
 * device's constant-rate clock (moe_mxfp4_wall_clock_khz); the kernel's span
 * is the smallest start to the largest end.  Every workgroup writes both.
 *
 * The caller reads events and spans after synchronizing. */
int moe_mxfp4_forward_profiled(const uint16_t* hidden,
                               const uint8_t* w13, const uint8_t* w13_scale,
                               const uint8_t* w2, const uint8_t* w2_scale,
                               const int32_t* topk_ids, const float* topk_w,
                               uint16_t* out,
                               int M, int D, int I, int E, int topk,
                               void* workspace, size_t workspace_bytes,
                               hipEvent_t* kernel_events, uint64_t* stage1_clock,
                               hipStream_t stream);

/* Frequency (kHz) of the clock of stage1_clock records on the current
 * device; 0 on error. */
int moe_mxfp4_wall_clock_khz(void);

/* Measurement aid, not part of the forward: the rate the gfx950 block-scaled
 * FP4 MFMA (both operands E2M1) sustains on register operands with no memory
 * traffic, the practical ceiling of the LDS-tiled GEMMs.  flags: bit 0 set,
 * operands with random bits, else a single set bit per 32-bit word; bit 1
 * set, v_mfma_scale_f32_16x16x128_f8f6f4 (8 independent MFMAs per wave and
 * iteration), else v_mfma_scale_f32_32x32x64_f8f6f4 (4); other bits must be
 * clear.  Two workgroups of four waves per CU run `iters` iterations per
 * wave (1 <= iters <= 2^24) after a shorter settling launch; the call blocks
 * until both have run on `stream`.  Outputs (host pointers): *tflops over
 * the measured launch (events), *shader_mhz the waves' mean shader clock
 * (cycle counter against the constant-rate real-time clock), *per_clock_frac
 * the rate over the FP4 peak at that clock (one 32x32x64 MFMA per 32 cycles
 * per SIMD).  Allocates and frees its own record buffers.  Returns OK,
 * INVALID_ARG (unknown flag bits, iters out of range or a null output),
 * UNSUPPORTED (not gfx950) or HIP. */
int moe_mxfp4_mfma_probe(int flags, int iters, double* tflops, double* shader_mhz,
                         double* per_clock_frac, hipStream_t stream);

/* Debug check of one block-scaled FP4 MFMA instruction, the building block of
 * every GEMM here.  The MXFP4 product it computes is the one kernelindex
 * submission 754773's FP4 branch (`custom_kernel`) runs on both GEMM inputs:
 * E2M1 codes with one e8m0 scale per 32 elements.  The value of a code times
 * 2^(scale-127) is the decode of submission 723815's `_dequant`.
 * rows 16: v_mfma_scale_f32_16x16x128_f8f6f4 on 16 x 128 operands; rows 32:
 * v_mfma_scale_f32_32x32x64_f8f6f4 on 32 x 64.  a, b: device, row-major
 * [rows][K/2] code bytes (element 2j in the low nibble), 16-byte aligned;
 * a_scales, b_scales: device [rows][K/32] e8m0 bytes; out: device fp32
 * [rows][rows], out[i][j] = sum_k A[i][k] * B[j][k], accumulated by the
 * instruction.  Each scale reaches the instruction in byte `sel` (0-3) of its
 * 32-bit word, the other bytes 0xFF (NaN), so a wrong byte select yields NaN.
 * One wave on `stream`; no allocation, stream-ordered.  Returns OK,
 * INVALID_ARG (rows not 16 or 32, sel outside 0-3, a null or misaligned
 * pointer), UNSUPPORTED (not gfx950) or HIP. */
int moe_mxfp4_debug_mfma(int rows, int sel, const uint8_t* a, const uint8_t* a_scales,
                         const uint8_t* b, const uint8_t* b_scales, float* out,
                         hipStream_t stream);

/* Number of workgroups of the stage-1 launch for this shape (0 for an
 * invalid shape or M = 0). */
int64_t moe_mxfp4_stage1_workgroups(int M, int D, int I, int E, int topk);

/* ---------------------------------------------------------------------------
 * A16W4 forward: bf16 activations, MXFP4 weights.
 *
 * The variant that kernelindex.com amd-moe-mxfp4 submission 754773 takes for
 * its 16-token shapes (`custom_kernel`, the branch taken when the shape's
 * ksplit is above 1): neither the activations nor the SwiGLU output are
 * quantized, so
 *
 * out[t, :] = bf16( sum_{s < topk, 0 <= e < E} topk_w[t, s] *
 *                   W2[e] . bf16( silu(Wg[e] . hidden[t]) * (Wu[e] . hidden[t]) ) )
 *
 * with each weight element widened to bf16 exactly (e2m1 value x 2^(s-127);
 * a magnitude past the bf16 range, possible only for scale bytes >= 253,
 * becomes +-inf), bf16 x bf16 products accumulated in fp32, h rounded to
 * bf16 once, and the per-token sum in fp32 over the experts in descending
 * id order, rounded to bf16 once.  Arguments, layouts, ownership, id
 * semantics and error behaviour are those of moe_mxfp4_forward (the same
 * prepared weights); the workspace size is moe_mxfp4_a16w4_workspace_bytes.
 *
 * Few tokens only: M <= 32, topk <= 16, M * topk <= 1024, E <= 1024, else
 * MOE_MXFP4_ERR_UNSUPPORTED (and moe_mxfp4_a16w4_workspace_bytes returns 0).
 * Two launches: stage 1 (route scan, gate_up GEMM + SwiGLU, h stored bf16
 * per route) and stage 2 (down GEMM x routing weight + per-token sum).
 * ------------------------------------------------------------------------- */
size_t moe_mxfp4_a16w4_workspace_bytes(int M, int D, int I, int E, int topk);

int moe_mxfp4_forward_a16w4(const uint16_t* hidden,
                            const uint8_t* w13, const uint8_t* w13_scale,
                            const uint8_t* w2, const uint8_t* w2_scale,
                            const int32_t* topk_ids, const float* topk_w,
                            uint16_t* out,
                            int M, int D, int I, int E, int topk,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* moe_mxfp4_forward_a16w4 with exports (any of them may be NULL):
 *   h             bf16 [M*topk, I]: silu(gate)*up of route r = t*topk + s in
 *                 row r (rows of invalid ids unspecified), 16-byte aligned
 *   kernel_events as in moe_mxfp4_forward_profiled (launches 1 and 2 only)
 *   stage1_clock  as in moe_mxfp4_forward_profiled, for the
 *                 (I/64) * min(E, M*topk) stage-1 workgroups of this path:
 *                 2 * (I/64) * min(E, M*topk) uint64, 8-byte aligned */
int moe_mxfp4_forward_a16w4_debug(const uint16_t* hidden,
                                  const uint8_t* w13, const uint8_t* w13_scale,
                                  const uint8_t* w2, const uint8_t* w2_scale,
                                  const int32_t* topk_ids, const float* topk_w,
                                  uint16_t* out,
                                  int M, int D, int I, int E, int topk,
                                  void* workspace, size_t workspace_bytes,
                                  uint16_t* h, hipEvent_t* kernel_events,
                                  uint64_t* stage1_clock, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Persistent forward: the route-indexed (few-token) forward in ONE launch.
 *
 * Passage: the b12x CuTeDSL W4A16 fused MoE kernel (`W4A16FusedMoeKernel.kernel`)
 * runs FC1 and FC2 in one persistent launch separated by a grid barrier
 * (`_grid_barrier`: an arrival count and a sense word in a caller buffer),
 * with the top-k sum folded into the FC2 epilogue for small-M decode
 * ("TC-decode").  Here: one launch of as many 256-thread workgroups as the
 * CUs hold at once; each runs stage-1 units (route scan, MXFP4 activation
 * quant, gate_up GEMM, SwiGLU, requant of h per route), then builds its
 * stage-2 tables from the routing and issues its first down-projection weight
 * loads, then waits at a grid barrier, then computes 16-column output slices
 * for all tokens with the per-token sum in fp32.  Result: the same operation
 * as moe_mxfp4_forward (same arguments, prepared weights, id semantics and
 * error behaviour; per-token sum over experts in descending id order, in
 * fp32, then one bf16 rounding; deterministic).
 *
 * Shapes: those of the A16W4 forward (M <= 32, topk <= 16, M*topk <= 1024,
 * E <= 1024); any other returns MOE_MXFP4_ERR_UNSUPPORTED and
 * moe_mxfp4_persistent_workspace_bytes returns 0 for it.
 *
 * Workspace: moe_mxfp4_persistent_workspace_bytes(...) bytes, 256-byte
 * aligned.  Its first 2048 bytes hold the barrier's words: they must be zero
 * before the first call, which moe_mxfp4_workspace_init arranges (enqueued
 * on `stream`; once per workspace), and every completed call leaves them
 * as it found them except the generation word (the uint32 at byte offset
 * 0), which counts the calls.  The barrier needs every workgroup resident at once; each wait
 * is bounded (50 ms of the device's constant-rate clock).  If a wait times
 * out (another kernel holding CUs), the waiting workgroups fill the output
 * slices they own with NaN, the uint32 at byte offset 4 of the workspace
 * becomes nonzero, the kernel still exits, and the workspace must be
 * initialized again before its next use.  Concurrent calls need different
 * workspaces.
 * ------------------------------------------------------------------------- */
size_t moe_mxfp4_persistent_workspace_bytes(int M, int D, int I, int E, int topk);

/* Fills a workspace with zeros (one kernel on `stream`, plain stores, no
 * memset, so it may be captured in a graph): the set-up the persistent
 * and split-K forwards need once per workspace (the persistent one again
 * after a timed-out call).
 * workspace_bytes must be a multiple of 256 (every workspace size the
 * library reports is).  INVALID_ARG for a null or misaligned pointer or a
 * bad size. */
int moe_mxfp4_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workgroups of the persistent launch for M tokens on the current device
 * (its per-CU occupancy times its CUs; 0 for M outside 1..32 or no usable
 * device): the size of its clock array below is twice this. */
int64_t moe_mxfp4_persistent_workgroups(int M);

int moe_mxfp4_forward_persistent(const uint16_t* hidden,
                                 const uint8_t* w13, const uint8_t* w13_scale,
                                 const uint8_t* w2, const uint8_t* w2_scale,
                                 const int32_t* topk_ids, const float* topk_w,
                                 uint16_t* out,
                                 int M, int D, int I, int E, int topk,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* moe_mxfp4_forward_persistent with exports (each may be NULL):
 *   h         bf16 [M*topk, I], a2_codes u8 [M*topk, I/2], a2_scales u8
 *             [M*topk, I/32]: silu(gate)*up and its MXFP4 form by route
 *             (rows of invalid ids unspecified), 16-byte aligned;
 *   kernel_events  as in moe_mxfp4_forward_profiled; the single launch is
 *             launch 1 (entries 2 and 3);
 *   clock     device uint64 [2 * moe_mxfp4_persistent_workgroups(M)],
 *             8-byte aligned: each workgroup's start and end on the
 *             constant-rate clock (moe_mxfp4_wall_clock_khz). */
int moe_mxfp4_forward_persistent_debug(const uint16_t* hidden,
                                       const uint8_t* w13, const uint8_t* w13_scale,
                                       const uint8_t* w2, const uint8_t* w2_scale,
                                       const int32_t* topk_ids, const float* topk_w,
                                       uint16_t* out,
                                       int M, int D, int I, int E, int topk,
                                       void* workspace, size_t workspace_bytes,
                                       uint16_t* h, uint8_t* a2_codes, uint8_t* a2_scales,
                                       hipEvent_t* kernel_events, uint64_t* clock,
                                       hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Split-K forward: the route-indexed (few-token) forward with stage 1's
 * contraction over D split across two workgroups per unit.
 *
 * Passage: submission 754773's per-shape override table (`_flower_shape_overrides`)
 * gives every 16-token shape ksplit = 2, and the b12x CuTeDSL W4A16 kernel
 * splits its persistent GEMM's K across CTAs (`_run_persistent_gemm`) and
 * merges the fp32 partial tiles under a per-tile lock (`_finish_tile`).
 * Here each stage-1 unit (expert, pair of 64-row gate_up groups) runs on two
 * workgroups, each over half of D; each writes its fp32 sums of gate and up
 * per route, and the second to finish adds the two halves in part order
 * (deterministic), applies SiLU(gate) * up and the MXFP4 requant.  Stage 2 is
 * the default forward's.  Same operation, arguments, limits (those of the
 * A16W4 forward) and error behaviour as moe_mxfp4_forward_persistent, with
 * this variant's own workspace size.
 *
 * Workspace: moe_mxfp4_splitk_workspace_bytes(...) bytes, 256-byte aligned,
 * zero before its first use (moe_mxfp4_workspace_init, once): its first
 * words count the finished parts of each unit and every call leaves them at
 * zero again.  Concurrent calls need different workspaces.
 * ------------------------------------------------------------------------- */
size_t moe_mxfp4_splitk_workspace_bytes(int M, int D, int I, int E, int topk);

int moe_mxfp4_forward_splitk(const uint16_t* hidden,
                             const uint8_t* w13, const uint8_t* w13_scale,
                             const uint8_t* w2, const uint8_t* w2_scale,
                             const int32_t* topk_ids, const float* topk_w,
                             uint16_t* out,
                             int M, int D, int I, int E, int topk,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* moe_mxfp4_forward_splitk with exports (each may be NULL): h, a2_codes,
 * a2_scales by route as in moe_mxfp4_forward_persistent_debug;
 * kernel_events as in moe_mxfp4_forward_profiled (launches 1 and 2);
 * stage1_clock: device uint64 [2 * 2 * (I/64) * min(E, M*topk)], 8-byte
 * aligned, each stage-1 workgroup's start and end. */
int moe_mxfp4_forward_splitk_debug(const uint16_t* hidden,
                                   const uint8_t* w13, const uint8_t* w13_scale,
                                   const uint8_t* w2, const uint8_t* w2_scale,
                                   const int32_t* topk_ids, const float* topk_w,
                                   uint16_t* out,
                                   int M, int D, int I, int E, int topk,
                                   void* workspace, size_t workspace_bytes,
                                   uint16_t* h, uint8_t* a2_codes, uint8_t* a2_scales,
                                   hipEvent_t* kernel_events, uint64_t* stage1_clock,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
