// C ABI of the fused MXFP4 MoE forward (declared in include/moe_mxfp4.h):
// host-side validation, workspace carving, the choice of path and block_m,
// and the launch sequence, all asynchronous on the caller's stream with no
// host synchronization (grids are sized for the worst-case route list;
// blocks past the real one exit):
//   route-indexed path (few tokens): stage 1 (own route scan + activation
//     quant) -> stage 2 (with the per-token sum over slots);
//   sorted paths: prologue (route sort + activation quant) [-> sorted copy of
//     the activations for the tiled kernels] -> stage 1 -> stage 2 -> slot
//     reduction;
//   A16W4 (bf16 activations, no quantization; few tokens only): the two
//     route-indexed kernels in their bf16 mode.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>

#include "moe_kernels.h"
#include "probe.h"
#include "moe_mxfp4.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxTopk = 32;
constexpr int64_t kMaxRoutes = int64_t(1) << 24;

std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<uintptr_t> g_scratch[kMaxDevices];  // device address of `scratch` per device
std::atomic<int> g_clock_khz[kMaxDevices];      // constant-rate clock of each device
// Longest wait of the persistent forward's grid barrier before it gives up,
// and the bytes its words take at the start of that forward's workspace.
constexpr uint64_t kBarrierTimeoutMs = 50;
constexpr size_t kBarrierBytes = 2048;

}  // namespace

// The workspace of moe_mxfp4_forward_noalloc, for callers that cannot
// allocate.  Every device the library runs on holds its own copy of this
// array (the module is loaded per device) until the process ends.  In host
// code the name `scratch` is only a host-side stand-in: its device address
// comes from hipGetSymbolAddress, taken once per device in device_check
// (with that device current) and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[MOE_MXFP4_NOALLOC_SCRATCH_BYTES];

namespace {

// Checks that the current device is gfx950; returns its CU count in *n_cu
// and, when asked, the device address of its `scratch` array.  The first call
// on a device also lifts the kernels' LDS limits and takes that address.
int device_check(int* n_cu, uint8_t** scratch_out = nullptr, int* clock_khz = nullptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_MXFP4_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_MXFP4_ERR_UNSUPPORTED;
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_MXFP4_ERR_HIP;
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_cu_count[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        if (st == 1) {
            if (moe::route_allow_lds(int(moe::route_lds_bytes(kMaxE))) != hipSuccess ||
                moe::tile_allow_lds() != hipSuccess || moe::direct_allow_lds() != hipSuccess ||
                moe::fused_allow_lds() != hipSuccess)
                return MOE_MXFP4_ERR_HIP;
            int khz = 0;
            if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
                return MOE_MXFP4_ERR_HIP;
            g_clock_khz[dev].store(khz, std::memory_order_relaxed);
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return MOE_MXFP4_ERR_HIP;
            g_scratch[dev].store(reinterpret_cast<uintptr_t>(p), std::memory_order_relaxed);
        }
        g_arch_state[dev].store(st, std::memory_order_release);
    }
    if (st != 1) return MOE_MXFP4_ERR_UNSUPPORTED;
    *n_cu = g_cu_count[dev].load(std::memory_order_relaxed);
    if (clock_khz) *clock_khz = g_clock_khz[dev].load(std::memory_order_relaxed);
    if (scratch_out)
        *scratch_out = reinterpret_cast<uint8_t*>(g_scratch[dev].load(std::memory_order_relaxed));
    return MOE_MXFP4_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool dims_ok(int D, int I)
{
    return D >= 256 && I >= 256 && D <= 65536 && I <= 65536 && D % 256 == 0 && I % 256 == 0;
}

int64_t route_capacity(int M, int E, int topk, int bm)
{
    const int64_t R = int64_t(M) * topk;
    if (R <= 0) return 0;
    const int64_t cap = R + (E < R ? E : R) * int64_t(bm - 1);
    return (cap + bm - 1) / bm * bm;
}

// Rows per expert block.  Few routes per expert (decode, E=257): 16-row
// blocks waste the least MFMA work on padding; with tens to thousands of
// routes per expert, larger blocks read each expert's weights fewer times.
// From 64 routes per expert on average the LDS-tiled kernels win although
// their 256-row blocks are then partly padding (measured at D=7168: M=512,
// E=33, I=2048 506 -> 280 us; I=512 172 -> 131 us; M=256, E=33, I=2048
// 326 -> 260 us); at 32-64 they lose (M=128, E=33: 91 -> 107 us; M=1024,
// E=257 Zipf: 255 -> 431 us).
int choose_block_m(int M, int I, int E, int topk)
{
    const double avg = double(M) * topk / double(E);
    if (avg < 8.0) return 16;
    if (avg < 32.0) return 32;
    if (avg < 37.0 && I <= 512) return 32;   // paired 32-row blocks (pair_blocks)
    if (avg < 64.0) return 64;
    return 256;       // LDS-tiled kernels (gemm_tile.hip)
}

// 32-row blocks whose pairs run as 64-row units (the streaming kernels'
// paired_block rule): an expert with 33 to 128 routes reads its weights once
// per pair instead of once per block, while a Zipf-hot expert keeps 32-row
// units, which spread it over more workgroups.  A pair's two workgroups split
// the 64-row unit by columns, which doubles the activation reads per weight
// byte; that pays where a block has few column units (I <= 512) and the
// experts' routes cluster around 32-37.  Measured at D=7168 against 64-row
// blocks: M=1024, E=257, I=256 Zipf 248.5 -> 235.2 us, uniform 233.4 -> 229.7;
// M=300, E=80, I=256 114.0 -> 104.2; M=128, E=33, I=512 79.2 -> 77.7; M=256,
// E=65, I=512 129.2 -> 128.6.  It loses at 38.5 routes per expert (M=1100,
// E=257, I=256: 237.7 -> 242.9), at 43.6 (M=160, E=33, I=512: 84.2 -> 86.4),
// at 59.5 (M=1700, E=257, I=256: 284 -> 318) and at I=2048 (M=140, E=33: 184
// -> 208 us; M=64, E=33, unpaired 32-row blocks: 146.1 -> 149.8).
bool pair_blocks(int M, int I, int E, int topk)
{
    const double avg = double(M) * topk / double(E);
    return choose_block_m(M, I, E, topk) == 32 && avg >= 32.0;
}

// Few tokens with few routes per expert: the route-indexed kernels, which
// need no route sort (a single-workgroup sort costs more than their whole
// bookkeeping); otherwise the expert-sorted kernels.
int choose_path(int M, int I, int E, int topk)
{
    const int64_t R = int64_t(M) * topk;
    if (M <= moe::kDirectMaxTokens && topk <= moe::kMaxTopkDirect && R <= moe::kDirectMaxRoutes &&
        E <= moe::kDirectMaxE && choose_block_m(M, I, E, topk) == 16)
        return MOE_MXFP4_PATH_DIRECT;
    return choose_block_m(M, I, E, topk) == 256 ? MOE_MXFP4_PATH_TILED : MOE_MXFP4_PATH_STREAM;
}

struct Layout {
    int path;
    int bm;
    bool pair;          // block_m 32 with paired blocks (pair_blocks)
    int64_t cap, nb;
    size_t sorted_route, sorted_w, block_expert, num_valid, a1q, a1s, a1f, a1fs, a2q, a2s, partial,
        slot_expert, slot_layers, route_of, n_active, block_info, h16, barrier,
        split_ctr, part, total;
};

// Forward variants that share the route-indexed kernels' workspace layout.
enum class Variant { Plain, A16W4, Persistent, SplitK };
constexpr int kSplitParts = 2;     // K parts of a split-K stage-1 unit

// The A16W4 forward runs the route-indexed kernels for any routing within
// their limits.
bool a16w4_shape_ok(int M, int E, int topk)
{
    return M <= moe::kDirectMaxTokens && topk <= moe::kMaxTopkDirect &&
           int64_t(M) * topk <= moe::kDirectMaxRoutes && E <= moe::kDirectMaxE;
}

Layout layout(int M, int D, int I, int E, int topk, Variant v = Variant::Plain)
{
    const bool a16 = v == Variant::A16W4;
    Layout L;
    L.path = v != Variant::Plain ? MOE_MXFP4_PATH_DIRECT : choose_path(M, I, E, topk);
    L.bm = choose_block_m(M, I, E, topk);
    L.pair = L.bm == 32 && pair_blocks(M, I, E, topk);
    L.cap = route_capacity(M, E, topk, L.bm);
    L.nb = L.cap / L.bm;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    L.slot_expert = L.slot_layers = L.route_of = L.n_active = L.block_info = 0;
    L.h16 = L.barrier = L.split_ctr = L.part = 0;
    // the persistent forward's barrier words and the split-K counters come
    // first (offset 0)
    if (v == Variant::Persistent) L.barrier = take(kBarrierBytes);
    if (v == Variant::SplitK)
        L.split_ctr = take(sizeof(uint32_t) * size_t(moe::direct_slots(M, E, topk)) *
                           size_t(moe::direct_stage1_x(I)));
    if (L.path == MOE_MXFP4_PATH_DIRECT) {
        // rows indexed by route: a2 codes and scales row-major (A16W4: h in
        // bf16); the expert slots with their token -> route tables
        const size_t R = size_t(M) * topk;
        const size_t slots = size_t(moe::direct_slots(M, E, topk));
        L.sorted_route = L.sorted_w = L.block_expert = L.num_valid = L.a1q = L.a1s = 0;
        L.a1f = L.a1fs = L.partial = L.a2q = L.a2s = 0;
        if (a16) {
            L.h16 = take(R * I * sizeof(uint16_t));
        } else {
            L.a2q = take(R * I / 2);
            L.a2s = take(R * I / 32);
        }
        L.slot_expert = take(sizeof(int32_t) * slots);
        L.slot_layers = take(sizeof(int32_t) * slots);
        L.route_of = take(sizeof(int32_t) * size_t(topk) * slots * size_t(M));
        L.n_active = take(sizeof(int32_t));
        if (v == Variant::SplitK) L.part = take(sizeof(float) * size_t(kSplitParts) * R * 2 * size_t(I));
        L.total = off;
        return L;
    }
    L.sorted_route = take(sizeof(int32_t) * size_t(L.cap));
    L.sorted_w = take(sizeof(float) * size_t(L.cap));
    L.block_expert = take(sizeof(int32_t) * size_t(L.nb));
    L.num_valid = take(sizeof(int32_t) * 4);
    L.block_info = take(sizeof(int32_t) * 4 * size_t(L.nb));
    L.a1q = take(size_t(M) * D / 2);
    L.a1s = take(size_t(M) * D / 32);
    // sorted fragment-layout copy of a1, only for the tiled kernels
    const bool tile = L.bm == 256;
    L.a1f = take(tile ? size_t(L.cap) * D / 2 : 0);
    L.a1fs = take(tile ? size_t(L.cap) * D / 32 : 0);
    L.a2q = take(size_t(L.cap) * I / 2);
    L.a2s = take(size_t(L.cap) * I / 32);
    L.partial = take(sizeof(uint16_t) * size_t(M) * topk * D);
    L.total = off;
    return L;
}

// The LDS-tiled kernels address one expert's weights and the sorted
// operands' K-major scale words with 32-bit per-lane offsets (gemm_tile.hip):
// an expert's gate_up codes (I*D bytes) must stay below 2^31, and the scale
// words of all K tiles (K/128 tiles x cap rows x 4 bytes, K = D in stage 1
// and I in stage 2) below 2^32.
bool tiled_offsets_ok(int M, int D, int I, int E, int topk)
{
    const int64_t cap = route_capacity(M, E, topk, 256);
    const int64_t kmax = D > I ? D : I;
    return int64_t(I) * D < (int64_t(1) << 31) && kmax / 128 * cap * 4 < (int64_t(1) << 32);
}

int check_shape(int M, int D, int I, int E, int topk)
{
    if (M < 0 || E < 1 || topk < 1 || topk > kMaxTopk || !dims_ok(D, I))
        return MOE_MXFP4_ERR_INVALID_ARG;
    if (E > kMaxE || int64_t(M) * topk > kMaxRoutes) return MOE_MXFP4_ERR_UNSUPPORTED;
    if (choose_path(M, I, E, topk) == MOE_MXFP4_PATH_TILED && !tiled_offsets_ok(M, D, I, E, topk))
        return MOE_MXFP4_ERR_UNSUPPORTED;
    return MOE_MXFP4_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_MXFP4_OK : MOE_MXFP4_ERR_HIP; }

struct DebugOut {
    int32_t* sorted_route;
    int32_t* num_valid;
    uint16_t* h;
    uint8_t* a2_codes;
    uint8_t* a2_scales;
    hipEvent_t* events;     // kernel events: start/stop of launches 0..3 (entries may be null)
    uint64_t* stage1_clock; // device [2 x stage-1 workgroups]: their start/end clocks (may be null)
};

// Events of launch i (0 prologue, 1 stage 1, 2 stage 2, 3 slot reduction),
// attached to the kernels' own dispatches.  The prologue's pair spans its
// two kernels on the tiled path (the stop event goes to the second).
moe::KernelEvents kernel_events(const DebugOut* d, int i)
{
    moe::KernelEvents ev;
    if (d && d->events) {
        ev.start = d->events[2 * i];
        ev.stop = d->events[2 * i + 1];
    }
    return ev;
}

int forward_direct(const uint16_t* hidden, const uint8_t* w13, const uint8_t* w13_scale,
                   const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                   const float* topk_w, uint16_t* out, int M, int D, int I, int E, int topk,
                   uint8_t* ws, const Layout& L, int n_cu, int clock_khz, const DebugOut* dbg,
                   Variant v, hipStream_t stream)
{
    const bool a16 = v == Variant::A16W4;
    moe::DirectArgs a{hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, ws + L.a2q,
                      ws + L.a2s, reinterpret_cast<int32_t*>(ws + L.slot_expert),
                      reinterpret_cast<int32_t*>(ws + L.slot_layers),
                      reinterpret_cast<int32_t*>(ws + L.route_of),
                      reinterpret_cast<int32_t*>(ws + L.n_active), out,
                      dbg ? dbg->h : nullptr, M, D, I, E, topk,
                      dbg ? dbg->stage1_clock : nullptr,
                      a16 ? reinterpret_cast<uint16_t*>(ws + L.h16) : nullptr};
    if (v == Variant::SplitK) {
        a.ks_parts = kSplitParts;
        a.part = reinterpret_cast<float*>(ws + L.part);
        a.split_ctr = reinterpret_cast<uint32_t*>(ws + L.split_ctr);
    }
    hipError_t e;
    if (v == Variant::Persistent) {
        // one launch: stage 1, the grid barrier, stage 2
        e = moe::launch_decode_fused(a, reinterpret_cast<uint32_t*>(ws + L.barrier), n_cu,
                                     uint64_t(clock_khz) * kBarrierTimeoutMs, stream,
                                     kernel_events(dbg, 1));
        if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;
    } else {
        // two launches: no prologue, and the slot sum is part of stage 2
        e = moe::launch_gemm1_direct(a, stream, kernel_events(dbg, 1));
        if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;
        e = moe::launch_gemm2_direct(a, stream, kernel_events(dbg, 2));
        if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;
    }
    if (dbg) {
        const int R = M * topk;
        if ((dbg->sorted_route || dbg->num_valid) &&
            moe::launch_direct_rows(topk_ids, R, E, dbg->sorted_route, dbg->num_valid, stream) !=
                hipSuccess)
            return MOE_MXFP4_ERR_HIP;
        if (!a16 && dbg->a2_codes &&
            hipMemcpyAsync(dbg->a2_codes, a.a2q, size_t(R) * I / 2, hipMemcpyDeviceToDevice,
                           stream) != hipSuccess)
            return MOE_MXFP4_ERR_HIP;
        if (!a16 && dbg->a2_scales &&
            hipMemcpyAsync(dbg->a2_scales, a.a2s, size_t(R) * I / 32, hipMemcpyDeviceToDevice,
                           stream) != hipSuccess)
            return MOE_MXFP4_ERR_HIP;
    }
    return MOE_MXFP4_OK;
}

// noalloc: the workspace is the current device's `scratch` array
// (`workspace` and `workspace_bytes` are ignored).
int forward_impl(const uint16_t* hidden, const uint8_t* w13, const uint8_t* w13_scale,
                 const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                 const float* topk_w, uint16_t* out, int M, int D, int I, int E, int topk,
                 void* workspace, size_t workspace_bytes, const DebugOut* dbg,
                 hipStream_t stream, Variant v = Variant::Plain, bool noalloc = false)
{
    int st = check_shape(M, D, I, E, topk);
    if (st) return st;
    if (v != Variant::Plain && !a16w4_shape_ok(M, E, topk)) return MOE_MXFP4_ERR_UNSUPPORTED;
    if (M == 0) return MOE_MXFP4_OK;
    const void* ptrs[] = {hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out};
    for (const void* p : ptrs)
        if (!p || !aligned(p, 16)) return MOE_MXFP4_ERR_INVALID_ARG;
    if (!noalloc && (!workspace || !aligned(workspace, 256))) return MOE_MXFP4_ERR_INVALID_ARG;
    if (noalloc) workspace_bytes = MOE_MXFP4_NOALLOC_SCRATCH_BYTES;
    const Layout L = layout(M, D, I, E, topk, v);
    if (workspace_bytes < L.total) return MOE_MXFP4_ERR_WORKSPACE;
    int n_cu = 0, clock_khz = 0;
    uint8_t* scratch_ptr = nullptr;
    st = device_check(&n_cu, noalloc ? &scratch_ptr : nullptr, &clock_khz);
    if (st) return st;
    if (noalloc) workspace = scratch_ptr;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (L.path == MOE_MXFP4_PATH_DIRECT)
        return forward_direct(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I,
                              E, topk, ws, L, n_cu, clock_khz, dbg, v, stream);
    int32_t* sorted_route = reinterpret_cast<int32_t*>(ws + L.sorted_route);
    float* sorted_w = reinterpret_cast<float*>(ws + L.sorted_w);
    int32_t* block_expert = reinterpret_cast<int32_t*>(ws + L.block_expert);
    int32_t* num_valid = reinterpret_cast<int32_t*>(ws + L.num_valid);
    int32_t* block_info = reinterpret_cast<int32_t*>(ws + L.block_info);
    uint8_t* a1q = ws + L.a1q;
    uint8_t* a1s = ws + L.a1s;
    uint8_t* a1f = ws + L.a1f;
    uint8_t* a1fs = ws + L.a1fs;
    uint8_t* a2q = ws + L.a2q;
    uint8_t* a2s = ws + L.a2s;
    uint16_t* partial = reinterpret_cast<uint16_t*>(ws + L.partial);
    const int nb = int(L.nb);

    // block_m 256 selects the LDS-tiled kernels (many routes per expert);
    // smaller blocks the weight-streaming kernels.
    const bool tile = L.bm == 256;
    moe::PrologueArgs pa{topk_ids, topk_w, M, topk, E, L.bm, nb, sorted_route, sorted_w,
                         block_expert, num_valid, hidden, D, a1q, a1s,
                         block_info};
    const moe::KernelEvents ev0 = kernel_events(dbg, 0);
    hipError_t e = moe::launch_prologue(pa, n_cu, stream,
                                        tile ? moe::KernelEvents{ev0.start, nullptr} : ev0);
    if (e == hipSuccess && tile)
        e = moe::launch_gather_a1(a1q, a1s, sorted_route, num_valid, M, D, topk, L.cap, a1f, a1fs,
                                  n_cu, stream, moe::KernelEvents{nullptr, ev0.stop});
    if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;

    moe::Gemm1Args g1{a1q, a1s, a1f, a1fs, w13, w13_scale, sorted_route, block_expert, num_valid,
                      a2q, a2s, dbg ? dbg->h : nullptr, M, D, I, topk, L.bm, nb, L.cap,
                      dbg ? dbg->stage1_clock : nullptr, block_info, n_cu, L.pair};
    const moe::KernelEvents ev1 = kernel_events(dbg, 1);
    e = tile ? moe::launch_gemm1_tile(g1, stream, ev1) : moe::launch_gemm1(g1, stream, ev1);
    if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;

    moe::Gemm2Args g2{a2q, a2s, w2, w2_scale, sorted_route, sorted_w, block_expert, num_valid,
                      partial, M, D, I, topk, L.bm, nb, L.cap, block_info, nullptr, n_cu, L.pair};
    const moe::KernelEvents ev2 = kernel_events(dbg, 2);
    e = tile ? moe::launch_gemm2_tile(g2, stream, ev2) : moe::launch_gemm2(g2, stream, ev2);
    if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;
    e = moe::launch_reduce_slots(partial, topk_ids, M, D, E, topk, out, n_cu, stream,
                                 kernel_events(dbg, 3));
    if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;

    if (dbg) {
        if (dbg->sorted_route &&
            hipMemcpyAsync(dbg->sorted_route, sorted_route, sizeof(int32_t) * size_t(L.cap),
                           hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return MOE_MXFP4_ERR_HIP;
        if (dbg->num_valid && hipMemcpyAsync(dbg->num_valid, num_valid, sizeof(int32_t) * 2,
                                             hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return MOE_MXFP4_ERR_HIP;
        if ((dbg->a2_codes || dbg->a2_scales) &&
            moe::launch_a2_to_canonical(a2q, a2s, L.cap, I, dbg->a2_codes, dbg->a2_scales,
                                        stream) != hipSuccess)
            return MOE_MXFP4_ERR_HIP;
    }
    return MOE_MXFP4_OK;
}

}  // namespace

MOE_API const char* moe_mxfp4_status_string(int status)
{
    switch (status) {
    case MOE_MXFP4_OK: return "ok";
    case MOE_MXFP4_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer or bad size)";
    case MOE_MXFP4_ERR_UNSUPPORTED: return "unsupported (device is not gfx950 or shape exceeds limits)";
    case MOE_MXFP4_ERR_WORKSPACE: return "workspace too small";
    case MOE_MXFP4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

MOE_API int moe_mxfp4_block_m(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk)) return 0;
    return choose_block_m(M, I, E, topk);
}

MOE_API int moe_mxfp4_launch_count(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk) || M == 0) return 0;
    const int path = choose_path(M, I, E, topk);
    if (path == MOE_MXFP4_PATH_DIRECT) return 2;
    // prologue (sort + quantization), the tiled path's sorted activation
    // copy, stage 1, stage 2, the slot sum
    return 1 + (path == MOE_MXFP4_PATH_TILED ? 1 : 0) + 3;
}

MOE_API int64_t moe_mxfp4_stage1_workgroups(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk) || M == 0) return 0;
    const Layout L = layout(M, D, I, E, topk);
    if (L.path == MOE_MXFP4_PATH_DIRECT)
        return int64_t(moe::direct_stage1_x(I)) * moe::direct_slots(M, E, topk);
    if (L.path == MOE_MXFP4_PATH_TILED) {
        // the persistent grid the launch takes on the current device
        int dev = 0, n_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n_cu = 0;
        return moe::tile_persistent_grid(2 * I / 256, int(L.nb), n_cu);
    }
    return moe::tile_grid(I / (32 * moe::stream_stage1_groups(L.bm)), int(L.nb));
}

MOE_API int moe_mxfp4_mfma_probe(int flags, int iters, double* tflops, double* shader_mhz,
                                 double* per_clock_frac, hipStream_t stream)
{
    if ((flags & ~3) || iters < 1 || iters > (1 << 24) || !tflops || !shader_mhz || !per_clock_frac)
        return MOE_MXFP4_ERR_INVALID_ARG;
    int n_cu = 0, khz = 0;
    int st = device_check(&n_cu, nullptr, &khz);
    if (st) return st;
    moe::ProbeResult r{};
    if (moe::run_mfma_probe(flags & 1, (flags >> 1) & 1, iters, n_cu, khz, stream, &r) != hipSuccess)
        return MOE_MXFP4_ERR_HIP;
    *tflops = r.tflops;
    *shader_mhz = r.shader_mhz;
    *per_clock_frac = r.per_clock_frac;
    return MOE_MXFP4_OK;
}

MOE_API int moe_mxfp4_debug_mfma(int rows, int sel, const uint8_t* a, const uint8_t* a_scales,
                                 const uint8_t* b, const uint8_t* b_scales, float* out,
                                 hipStream_t stream)
{
    if ((rows != 16 && rows != 32) || sel < 0 || sel > 3 || !a || !a_scales || !b || !b_scales ||
        !out || reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(b) % 16 ||
        reinterpret_cast<uintptr_t>(out) % 4)
        return MOE_MXFP4_ERR_INVALID_ARG;
    int n_cu = 0;
    const int st = device_check(&n_cu, nullptr, nullptr);
    if (st) return st;
    return hip_status(moe::run_mfma_unit(rows, sel, a, a_scales, b, b_scales, out, stream));
}

MOE_API int moe_mxfp4_wall_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return 0;
    return khz;
}

MOE_API int moe_mxfp4_path(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk)) return 0;
    return choose_path(M, I, E, topk);
}

MOE_API int64_t moe_mxfp4_route_capacity(int M, int E, int topk, int block_m)
{
    if (M < 0 || E < 1 || topk < 1 || block_m < 1) return 0;
    return route_capacity(M, E, topk, block_m);
}

MOE_API size_t moe_mxfp4_workspace_bytes(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk)) return 0;
    return layout(M, D, I, E, topk).total;
}

static int prepare_impl(const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2,
                        const uint8_t* w2_scale, int E, int D, int I, uint8_t* w13_out,
                        uint8_t* w13_scale_out, uint8_t* w2_out, uint8_t* w2_scale_out,
                        int inverse, hipStream_t stream)
{
    if (E < 1 || !dims_ok(D, I)) return MOE_MXFP4_ERR_INVALID_ARG;
    if (E > kMaxE) return MOE_MXFP4_ERR_UNSUPPORTED;
    const void* ptrs[] = {w13, w13_scale, w2, w2_scale, w13_out, w13_scale_out, w2_out, w2_scale_out};
    for (const void* p : ptrs)
        if (!p || !aligned(p, 16)) return MOE_MXFP4_ERR_INVALID_ARG;
    if (w13 == w13_out || w2 == w2_out || w13_scale == w13_scale_out || w2_scale == w2_scale_out)
        return MOE_MXFP4_ERR_INVALID_ARG;
    int n_cu = 0;
    int st = device_check(&n_cu);
    if (st) return st;
    hipError_t e = moe::launch_prepare(w13, w13_scale, w13_out, w13_scale_out, E, 2 * I, D, I,
                                       inverse, n_cu, stream);
    if (e != hipSuccess) return MOE_MXFP4_ERR_HIP;
    e = moe::launch_prepare(w2, w2_scale, w2_out, w2_scale_out, E, D, I, 0, inverse, n_cu, stream);
    return hip_status(e);
}

MOE_API int moe_mxfp4_prepare_weights(const uint8_t* w13, const uint8_t* w13_scale,
                                      const uint8_t* w2, const uint8_t* w2_scale, int E, int D,
                                      int I, uint8_t* w13_out, uint8_t* w13_scale_out,
                                      uint8_t* w2_out, uint8_t* w2_scale_out, hipStream_t stream)
{
    return prepare_impl(w13, w13_scale, w2, w2_scale, E, D, I, w13_out, w13_scale_out, w2_out,
                        w2_scale_out, 0, stream);
}

MOE_API int moe_mxfp4_unprepare_weights(const uint8_t* w13p, const uint8_t* w13p_scale,
                                        const uint8_t* w2p, const uint8_t* w2p_scale, int E,
                                        int D, int I, uint8_t* w13_out, uint8_t* w13_scale_out,
                                        uint8_t* w2_out, uint8_t* w2_scale_out,
                                        hipStream_t stream)
{
    return prepare_impl(w13p, w13p_scale, w2p, w2p_scale, E, D, I, w13_out, w13_scale_out, w2_out,
                        w2_scale_out, 1, stream);
}

MOE_API int moe_mxfp4_forward(const uint16_t* hidden, const uint8_t* w13, const uint8_t* w13_scale,
                              const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                              const float* topk_w, uint16_t* out, int M, int D, int I, int E,
                              int topk, void* workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, nullptr, stream);
}

MOE_API int moe_mxfp4_forward_noalloc(const uint16_t* hidden, const uint8_t* w13,
                                      const uint8_t* w13_scale, const uint8_t* w2,
                                      const uint8_t* w2_scale, const int32_t* topk_ids,
                                      const float* topk_w, uint16_t* out, int M, int D, int I,
                                      int E, int topk, hipStream_t stream)
{
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, nullptr, 0, nullptr, stream, Variant::Plain, true);
}

MOE_API int moe_mxfp4_forward_debug(const uint16_t* hidden, const uint8_t* w13,
                                    const uint8_t* w13_scale, const uint8_t* w2,
                                    const uint8_t* w2_scale, const int32_t* topk_ids,
                                    const float* topk_w, uint16_t* out, int M, int D, int I, int E,
                                    int topk, void* workspace, size_t workspace_bytes,
                                    int32_t* sorted_route, int32_t* num_valid, uint16_t* h,
                                    uint8_t* a2_codes, uint8_t* a2_scales, hipStream_t stream)
{
    const void* opt[] = {sorted_route, num_valid, h, a2_codes, a2_scales};
    for (const void* p : opt)
        if (p && !aligned(p, 16)) return MOE_MXFP4_ERR_INVALID_ARG;
    DebugOut d{sorted_route, num_valid, h, a2_codes, a2_scales, nullptr, nullptr};
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, &d, stream);
}

MOE_API int moe_mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream)
{
    if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_MXFP4_ERR_INVALID_ARG;
    if (rows == 0) return MOE_MXFP4_OK;
    if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 4))
        return MOE_MXFP4_ERR_INVALID_ARG;
    int n_cu = 0;
    int st = device_check(&n_cu);
    if (st) return st;
    return hip_status(moe::launch_quant_rows(x, rows, cols, codes, scales, n_cu, stream));
}

MOE_API int moe_mxfp4_route(const int32_t* topk_ids, const float* topk_w, int M, int E, int topk,
                            int block_m, int32_t* sorted_route, float* sorted_w,
                            int32_t* block_expert, int32_t* num_valid, hipStream_t stream)
{
    if (M < 0 || E < 1 || topk < 1 || topk > kMaxTopk) return MOE_MXFP4_ERR_INVALID_ARG;
    if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128 && block_m != 256)
        return MOE_MXFP4_ERR_INVALID_ARG;
    if (E > kMaxE || int64_t(M) * topk > kMaxRoutes) return MOE_MXFP4_ERR_UNSUPPORTED;
    const void* ptrs[] = {topk_ids, topk_w, sorted_route, sorted_w, block_expert, num_valid};
    for (const void* p : ptrs)
        if (!p || !aligned(p, 4)) return MOE_MXFP4_ERR_INVALID_ARG;
    int n_cu = 0;
    int st = device_check(&n_cu);
    if (st) return st;
    const int64_t cap = route_capacity(M, E, topk, block_m);
    return hip_status(moe::launch_route_sort(topk_ids, topk_w, M, topk, E, block_m,
                                             int(cap / block_m), sorted_route, sorted_w,
                                             block_expert, num_valid, stream));
}

MOE_API int moe_mxfp4_forward_profiled(const uint16_t* hidden, const uint8_t* w13,
                                       const uint8_t* w13_scale, const uint8_t* w2,
                                       const uint8_t* w2_scale, const int32_t* topk_ids,
                                       const float* topk_w, uint16_t* out, int M, int D, int I,
                                       int E, int topk, void* workspace, size_t workspace_bytes,
                                       hipEvent_t* kernel_events, uint64_t* stage1_clock,
                                       hipStream_t stream)
{
    if (stage1_clock && !aligned(stage1_clock, 8)) return MOE_MXFP4_ERR_INVALID_ARG;
    DebugOut d{nullptr, nullptr, nullptr, nullptr, nullptr, kernel_events, stage1_clock};
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, &d, stream);
}

MOE_API size_t moe_mxfp4_a16w4_workspace_bytes(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk) || !a16w4_shape_ok(M, E, topk)) return 0;
    return layout(M, D, I, E, topk, Variant::A16W4).total;
}

MOE_API int moe_mxfp4_forward_a16w4(const uint16_t* hidden, const uint8_t* w13,
                                    const uint8_t* w13_scale, const uint8_t* w2,
                                    const uint8_t* w2_scale, const int32_t* topk_ids,
                                    const float* topk_w, uint16_t* out, int M, int D, int I, int E,
                                    int topk, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream)
{
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, nullptr, stream, Variant::A16W4);
}

MOE_API int moe_mxfp4_forward_a16w4_debug(const uint16_t* hidden, const uint8_t* w13,
                                          const uint8_t* w13_scale, const uint8_t* w2,
                                          const uint8_t* w2_scale, const int32_t* topk_ids,
                                          const float* topk_w, uint16_t* out, int M, int D, int I,
                                          int E, int topk, void* workspace,
                                          size_t workspace_bytes, uint16_t* h,
                                          hipEvent_t* kernel_events, uint64_t* stage1_clock,
                                          hipStream_t stream)
{
    if ((h && !aligned(h, 16)) || (stage1_clock && !aligned(stage1_clock, 8)))
        return MOE_MXFP4_ERR_INVALID_ARG;
    DebugOut d{nullptr, nullptr, h, nullptr, nullptr, kernel_events, stage1_clock};
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, &d, stream, Variant::A16W4);
}

MOE_API size_t moe_mxfp4_persistent_workspace_bytes(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk) || !a16w4_shape_ok(M, E, topk)) return 0;
    return layout(M, D, I, E, topk, Variant::Persistent).total;
}

MOE_API int moe_mxfp4_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!workspace || !aligned(workspace, 256) || workspace_bytes % 256 != 0)
        return MOE_MXFP4_ERR_INVALID_ARG;
    if (workspace_bytes == 0) return MOE_MXFP4_OK;
    int n_cu = 0;
    const int st = device_check(&n_cu);
    if (st) return st;
    return hip_status(moe::launch_zero_fill(static_cast<uint8_t*>(workspace), workspace_bytes,
                                            n_cu, stream));
}

MOE_API int64_t moe_mxfp4_persistent_workgroups(int M)
{
    int n_cu = 0;
    if (M < 1 || M > moe::kDirectMaxTokens || device_check(&n_cu)) return 0;
    return moe::fused_grid(M, n_cu);
}

MOE_API int moe_mxfp4_forward_persistent(const uint16_t* hidden, const uint8_t* w13,
                                         const uint8_t* w13_scale, const uint8_t* w2,
                                         const uint8_t* w2_scale, const int32_t* topk_ids,
                                         const float* topk_w, uint16_t* out, int M, int D, int I,
                                         int E, int topk, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream)
{
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, nullptr, stream, Variant::Persistent);
}

MOE_API int moe_mxfp4_forward_persistent_debug(const uint16_t* hidden, const uint8_t* w13,
                                               const uint8_t* w13_scale, const uint8_t* w2,
                                               const uint8_t* w2_scale, const int32_t* topk_ids,
                                               const float* topk_w, uint16_t* out, int M, int D,
                                               int I, int E, int topk, void* workspace,
                                               size_t workspace_bytes, uint16_t* h,
                                               uint8_t* a2_codes, uint8_t* a2_scales,
                                               hipEvent_t* kernel_events, uint64_t* clock,
                                               hipStream_t stream)
{
    const void* opt[] = {h, a2_codes, a2_scales};
    for (const void* p : opt)
        if (p && !aligned(p, 16)) return MOE_MXFP4_ERR_INVALID_ARG;
    if (clock && !aligned(clock, 8)) return MOE_MXFP4_ERR_INVALID_ARG;
    DebugOut d{nullptr, nullptr, h, a2_codes, a2_scales, kernel_events, clock};
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, &d, stream, Variant::Persistent);
}

MOE_API size_t moe_mxfp4_splitk_workspace_bytes(int M, int D, int I, int E, int topk)
{
    if (check_shape(M, D, I, E, topk) || !a16w4_shape_ok(M, E, topk)) return 0;
    return layout(M, D, I, E, topk, Variant::SplitK).total;
}

MOE_API int moe_mxfp4_forward_splitk(const uint16_t* hidden, const uint8_t* w13,
                                     const uint8_t* w13_scale, const uint8_t* w2,
                                     const uint8_t* w2_scale, const int32_t* topk_ids,
                                     const float* topk_w, uint16_t* out, int M, int D, int I, int E,
                                     int topk, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream)
{
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, nullptr, stream, Variant::SplitK);
}

MOE_API int moe_mxfp4_forward_splitk_debug(const uint16_t* hidden, const uint8_t* w13,
                                           const uint8_t* w13_scale, const uint8_t* w2,
                                           const uint8_t* w2_scale, const int32_t* topk_ids,
                                           const float* topk_w, uint16_t* out, int M, int D, int I,
                                           int E, int topk, void* workspace,
                                           size_t workspace_bytes, uint16_t* h, uint8_t* a2_codes,
                                           uint8_t* a2_scales, hipEvent_t* kernel_events,
                                           uint64_t* stage1_clock, hipStream_t stream)
{
    const void* opt[] = {h, a2_codes, a2_scales};
    for (const void* p : opt)
        if (p && !aligned(p, 16)) return MOE_MXFP4_ERR_INVALID_ARG;
    if (stage1_clock && !aligned(stage1_clock, 8)) return MOE_MXFP4_ERR_INVALID_ARG;
    DebugOut d{nullptr, nullptr, h, a2_codes, a2_scales, kernel_events, stage1_clock};
    return forward_impl(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, M, D, I, E,
                        topk, workspace, workspace_bytes, &d, stream, Variant::SplitK);
}
