"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Bit-exact: MXFP4 codes/scales (activation quantizer, fused stage-1 requant),
route lists, weight preparation.  Floating point: the end-to-end tolerance
|gpu - oracle| <= 2e-2 rms + 2^-7 |oracle| on >= 99.9 % of elements, none
beyond 0.1 rms.  Where the debug outputs are at hand, a requant code may sit
one E2M1 grid step from the oracle's only where the GPU h and the oracle h lie
on opposite sides of that rounding midpoint (or the block maxima on opposite
sides of a scale step); then, and only then, the token's bound grows by what
the moved code carries (tests/moe_cases.requant_moves / requant_slack).
Without such a move the strict bound is asserted.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_mxfp4_amd import inputs
from tests.moe_cases import (Case, bf16_to_f64, check_close, covering_tokens, custom_case, log,
                             requant_slack, workload_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding(gpu_device):
    from mixture_experts_mxfp4_amd import binding as b
    return b


# ------------------------------------------------------------- quantizer ---

def _adversarial_rows(cols, rng):
    rows = []
    for scale in (2.0 ** -130, 2.0 ** -125, 2.0 ** -20, 1.0, 2.0 ** 40, 2.0 ** 120):
        x = rng.standard_normal(cols) * scale
        rows.append(x)
        t = np.round(rng.standard_normal(cols) * 8) / 4 * scale      # exact midpoints
        rows.append(t)
    z = np.zeros(cols)
    z[1::3] = -0.0
    rows.append(z)
    sat = np.full(cols, 1.875)
    sat[::2] = -1.75
    rows.append(sat)
    return np.stack(rows)


def _f32_to_bf16_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("rows,cols", [(1, 32), (13, 512), (64, 7168), (257, 2048)])
def test_quantize_bit_exact(binding, rows, cols):
    log(f"quantize rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-30, 30, (rows, 1)))
    if rows >= 13:
        adv = _adversarial_rows(cols, rng)
        x[: adv.shape[0]] = adv[: rows]
    bits = _f32_to_bf16_bits(x)
    codes, scales = binding.moe_mxfp4_quantize(inputs.bits_to_bf16(bits).cuda())
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_rows(bits)
    np.testing.assert_array_equal(scales.cpu().numpy(), os_)
    np.testing.assert_array_equal(codes.cpu().numpy(), oc)


def _domain_blocks():
    """Every finite bf16 value under every reachable scale byte s (0..252), in
    blocks of 32 whose first element fixes the block maximum (and so s):
    the largest bf16 with exponent field s + 2 (2 for s = 0); the other 31
    elements run through every bf16 whose exponent field is <= that, both
    signs.  About 8.4 M elements."""
    blocks = []
    for s in range(0, 253):
        e_max = max(s + 2, 2)
        amax = np.uint16((e_max << 7) | 0x7F)
        mags = np.arange(0, (e_max + 1) << 7, dtype=np.uint32).astype(np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        n = -(-vals.size // 31) * 31
        vals = np.concatenate([vals, np.zeros(n - vals.size, np.uint16)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((vals.shape[0], 1), amax, np.uint16), vals], 1))
    b = np.concatenate(blocks).reshape(-1)
    pad = -(-b.size // 256) * 256 - b.size
    return np.concatenate([b, np.zeros(pad, np.uint16)]).reshape(-1, 256)


def test_quantize_whole_domain_bit_exact(binding):
    """The device quantizer equals the oracle on its whole input domain."""
    bits = _domain_blocks()
    log(f"quantize whole domain: {bits.size} elements")
    codes, scales = binding.moe_mxfp4_quantize(inputs.bits_to_bf16(bits).cuda())
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_rows(bits)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


def test_quantize_weights_of_decode_bit_exact(binding):
    """The product quantizer on the decode workload's full gate_up weight."""
    w = inputs.WORKLOADS["decode"]
    log("quantize decode weights (257 x 512 x 7168)")
    w13f, _ = inputs.make_weights(w.E, w.D, w.I, w.seed, device="cuda")
    flat = w13f.reshape(-1, w.D)
    codes, scales = binding.moe_mxfp4_quantize(flat)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_rows(inputs.bf16_bits(flat))
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


# ----------------------------------------------------------------- route ---

def _route_cases():
    out = []
    for name, w in inputs.WORKLOADS.items():
        out.append((name, w.M, w.E, w.n_routed, w.routing, w.seed))
    return out


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("case", _route_cases(), ids=lambda c: c[0])
def test_route_matches_oracle(binding, case, bm):
    name, M, E, n_routed, routing, seed = case
    log(f"route {name} bm={bm}")
    _, ids, tw = inputs.make_activations(M, 256, E, n_routed, routing, seed)
    got = binding.moe_mxfp4_route(ids.cuda(), tw.cuda(), E, bm)
    torch.cuda.synchronize()
    want = oracle.route(ids.numpy(), tw.numpy(), E, bm)
    n = int(want["num_valid"][0])
    np.testing.assert_array_equal(got["num_valid"].cpu().numpy(), want["num_valid"])
    np.testing.assert_array_equal(got["sorted_route"].cpu().numpy()[:n], want["sorted_route"])
    np.testing.assert_array_equal(got["sorted_w"].cpu().numpy()[:n], want["sorted_w"])
    be = got["block_expert"].cpu().numpy()
    np.testing.assert_array_equal(be[: n // bm], want["block_expert"])
    assert np.all(be[n // bm:] == -1)


@pytest.mark.parametrize("M,E,k,bm", [(1, 1, 1, 16), (5, 3, 4, 16), (300, 7, 5, 32),
                                      (2000, 1024, 8, 16), (513, 64, 32, 64)])
def test_route_edge_cases(binding, M, E, k, bm):
    """Invalid ids (-1, E, large), duplicates within a row, one hot expert."""
    log(f"route edge M={M} E={E} k={k} bm={bm}")
    rng = np.random.default_rng(M + E)
    ids = rng.integers(-2, E + 2, (M, k)).astype(np.int32)
    ids[:, 0] = 0                                   # a hot expert
    if k > 1:
        ids[::3, 1] = ids[::3, 0]                   # duplicates
    ids[::7, -1] = 1 << 20
    tw = rng.random((M, k)).astype(np.float32)
    got = binding.moe_mxfp4_route(torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda(), E, bm)
    torch.cuda.synchronize()
    want = oracle.route(ids, tw, E, bm)
    n = int(want["num_valid"][0])
    np.testing.assert_array_equal(got["num_valid"].cpu().numpy(), want["num_valid"])
    np.testing.assert_array_equal(got["sorted_route"].cpu().numpy()[:n], want["sorted_route"])
    np.testing.assert_array_equal(got["sorted_w"].cpu().numpy()[:n], want["sorted_w"])
    np.testing.assert_array_equal(got["block_expert"].cpu().numpy()[: n // bm],
                                  want["block_expert"])


def _random_route_cases(n=30, seed=7):
    """Seeded route lists: M up to 20,000, E up to 1,024, up to 32 slots, every
    block size; ids uniform, Zipf-skewed or one hot expert, a third with
    invalid (-1, E, large) and repeated ids.  They span the one-wave sort
    (up to 768 routes) and the chunked workgroup sort (1 to ~300 chunks)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 65)) if i % 4 == 0 else int(rng.integers(65, 20001))
        E = int(rng.integers(1, 1025))
        k = int(rng.integers(1, 33))
        bm = int(rng.choice([16, 32, 64, 128, 256]))
        kind = ["uniform", "zipf", "hot"][i % 3]
        out.append((M, E, k, bm, kind, bool(rng.random() < 0.34), 1000 + i))
    return out


@pytest.mark.parametrize("M,E,k,bm,kind,dirty,seed", _random_route_cases())
def test_route_random(binding, M, E, k, bm, kind, dirty, seed):
    """The sorted route list, weights, block experts and counts equal the
    oracle's bit for bit on seeded random routings."""
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        ids = rng.integers(0, E, (M, k))
    elif kind == "zipf":
        ids = (rng.zipf(1.3, (M, k)) - 1) % E
    else:
        ids = np.where(rng.random((M, k)) < 0.7, E // 2, rng.integers(0, E, (M, k)))
    ids = ids.astype(np.int32)
    if dirty:
        if k > 1:
            ids[::3, 1] = ids[::3, 0]
        ids[::5, 0] = -1
        ids[1::7, -1] = E
        ids[2::11, k // 2] = 1 << 30
    tw = rng.random((M, k)).astype(np.float32)
    log(f"route random M={M} E={E} k={k} bm={bm} {kind} dirty={dirty}")
    got = binding.moe_mxfp4_route(torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda(), E, bm)
    torch.cuda.synchronize()
    want = oracle.route(ids, tw, E, bm)
    n = int(want["num_valid"][0])
    np.testing.assert_array_equal(got["num_valid"].cpu().numpy(), want["num_valid"])
    np.testing.assert_array_equal(got["sorted_route"].cpu().numpy()[:n], want["sorted_route"])
    np.testing.assert_array_equal(got["sorted_w"].cpu().numpy()[:n], want["sorted_w"])
    be = got["block_expert"].cpu().numpy()
    np.testing.assert_array_equal(be[: n // bm], want["block_expert"])
    assert np.all(be[n // bm:] == -1)


# --------------------------------------------------------------- prepare ---

def _layout_reference(raw_codes, raw_scales, N, K, gate_up_I):
    """The documented prepared layout, rebuilt with numpy for one expert."""
    rows = np.arange(N)
    if gate_up_I:
        c, q, j = rows // 64, (rows % 64) // 16, rows % 16
        perm = np.where(q < 2, 0, gate_up_I) + c * 32 + (q & 1) * 16 + j
    else:
        perm = rows
    KT = K // 128
    codes = raw_codes[perm]                              # prepared row order [N, K/2]
    # [N/64, 4, 16, KT, 4(k-chunk), 16B] -> [N/64, KT, 4, (k-chunk, 16 rows), 16B]
    t = codes.reshape(N // 64, 4, 16, KT, 4, 16).transpose(0, 3, 1, 4, 2, 5)
    pc = t.reshape(-1)
    sc = raw_scales[perm]                                 # [N, K/32]
    # [N/64, 4(q), 16, KT, 4(k-chunk)] -> [N/64, KT, (k-chunk, 16 rows), q]
    s = sc.reshape(N // 64, 4, 16, KT, 4).transpose(0, 3, 4, 2, 1)
    ps = s.reshape(-1)
    return pc, ps


@pytest.mark.parametrize("E,D,I", [(3, 512, 256), (2, 768, 768), (1, 7168, 2048)])
def test_prepare_layout_and_round_trip(binding, E, D, I):
    log(f"prepare E={E} D={D} I={I}")
    rng = np.random.default_rng(D + I)
    raw = [rng.integers(0, 256, s).astype(np.uint8)
           for s in ((E, 2 * I, D // 2), (E, 2 * I, D // 32), (E, D, I // 2), (E, D, I // 32))]
    dev = [torch.from_numpy(a).cuda() for a in raw]
    prep = binding.moe_mxfp4_prepare_weights(*dev)
    back = binding.moe_mxfp4_unprepare_weights(*prep)
    torch.cuda.synchronize()
    for a, b in zip(raw, back):
        np.testing.assert_array_equal(b.cpu().numpy(), a)
    p = [t.cpu().numpy() for t in prep]
    for e in range(E):
        pc, ps = _layout_reference(raw[0][e], raw[1][e], 2 * I, D, I)
        np.testing.assert_array_equal(p[0][e].reshape(-1), pc)
        np.testing.assert_array_equal(p[1][e].reshape(-1), ps)
        pc, ps = _layout_reference(raw[2][e], raw[3][e], D, I, 0)
        np.testing.assert_array_equal(p[2][e].reshape(-1), pc)
        np.testing.assert_array_equal(p[3][e].reshape(-1), ps)


# --------------------------------------------------------------- forward ---

def _check_intermediates(case, dbg, h_or, tokens=None):
    """The route list the forward used (bit for bit), h per row against the
    oracle's h, and the fused requant bit for bit against the oracle quantizer
    applied to the GPU's own h; h_or is the oracle's h [ntok, topk, I] for
    `tokens` (all tokens when None): only their rows are compared."""
    from mixture_experts_mxfp4_amd import binding
    sr = dbg["sorted_route"].cpu().numpy()
    n = int(dbg["num_valid"].cpu().numpy()[0])
    bm = dbg["block_m"]
    R = case.M * case.topk
    if dbg["path"] == binding.PATH_DIRECT:
        # rows indexed by route: row r = route r, invalid ids -> sentinel R
        ok = (case.ids.reshape(-1) >= 0) & (case.ids.reshape(-1) < case.E)
        np.testing.assert_array_equal(sr[:n], np.where(ok, np.arange(R), R))
        assert n == R and int(dbg["num_valid"].cpu().numpy()[1]) == int(ok.sum())
    else:
        want_route = oracle.route(case.ids, case.tw, case.E, bm)
        np.testing.assert_array_equal(sr[:n], want_route["sorted_route"])
    tok_list = np.arange(case.M) if tokens is None else np.asarray(tokens)
    pos = np.full(case.M, -1, np.int64)
    pos[tok_list] = np.arange(tok_list.size)
    valid = np.nonzero(sr[:n] < R)[0]
    valid = valid[pos[sr[valid] // case.topk] >= 0]
    h_gpu = dbg["h"].cpu().view(torch.int16).numpy().view(np.uint16)[valid]
    r = sr[valid]
    h_ref = h_or[pos[r // case.topk], r % case.topk]
    g, o = bf16_to_f64(h_gpu), bf16_to_f64(h_ref)
    rms = float(np.sqrt(np.mean(o * o)))
    assert np.all(np.abs(g - o) <= 2.0 ** -6 * np.abs(o) + 1e-3 * rms)
    exact = float(np.mean(h_gpu == h_ref))
    log(f"h: {valid.size} rows compared, exact-bits fraction {exact:.4f}")
    assert exact >= 0.95
    codes, scales = oracle.quantize_rows(h_gpu)
    np.testing.assert_array_equal(dbg["a2_scales"].cpu().numpy()[valid], scales)
    np.testing.assert_array_equal(dbg["a2_codes"].cpu().numpy()[valid], codes)
    return valid.size


def _check_forward(case, dbg, what, tokens=None):
    """One oracle run (output and h) over `tokens` (all when None): the
    intermediates, then the output.  Requant codes may differ from the
    oracle's only as tests/moe_cases.requant_moves explains; without any
    such difference the strict tolerance is asserted, with one the output's
    bound grows by what the moved codes carry (requant_slack)."""
    out_or, h_or = case.run_oracle(tokens=tokens, want_h=True)
    _check_intermediates(case, dbg, h_or, tokens)
    slack, moved, total = requant_slack(case, dbg, h_or, tokens)
    log(f"{what}: requant codes moved across a rounding boundary: {moved} of {total}")
    assert moved <= 1e-3 * max(total, 1)
    out = dbg["out"].cpu().view(torch.int16).numpy().view(np.uint16)
    if tokens is not None:
        out = out[tokens]
    return check_close(out, out_or, what, slack=slack)


def test_forward_tiny_full_and_intermediates(binding):
    case = workload_case("tiny")
    _check_forward(case, case.run_gpu(debug=True), "tiny")


# (workload, part, parts): large_prefill's covering tokens are checked in two
# halves so that each test's oracle run stays near a minute
_COVERING = [("decode", 0, 1), ("small_batch", 0, 1), ("prefill", 0, 1),
             ("large_prefill", 0, 2), ("large_prefill", 1, 2)]


_LAST_CASE = {}


def _workload_case_cached(name):
    """The workload's case, kept for the next test when it asks for the same
    one (large_prefill's two halves share one oracle weight quantization)."""
    if name not in _LAST_CASE:
        _LAST_CASE.clear()
        _LAST_CASE[name] = workload_case(name)
    return _LAST_CASE[name]


@pytest.mark.parametrize("name,part,parts", _COVERING,
                         ids=[f"{c[0]}-{c[1]}" for c in _COVERING])
def test_forward_workload_covering(binding, name, part, parts):
    """The full-size workloads, in the launch configuration the benchmark
    times: the plain forward's output equals the debug forward's bit for bit,
    and on tokens whose routes touch every used block of the sorted list (every
    64-row group's first 16-row slice and the slice of its last route; all
    tokens at decode) the route list, h, the requant codes and the output
    match the oracle.  Every other output element must be finite."""
    case = _workload_case_cached(name)
    plain = case.run_gpu().cpu().view(torch.int16).numpy().view(np.uint16)
    dbg = case.run_gpu(debug=True)
    got = dbg["out"].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(plain, got), "debug forward and plain forward differ"
    assert np.all(np.isfinite(bf16_to_f64(plain)))
    toks = covering_tokens(case.ids, case.tw, case.E, dbg["block_m"], must=(0, case.M - 1))
    if name == "small_batch":                       # a few more tokens than the 10 that cover
        rng = np.random.default_rng(11)
        toks = np.union1d(toks, rng.choice(case.M, 16, replace=False))
    toks = np.array_split(toks, parts)[part]
    log(f"{name} part {part + 1}/{parts}: path {binding.PATH_NAMES[dbg['path']]}, block_m "
        f"{dbg['block_m']}, oracle on {toks.size} tokens")
    _check_forward(case, dbg, f"{name} ({toks.size} covering tokens)", tokens=toks)


@pytest.mark.parametrize("name", ["prefill", "large_prefill"])
def test_forward_route_list_long(binding, name):
    """Long route lists are sorted in chunks over several workgroups inside the
    forward; the list the forward used is the oracle's, bit for bit."""
    w = inputs.WORKLOADS[name]
    hidden, ids, tw = inputs.make_activations(w.M, w.D, w.E, w.n_routed, w.routing, w.seed)
    E, D, I = w.E, w.D, w.I
    # weights only need the right shapes here (the route list does not depend on them)
    prep = binding.moe_mxfp4_prepare_weights(
        *[torch.zeros(s, dtype=torch.uint8, device="cuda")
          for s in ((E, 2 * I, D // 2), (E, 2 * I, D // 32), (E, D, I // 2), (E, D, I // 32))])
    dbg = binding.moe_mxfp4_forward_debug(hidden.cuda(), *prep, ids.cuda(), tw.cuda())
    torch.cuda.synchronize()
    want = oracle.route(ids.numpy(), tw.numpy(), E, dbg["block_m"])
    n = int(want["num_valid"][0])
    log(f"{name}: {w.M * w.topk} routes, block_m {dbg['block_m']}, {n} sorted rows")
    np.testing.assert_array_equal(dbg["num_valid"].cpu().numpy(), want["num_valid"])
    np.testing.assert_array_equal(dbg["sorted_route"].cpu().numpy()[:n], want["sorted_route"])


@pytest.mark.parametrize("M,k,E", [
    (3000, 9, 40), (5000, 9, 257), (4100, 9, 5),
    (86, 9, 40),        # 774 routes: just past the one-wave sort's limit, one chunk
    (300, 9, 257),      # 2,700 routes: two chunks
    (456, 9, 40),       # 4,104 routes: three chunks, a last chunk of 8
    (1137, 9, 33),      # every chunk sees at most 8,192 other routes (loaded up front)
    (1138, 9, 33),      # the first chunks see 8,194 (loaded in two batches)
    (5000, 1, 1),       # one expert, one slot per token
])
def test_forward_route_list_chunked_edge_ids(binding, M, k, E):
    """Long lists sorted in chunks over several workgroups, with invalid ids,
    repeated ids within a token and one hot expert: the forward's route list
    is the oracle's, bit for bit."""
    D, I = 256, 256
    rng = np.random.default_rng(M + E)
    ids = rng.integers(-2, E + 2, (M, k)).astype(np.int32)
    ids[:, 0] = 0
    if k > 1:
        ids[::3, 1] = ids[::3, 0]
    ids[::7, -1] = 1 << 20
    tw = rng.random((M, k)).astype(np.float32)
    prep = binding.moe_mxfp4_prepare_weights(
        *[torch.zeros(s, dtype=torch.uint8, device="cuda")
          for s in ((E, 2 * I, D // 2), (E, 2 * I, D // 32), (E, D, I // 2), (E, D, I // 32))])
    hidden = torch.zeros((M, D), dtype=torch.bfloat16, device="cuda")
    dbg = binding.moe_mxfp4_forward_debug(hidden, *prep, torch.from_numpy(ids).cuda(),
                                          torch.from_numpy(tw).cuda())
    torch.cuda.synchronize()
    want = oracle.route(ids, tw, E, dbg["block_m"])
    n = int(want["num_valid"][0])
    log(f"chunked route list M={M} k={k} E={E}: block_m {dbg['block_m']}, {n} sorted rows")
    np.testing.assert_array_equal(dbg["num_valid"].cpu().numpy(), want["num_valid"])
    got = dbg["sorted_route"].cpu().numpy()
    np.testing.assert_array_equal(got[:n], want["sorted_route"])
    assert np.all(got[n:] == M * k)        # rows past the used blocks are padding too
    assert torch.all(dbg["out"].float() == 0)


@pytest.mark.parametrize("high", [False, True])
def test_tiled_workspace_address_bit31(binding, high):
    """The tiled kernels form the scalar address of each tile's record from two
    32-bit halves: a workspace whose address has bit 31 of its low word set
    (or clear) gives the same bits as one from the allocator."""
    M, D, I, E, n_routed, seed = 1400, 512, 256, 5, 2, 25
    case = custom_case(M, D, I, E, n_routed, seed)
    d = case.device_inputs()
    ref = binding.moe_mxfp4_forward(d["hidden"], *d["prepared"], d["ids"], d["tw"])
    n = binding.moe_mxfp4_workspace_bytes(M, D, I, E, case.topk)
    raw = torch.empty(n + (1 << 32) + 256, dtype=torch.uint8, device="cuda")
    base = raw.data_ptr()
    want = (0x80000000 if high else 0) + 0x100
    off = (want - (base & 0xFFFFFFFF)) % (1 << 32)
    ws = raw[off:off + n]
    assert (ws.data_ptr() & 0x80000000 != 0) == high and ws.data_ptr() % 256 == 0
    log(f"tiled forward with workspace at {ws.data_ptr():#x}")
    out = binding.moe_mxfp4_forward(d["hidden"], *d["prepared"], d["ids"], d["tw"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M,D,I,E,n_routed,seed", [
    (1, 512, 256, 9, 2, 21),          # single token (route-indexed path)
    (32, 512, 256, 65, 8, 27),        # route-indexed, shared expert spans two row tiles
    (200, 512, 256, 257, 8, 28),      # sorted streaming path with block_m 16
    (200, 768, 256, 257, 8, 33),      # block_m 16, an odd number of 256-column tiles
    (37, 768, 768, 5, 3, 22),         # ragged M, D and I not multiples of 512
    (130, 1024, 512, 33, 8, 23),      # several blocks per expert (paired 32-row blocks)
    (200, 512, 256, 33, 8, 32),       # 64-row blocks (54.5 routes per expert)
    (3, 256, 256, 2, 1, 24),          # smallest dims
    (1400, 512, 256, 5, 2, 25),       # LDS-tiled path (block_m 256), ragged blocks
    (1000, 768, 512, 3, 1, 26),       # LDS-tiled path, D not a multiple of 512
    (200, 512, 256, 17, 8, 29),       # LDS-tiled path at ~106 routes per expert: blocks half padding
    (1100, 512, 256, 9, 2, 30),       # LDS-tiled, 7 of 9 experts end in a block of <= 64 routes
    (560, 256, 256, 3, 1, 31),        # the same with two K tiles per stage loop
])
def test_forward_shapes(binding, M, D, I, E, n_routed, seed):
    log(f"forward shape M={M} D={D} I={I} E={E} topk={n_routed + 1}")
    case = custom_case(M, D, I, E, n_routed, seed)
    _check_forward(case, case.run_gpu(debug=True), f"shape M={M} D={D} I={I} E={E}")


@pytest.mark.parametrize("M,D,I,E,n_routed,seed,path", [
    (96, 16384, 1024, 9, 2, 71, "stream"),     # 128 K tiles per stage-1 unit, 64-row blocks
    (640, 16384, 512, 3, 1, 72, "tiled"),      # 128 K stages per stage-1 tile, 4 per stage-2 tile
])
def test_forward_long_k(binding, M, D, I, E, n_routed, seed, path):
    """D = 16,384, beyond the workloads' 7,168: the K loops of both stage-1
    kernels run 128 K tiles.  Checked on a set of tokens covering every used
    block (and its first and last 16-row slices), intermediates included."""
    case = custom_case(M, D, I, E, n_routed, seed)
    dbg = case.run_gpu(debug=True)
    want = {"stream": binding.PATH_STREAM, "tiled": binding.PATH_TILED}[path]
    assert dbg["path"] == want
    toks = covering_tokens(case.ids, case.tw, case.E, dbg["block_m"], must=(0, case.M - 1))
    log(f"long K {path} M={M} D={D} I={I} E={E}: block_m {dbg['block_m']}, oracle on {toks.size} tokens")
    _check_forward(case, dbg, f"long K {path}", tokens=toks)


@pytest.mark.parametrize("M,D,I,E,n_routed,seed,path", [
    (20, 512, 256, 130, 15, 51, "direct"),     # 16 slots: the route-indexed path's limit
    (100, 512, 256, 64, 19, 52, "stream"),     # 20 slots: the 32-slot reduction
    (300, 512, 256, 20, 16, 53, "tiled"),      # 17 slots on the LDS-tiled path
    (60, 512, 256, 40, 14, 54, "stream"),      # 15 slots: the 16-slot reduction, two columns per thread
    (600, 1024, 256, 40, 14, 55, "tiled"),     # 15 slots, eight columns per thread
    (600, 1024, 256, 40, 19, 56, "tiled"),     # 20 slots, eight columns per thread
])
def test_forward_large_topk(binding, M, D, I, E, n_routed, seed, path):
    """Many slots per token: per-token route tables on the route-indexed path,
    the reduction instances for more than 8 and more than 16 slots."""
    case = custom_case(M, D, I, E, n_routed, seed)
    dbg = case.run_gpu(debug=True)
    want = {"direct": binding.PATH_DIRECT, "stream": binding.PATH_STREAM,
            "tiled": binding.PATH_TILED}[path]
    assert dbg["path"] == want
    _check_forward(case, dbg, f"top-{case.topk} {path} M={M} E={E}")


def _random_shapes(n=None, seed=None):
    """Seeded shapes across all paths and block sizes: M from 1 to 3,200, D up
    to 1,536 and I up to 1,024 (multiples of 256), E from 2 to 400 (halved
    while E*D*I exceeds 3.5e8, to keep the oracle's weight quantization short),
    up to 16 slots, uniform or Zipf routing, a quarter with repeated and
    invalid ids; every sixth aims at the paired 32-row blocks (30 to 40 routes
    per expert, I <= 512).  MOE_RANDOM_SHAPES and MOE_RANDOM_SEED set the count
    (40) and the generator's seed (2026) for a longer sweep."""
    import os
    n = int(os.environ.get("MOE_RANDOM_SHAPES", 40)) if n is None else n
    seed = int(os.environ.get("MOE_RANDOM_SEED", 2026)) if seed is None else seed
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 41)) if i % 3 == 0 else int(rng.integers(41, 3201))
        D = 256 * int(rng.integers(1, 7))
        I = 256 * int(rng.integers(1, 5))
        E = int(rng.integers(2, 401))
        while E * D * I > 3.5e8:
            E = max(2, E // 2)
        n_routed = int(rng.integers(1, min(E - 1, 15) + 1))
        if i % 6 == 5:
            M = int(rng.integers(100, 2001))
            I = 256 * int(rng.integers(1, 3))
            n_routed = int(rng.integers(1, 9))
            E = max(n_routed + 1, round(M * (n_routed + 1) / float(rng.uniform(30, 40))))
        routing = "zipf" if rng.random() < 0.3 else "uniform"
        dirty = bool(rng.random() < 0.25)
        out.append((M, D, I, E, n_routed, routing, dirty, seed * 1000 + i))
    return out


@pytest.mark.parametrize("M,D,I,E,n_routed,routing,dirty,seed", _random_shapes())
def test_forward_random_shapes(binding, M, D, I, E, n_routed, routing, dirty, seed):
    """Seeded random shapes, intermediates included, checked on a set of
    tokens covering every used block of the oracle's route list."""
    hidden, ids, tw = inputs.make_activations(M, D, E, n_routed, routing, seed)
    if dirty:
        ids = ids.clone()
        if n_routed > 1:
            ids[::3, 1] = ids[::3, 0]           # a repeated id within a token
        ids[::5, 0] = -1                        # invalid ids
        ids[1::7, -1] = E + 11
    case = custom_case(M, D, I, E, n_routed, seed, routing=routing, ids=ids, tw=tw)
    dbg = case.run_gpu(debug=True)
    toks = covering_tokens(case.ids, case.tw, case.E, dbg["block_m"], must=(0, case.M - 1))
    log(f"random shape M={M} D={D} I={I} E={E} topk={n_routed + 1} {routing} dirty={dirty}: path "
        f"{binding.PATH_NAMES[dbg['path']]}, block_m {dbg['block_m']}, oracle on {toks.size} tokens")
    _check_forward(case, dbg, f"random shape seed {seed}", tokens=toks)


# sorted path (32-row blocks), paired 32-row blocks (33.3 routes per expert at
# I=256), route-indexed path
@pytest.mark.parametrize("M,E", [(20, 6), (100, 12), (8, 40)])
def test_forward_invalid_and_duplicate_ids(binding, M, E):
    D, I = 512, 256
    rng = np.random.default_rng(5)
    ids = rng.integers(0, E, (M, 4)).astype(np.int32)
    ids[:, 1] = ids[:, 0]            # duplicate slot
    ids[::2, 2] = -1                 # invalid
    ids[1::4, 3] = E + 3             # invalid
    tw = rng.random((M, 4)).astype(np.float32)
    case = custom_case(M, D, I, E, 2, 31, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    out = case.run_gpu().cpu().view(torch.int16).numpy().view(np.uint16)
    check_close(out, case.run_oracle(), "invalid/duplicate ids")


def test_forward_tiled_invalid_and_duplicate_ids(binding):
    """The LDS-tiled path (block_m 256, chunked sort) with invalid and repeated
    ids: an expert's valid routes decide which of its rows are computed."""
    M, D, I, E = 1100, 512, 256, 5
    rng = np.random.default_rng(41)
    ids = rng.integers(0, E, (M, 4)).astype(np.int32)
    ids[:, 1] = ids[:, 0]            # duplicate slot
    ids[::2, 2] = -1                 # invalid
    ids[1::4, 3] = E + 3             # invalid
    ids[::5, 3] = E - 1              # one expert with more routes
    tw = rng.random((M, 4)).astype(np.float32)
    case = custom_case(M, D, I, E, 2, 43, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    dbg = case.run_gpu(debug=True)
    assert dbg["block_m"] == 256
    _check_forward(case, dbg, "tiled invalid/duplicate ids")


def test_forward_paired_blocks(binding):
    """32-row blocks whose pairs run as 64-row units split by columns (35.7
    routes per expert at I=256): experts with 33 and 64 routes (one pair), 65
    (a pair and a lone block), 97 and 128 (two pairs), 129 (five blocks: 32-row
    units), a lone 20-route block, unused experts, and the shared expert with
    every token (seventeen blocks: 32-row units)."""
    M, D, I, E = 536, 512, 256, 30
    counts = [33, 64, 65, 97, 128, 129, 20]
    rng = np.random.default_rng(61)
    ids = np.empty((M, 2), np.int32)
    ids[:, 0] = rng.permutation(np.repeat(np.arange(len(counts), dtype=np.int32), counts))
    ids[:, 1] = E - 1
    tw = rng.random((M, 2)).astype(np.float32)
    assert 32 <= M * 2 / E < 37                  # the paired-block range at I <= 512
    case = custom_case(M, D, I, E, 1, 62, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    dbg = case.run_gpu(debug=True)
    assert dbg["path"] == binding.PATH_STREAM and dbg["block_m"] == 32
    _check_forward(case, dbg, "paired 32-row blocks")


def test_forward_all_tokens_one_expert(binding):
    """Every token routed to expert 0 (many blocks of one expert) plus the shared one."""
    M, D, I, E = 300, 512, 512, 4
    ids = np.zeros((M, 2), np.int32)
    ids[:, 1] = E - 1
    tw = np.ones((M, 2), np.float32)
    tw[:, 0] = 0.25
    case = custom_case(M, D, I, E, 1, 41, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    out = case.run_gpu().cpu().view(torch.int16).numpy().view(np.uint16)
    check_close(out, case.run_oracle(), "one hot expert")


def test_forward_no_valid_routes(binding):
    M, D, I, E = 4, 512, 256, 3
    ids = np.full((M, 2), -1, np.int32)
    tw = np.ones((M, 2), np.float32)
    case = custom_case(M, D, I, E, 1, 51, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    out = case.run_gpu()
    assert torch.all(out.cpu().float() == 0)


def test_forward_m_zero(binding):
    E, D, I = 2, 512, 256
    w = [torch.zeros(s, dtype=torch.uint8, device="cuda")
         for s in ((E, 2 * I, D // 2), (E, 2 * I, D // 32), (E, D, I // 2), (E, D, I // 32))]
    h = torch.zeros((0, D), dtype=torch.bfloat16, device="cuda")
    out = binding.moe_mxfp4_forward(h, *w, torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
                                    torch.zeros((0, 2), dtype=torch.float32, device="cuda"),
                                    workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert out.shape == (0, D)


def test_forward_deterministic(binding):
    """The forward is deterministic: two calls give identical bits."""
    case = workload_case("small_batch", M=40)
    a = case.run_gpu().cpu()
    b = case.run_gpu().cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name,M", [("tiny", None), ("small_batch", 40), ("prefill", 1100)])
def test_forward_profiled_matches_forward(binding, name, M):
    """The timed forward gives the same bits as the plain one, and records
    exactly the launches of its path (events attached to the kernels)."""
    import bench
    case = workload_case(name, M=M)
    d = case.device_inputs()
    ref = case.run_gpu()
    ev = bench.Events(8)
    out = torch.empty_like(d["hidden"])
    ws = binding.alloc_workspace(case.M, case.D, case.I, case.E, case.topk)
    n_wg = binding.moe_mxfp4_stage1_workgroups(case.M, case.D, case.I, case.E, case.topk)
    span = torch.zeros(2 * n_wg, dtype=torch.int64, device="cuda")
    binding.moe_mxfp4_forward_profiled(d["hidden"], *d["prepared"], d["ids"], d["tw"], out, ws,
                                       ev.ev, span)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    rec = span.cpu().reshape(-1, 2)
    khz = binding.moe_mxfp4_wall_clock_khz()
    assert khz > 0 and bool((rec > 0).all()) and bool((rec[:, 1] >= rec[:, 0]).all())
    ms = binding.stage1_span_ms(rec, khz)
    log(f"{name} M={case.M} stage-1 span {1000.0 * ms:.2f} us over {n_wg} workgroups")
    assert 0.0 < ms < 1000.0
    path = binding.moe_mxfp4_path(case.M, case.D, case.I, case.E, case.topk)
    for i in binding.PATH_LAUNCHES[path]:
        ms = ev.ms(2 * i, 2 * i + 1)
        log(f"{name} M={case.M} launch {binding.LAUNCHES[i]}: {1000 * ms:.2f} us")
        assert ms > 0.0
    ev.close()
