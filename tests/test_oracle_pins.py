"""Pins of the CPU oracle against things other than itself (CPU only).

- hand-written E2M1 / e8m0 tables (tests/golden), from the decoders printed on
  kernelindex submission 723815 and the OCP MX v1.0 definitions;
- hand-worked MXFP4 quantization cases (tests/golden/mx_quant_cases.txt);
- the MXFP4 dequantizer element by element against the hand tables;
- brute force: every quantized element is the nearest grid point (ties to even);
- invariants: requantizing an MXFP4-representable block is the identity;
- the textbook float32 -> bf16 round-to-nearest-even bit trick;
- closed forms of the whole forward (M=1, E=1, all-ones weights);
- an independent dense numpy forward (tests/dense_ref.py);
- brute-force routing lists.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import dense_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _f64_to_bf16_bits(v):
    """Exact conversion of a bf16-representable double to its bit pattern."""
    b = np.array([v], np.float32).view(np.uint32)[0]
    assert (b & 0xFFFF) == 0, v
    return np.uint16(b >> 16)


# ---------------------------------------------------------------- tables ---

def test_e2m1_table_every_code():
    for code_s, val_s in _read_pairs("e2m1_table.txt"):
        code, val = int(code_s, 16), float(val_s)
        got = oracle.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


def test_e8m0_table():
    for s_s, v_s in _read_pairs("e8m0_table.txt"):
        s = int(s_s)
        got = oracle.e8m0_value(s)
        if v_s == "nan":
            assert math.isnan(got)
        else:
            assert got == float.fromhex(v_s), (s, got)


def test_e2m1_codes_round_trip_through_quantizer():
    """Each of the 16 codes, placed in a block whose amax pins the scale to 127,
    decodes and re-quantizes to itself."""
    for code in range(16):
        x = np.zeros(32)
        x[0] = 6.0          # amax 6 -> floor(log2 6) - 2 + 127 = 127
        x[1] = oracle.e2m1_value(code)
        codes, s = oracle.quant_block(x)
        assert s == 127
        assert codes[0] == 0x7 and codes[1] == code, (code, codes[1])


def test_e8m0_scales_round_trip_through_quantizer():
    """A block with amax 4 * 2^(s-127) quantizes to scale byte s for every s."""
    for s in range(0, 255):
        x = np.zeros(32)
        x[5] = 4.0 * 2.0 ** (s - 127)
        codes, got = oracle.quant_block(x)
        if s == 0:
            assert got == 0 and codes[5] == 0x6
        else:
            assert got == s, (s, got)
            assert codes[5] == 0x6


# -------------------------------------------------------------- bf16 RNE ---

def test_bf16_round_matches_float32_bit_trick():
    """For float32 inputs (exact doubles) RNE to bf16 is the textbook
    (u + 0x7FFF + ((u >> 16) & 1)) >> 16 on the bit pattern."""
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) < 3.3e38)
    f = f[keep]
    u = f.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    for x, w in zip(f[:5000], want[:5000]):
        assert oracle.bf16_round(float(x)) == int(w), (x, w)


def test_bf16_round_ties_and_signs():
    one = 1.0
    ulp = 2.0 ** -7
    assert oracle.bf16_round(one + ulp / 2) == 0x3F80          # tie -> even (1.0)
    assert oracle.bf16_round(one + 3 * ulp / 2) == 0x3F82      # tie -> even (1+2ulp)
    assert oracle.bf16_round(-0.0) == 0x8000
    assert oracle.bf16_round(0.73105857863) == 0x3F3B          # 0.73046875
    assert oracle.bf16_value(0x3F3B) == 0.73046875


# ----------------------------------------------------------- MX quantize ---

def _golden_quant_cases():
    cases = []
    with open(os.path.join(GOLDEN, "mx_quant_cases.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, scale, xs, cs = [p.strip() for p in line.split("|")]
            x = np.zeros(32)
            codes = np.zeros(32, np.uint8)
            for tok in xs.split():
                i, v = tok.split(":")
                x[int(i)] = float.fromhex(v)
            for tok in cs.split():
                i, c = tok.split(":")
                codes[int(i)] = int(c, 16)
            cases.append((name, int(scale), x, codes))
    return cases


@pytest.mark.parametrize("case", _golden_quant_cases(), ids=lambda c: c[0])
def test_quant_hand_worked_cases(case):
    name, scale, x, codes = case
    bits = np.array([_f64_to_bf16_bits(v) for v in x], np.uint16)
    got_codes, got_scale = oracle.quant_block(bits)
    assert got_scale == scale, name
    np.testing.assert_array_equal(got_codes, codes, err_msg=name)


def _brute_force_check(x, codes, s):
    """Exact check of one block: scale from the OCP rule, each code the nearest
    grid point of |x|/X with ties to the even index, saturating, sign copied."""
    amax = max(abs(v) for v in x)
    if amax == 0:
        assert s == 0
    else:
        e = math.frexp(amax)[1] - 1
        assert s == min(max(e - 2 + 127, 0), 254)
    X = Fraction(2) ** (s - 127)
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    for v, c in zip(x, codes):
        q = abs(Fraction(v)) / X
        dist = [abs(q - g) for g in grid]
        best = min(dist)
        cand = [j for j in range(8) if dist[j] == best]
        want = 7 if q >= 6 else (cand[0] if len(cand) == 1 else [j for j in cand if j % 2 == 0][0])
        assert (c & 7) == want, (v, q, c)
        assert (c >> 3) == (1 if math.copysign(1, v) < 0 else 0)


def test_quant_brute_force_random_blocks():
    rng = np.random.default_rng(1)
    for trial in range(400):
        scale = 2.0 ** rng.integers(-130, 120)
        x = rng.standard_normal(32) * scale
        if trial % 7 == 0:
            x[rng.integers(0, 32, 5)] = 0.0
        if trial % 11 == 0:
            x = np.round(x / scale * 4) / 4 * scale           # many exact ties
        f32 = x.astype(np.float32).view(np.uint32)
        bits = ((f32.astype(np.uint64) + 0x7FFF + ((f32 >> 16) & 1)) >> 16).astype(np.uint16)
        xv = [oracle.bf16_value(int(b)) for b in bits]
        codes, s = oracle.quant_block(bits)
        _brute_force_check(xv, codes, s)


def test_quant_idempotent_on_representable_blocks():
    """dequant(quant(dequant(q, s))) == dequant(q, s); codes are identical when
    the block's largest magnitude is 4 or 6 (the scale is then recovered)."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        s = int(rng.integers(3, 250))
        codes = rng.integers(0, 16, 32).astype(np.uint8)
        codes[rng.integers(0, 32)] = rng.choice([0x6, 0x7, 0xE, 0xF])
        x = np.array([oracle.e2m1_value(int(c)) * 2.0 ** (s - 127) for c in codes])
        c2, s2 = oracle.quant_block(x)
        x2 = np.array([oracle.e2m1_value(int(c)) * 2.0 ** (s2 - 127) for c in c2])
        np.testing.assert_array_equal(x2, x)
        assert s2 == s
        np.testing.assert_array_equal(c2, codes)


def test_quantize_rows_matches_numpy_quantizer():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((37, 256)) * np.exp2(rng.integers(-20, 20, (37, 1)))).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    packed, scales = oracle.quantize_rows(bits)
    codes_np, scales_np = dense_ref.quantize(dense_ref.bf16_bits_to_f64(bits))
    np.testing.assert_array_equal(scales, scales_np)
    np.testing.assert_array_equal(dense_ref.unpack(packed), codes_np)


def test_dequantize_rows_against_hand_tables():
    """oracle_mx_dequantize_rows on a non-square matrix (3 rows x 3 blocks):
    every byte holds two different nibbles, every (row, block) its own scale
    byte from the hand-written e8m0 table, so a swapped nibble order, a wrong
    row pitch of the scales (cols/32) or a wrong block index (i/32) changes
    the result.  Expected values: the hand tables, element by element."""
    e2m1 = {int(c, 16): float(v) for c, v in _read_pairs("e2m1_table.txt")}
    e8m0 = {int(b): float.fromhex(v) for b, v in _read_pairs("e8m0_table.txt") if v != "nan"}
    rows, cols = 3, 96
    rng = np.random.default_rng(17)
    lo = rng.integers(0, 16, (rows, cols // 2))
    hi = (lo + rng.integers(1, 16, (rows, cols // 2))) % 16        # differs from lo
    packed = (lo | (hi << 4)).astype(np.uint8)
    table_bytes = sorted(e8m0)                                    # 0, 1, 126, 127, 128, 200, 254
    scales = np.array(table_bytes + table_bytes[:2], np.uint8).reshape(rows, cols // 32)
    got = oracle.dequantize_rows(packed, scales)
    for r in range(rows):
        for i in range(cols):
            code = int(packed[r, i // 2]) >> (4 * (i % 2)) & 0xF
            want = e2m1[code] * e8m0[int(scales[r, i // 32])]
            assert got[r, i] == want and math.copysign(1, got[r, i]) == math.copysign(1, want), \
                (r, i, got[r, i], want)


def test_dequantize_rows_matches_numpy_dequant():
    """The same function against the independent numpy decoder on random
    codes and random (finite) scale bytes per block."""
    rng = np.random.default_rng(23)
    packed = rng.integers(0, 256, (7, 160)).astype(np.uint8)
    scales = rng.integers(0, 255, (7, 10)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.dequantize_rows(packed, scales),
                                  dense_ref.dequant(packed, scales))


def test_mx_dot_matches_dense_dot():
    rng = np.random.default_rng(4)
    for K in (32, 256, 7168):
        ap = rng.integers(0, 256, K // 2).astype(np.uint8)
        wp = rng.integers(0, 256, K // 2).astype(np.uint8)
        as_ = rng.integers(110, 140, K // 32).astype(np.uint8)
        ws = rng.integers(110, 140, K // 32).astype(np.uint8)
        got = oracle.mx_dot(ap, as_, wp, ws)
        want = float(np.dot(dense_ref.dequant(ap, as_), dense_ref.dequant(wp, ws)))
        assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (K, got, want)


# ------------------------------------------------------- forward closed forms ---

def _ones_expert(D, I, E=1):
    w13 = np.full((E, 2 * I, D // 2), 0x22, np.uint8)       # every code 0x2 = 1.0
    w13s = np.full((E, 2 * I, D // 32), 127, np.uint8)
    w2 = np.full((E, D, I // 2), 0x22, np.uint8)
    w2s = np.full((E, D, I // 32), 127, np.uint8)
    return w13, w13s, w2, w2s


def test_closed_form_small_input():
    """D=I=256, hidden = 2^-8: a1 = code 4.0 at scale 2^-10, g = u = 1,
    h = bf16(silu(1)) = 0.73046875 -> requantized 0.75, out = 0.75 * 256 = 192."""
    D = I = 256
    hidden = np.full((1, D), _f64_to_bf16_bits(2.0 ** -8), np.uint16)
    w = _ones_expert(D, I)
    out, h = oracle.forward(hidden, *w, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                            want_h=True)
    assert np.all(h == 0x3F3B)
    assert np.all(out == _f64_to_bf16_bits(192.0))


def test_closed_form_large_input():
    """D=512, I=256, hidden = 1: g = u = 512, silu(512)*512 = 2^18 exactly,
    out = 256 * 2^18 = 2^26."""
    D, I = 512, 256
    hidden = np.full((1, D), _f64_to_bf16_bits(1.0), np.uint16)
    w = _ones_expert(D, I)
    out = oracle.forward(hidden, *w, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32))
    assert np.all(out == _f64_to_bf16_bits(2.0 ** 26))


def test_closed_form_duplicate_slots_and_weights():
    """Two slots naming one expert with weight 0.5 each equal one slot with
    weight 1; an id outside [0, E) contributes nothing."""
    D, I = 256, 256
    hidden = np.full((1, D), _f64_to_bf16_bits(2.0 ** -8), np.uint16)
    w = _ones_expert(D, I)
    one = oracle.forward(hidden, *w, np.array([[0]], np.int32), np.array([[1.0]], np.float32))
    two = oracle.forward(hidden, *w, np.array([[0, 0]], np.int32),
                         np.array([[0.5, 0.5]], np.float32))
    bad = oracle.forward(hidden, *w, np.array([[0, 1, -1]], np.int32),
                         np.array([[1.0, 7.0, 7.0]], np.float32))
    np.testing.assert_array_equal(one, two)
    np.testing.assert_array_equal(one, bad)


def test_closed_form_weighted_rows():
    """Rows with distinct scales pin row/scale indexing and the requant.

    hidden = 2^-8 (a1 = 4.0 at scale 2^-10, i.e. exactly 2^-8), gate row n has
    scale byte 127 + n%4, up rows scale 127, all codes 1.0, so g_n = 2^(n%4),
    u_n = 1 and h_n = bf16(silu(2^(n%4))):
      silu(1) = 0.7310586 -> 0.73046875   silu(2) = 1.7615942 -> 1.7578125
      silu(4) = 3.9280552 -> 3.921875     silu(8) = 7.9973172 -> 8.0
    Each 32-group of h holds 8 of each; amax 8 gives scale 2^(3-2) = 2 and
    |h|/2 = 0.365, 0.879, 1.961, 4 -> 0.5, 1, 2, 4, i.e. values 1, 2, 4, 8,
    group sum 8 * 15 = 120.  Down row d has scale 127 + d%3, so
    y_d = 8 groups * 120 * 2^(d%3) and with weight 0.5 out_d = 480 * 2^(d%3).
    """
    D, I = 256, 256
    w13, w13s, w2, w2s = _ones_expert(D, I)
    for n in range(I):
        w13s[0, n, :] = 127 + n % 4           # gate rows
    for d in range(D):
        w2s[0, d, :] = 127 + d % 3
    hidden = np.full((1, D), _f64_to_bf16_bits(2.0 ** -8), np.uint16)
    out, of, h = oracle.forward(hidden, w13, w13s, w2, w2s, np.zeros((1, 1), np.int32),
                                np.full((1, 1), 0.5, np.float32), want_f64=True, want_h=True)
    hv = {0: 0.73046875, 1: 1.7578125, 2: 3.921875, 3: 8.0}
    assert [oracle.bf16_value(int(b)) for b in h[0, 0]] == [hv[n % 4] for n in range(I)]
    want = np.array([480.0 * 2.0 ** (d % 3) for d in range(D)])
    np.testing.assert_array_equal(of[0], want)
    np.testing.assert_array_equal(out[0], [_f64_to_bf16_bits(v) for v in want])


# ------------------------------------------------------- dense cross-check ---

def _tiny_case(seed=0, M=8, D=512, I=256, E=9, n_routed=2):
    import torch
    from mixture_experts_mxfp4_amd import inputs
    hidden, ids, tw = inputs.make_activations(M, D, E, n_routed, "uniform", seed)
    w13f, w2f = inputs.make_weights(E, D, I, seed)
    hb = inputs.bf16_bits(hidden)
    w13, w13s = oracle.quantize_rows(inputs.bf16_bits(w13f).reshape(E * 2 * I, D))
    w2, w2s = oracle.quantize_rows(inputs.bf16_bits(w2f).reshape(E * D, I))
    return (hb, w13.reshape(E, 2 * I, D // 2), w13s.reshape(E, 2 * I, D // 32),
            w2.reshape(E, D, I // 2), w2s.reshape(E, D, I // 32), ids.numpy(), tw.numpy())


@pytest.mark.parametrize("act_quant", [True, False])
def test_oracle_matches_dense_numpy(act_quant):
    args = _tiny_case()
    out, of = oracle.forward(*args, act_quant=act_quant, want_f64=True)
    dense = dense_ref.dense_forward(*args, act_quant=act_quant)
    rms = np.sqrt(np.mean(dense ** 2))
    assert rms > 0
    # only summation order differs: fp64 round-off, plus the rare bf16/MX
    # rounding flip it can cause; these stay far below the GPU tolerance
    diff = np.abs(of - dense)
    assert np.mean(diff <= 1e-9 * rms) >= 0.999
    assert diff.max() <= 1e-2 * rms
    np.testing.assert_array_equal(out, np.array(
        [[_f64_to_bf16_bits(v) for v in row] for row in dense_ref.round_bf16(of)]))


def test_token_subset_matches_full_forward():
    args = _tiny_case(seed=5)
    full = oracle.forward(*args)
    sub = oracle.forward(*args, tokens=[6, 1, 1])
    np.testing.assert_array_equal(sub, full[[6, 1, 1]])


def test_thread_count_does_not_change_result():
    args = _tiny_case(seed=6)
    np.testing.assert_array_equal(oracle.forward(*args, nthreads=1),
                                  oracle.forward(*args, nthreads=5))


# ---------------------------------------------------------------- routing ---

def _brute_route(ids, tw, E, bm):
    M, k = ids.shape
    lists = {e: [] for e in range(E)}
    for r in range(M * k):
        e = int(ids.reshape(-1)[r])
        if 0 <= e < E:
            lists[e].append(r)
    sr, sw, be = [], [], []
    for e in range(E):
        n = len(lists[e])
        if n == 0:
            continue
        padded = -(-n // bm) * bm
        sr += lists[e] + [M * k] * (padded - n)
        sw += [float(tw.reshape(-1)[r]) for r in lists[e]] + [0.0] * (padded - n)
        be += [e] * (padded // bm)
    return np.array(sr, np.int32), np.array(sw, np.float32), np.array(be, np.int32)


@pytest.mark.parametrize("M,E,k,bm", [(8, 9, 3, 16), (16, 257, 9, 16), (64, 33, 9, 32),
                                      (1, 4, 1, 16), (0, 5, 2, 16), (37, 6, 4, 64)])
def test_route_matches_brute_force(M, E, k, bm):
    rng = np.random.default_rng(M * 31 + E)
    ids = rng.integers(-1, E + 1, (M, k)).astype(np.int32)     # includes invalid ids
    tw = rng.random((M, k)).astype(np.float32)
    got = oracle.route(ids, tw, E, bm)
    sr, sw, be = _brute_route(ids, tw, E, bm)
    np.testing.assert_array_equal(got["sorted_route"], sr)
    np.testing.assert_array_equal(got["sorted_w"], sw)
    np.testing.assert_array_equal(got["block_expert"], be)
    valid = int(np.sum((ids >= 0) & (ids < E)))
    assert got["num_valid"][1] == valid
    assert got["num_valid"][0] == sr.size <= got["cap"]
