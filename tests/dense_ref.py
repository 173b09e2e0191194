"""An independent, vectorized numpy cross-check of the oracle (test code).

Written separately from the C oracle: weights are dequantized through the
hand-written E2M1 table in tests/golden/e2m1_table.txt, the MX quantizer picks
the nearest grid point with numpy argmin, bf16 rounding uses numpy's
round-half-even, and the experts run as dense matmuls over a dense [M, E]
routing-weight matrix.  Its agreement with the oracle pins the oracle's
indexing (gate/up rows, nibble order, scale blocks, slot weights).
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_e2m1_table():
    vals = np.zeros(16, np.float64)
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            vals[int(code, 16)] = float(val)
    return vals


E2M1 = load_e2m1_table()
MAGS = E2M1[:8]


def unpack(packed):
    """[..., n/2] bytes -> [..., n] codes, low nibble first."""
    p = np.asarray(packed, np.uint8)
    lo = p & 0xF
    hi = p >> 4
    return np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)


def dequant(packed, scales):
    codes = unpack(packed)
    v = E2M1[codes]
    s = np.asarray(scales, np.float64)
    sv = np.where(s == 255, np.nan, np.exp2(s - 127.0))
    shp = v.shape
    v = v.reshape(*shp[:-1], shp[-1] // 32, 32) * sv[..., None]
    return v.reshape(shp)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x):
    """Round float64 -> nearest bf16 value (ties to even), returned as float64."""
    x = np.asarray(x, np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    m, e = np.frexp(np.abs(x[nz]))        # |x| = m * 2^e, m in [0.5, 1)
    e = e - 1                              # floor(log2|x|)
    q = np.where(e < -126, -133, e - 7).astype(np.float64)
    r = np.rint(np.abs(x[nz]) / np.exp2(q)) * np.exp2(q)   # np.rint: half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out[nz] = np.sign(x[nz]) * r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def quantize(x):
    """x: float64 [..., n] (n % 32 == 0) -> (codes [..., n] u8 unpacked, scales [..., n/32])."""
    x = np.asarray(x, np.float64)
    shp = x.shape
    xb = x.reshape(*shp[:-1], shp[-1] // 32, 32)
    amax = np.abs(xb).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    s = np.where(amax > 0, np.clip(e - 1 - 2 + 127, 0, 254), 0).astype(np.int64)
    v = np.abs(xb) / np.exp2(s - 127.0)[..., None]
    d = np.abs(v[..., None] - MAGS)                       # distance to the 8 magnitudes
    nearest = d == d.min(axis=-1, keepdims=True)          # one index, or two on a tie
    even = nearest & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(nearest, axis=-1))
    idx = np.where(v >= 6.0, 7, idx)
    neg = np.signbit(xb)
    codes = (idx | (neg.astype(np.int64) << 3)).astype(np.uint8)
    return codes.reshape(shp), s.astype(np.uint8)


def dense_forward(hidden_bits, w13, w13s, w2, w2s, ids, tw, act_quant=True):
    """Dense cross-check: every expert runs on every token, masked by a dense
    [M, E] weight matrix built from (ids, tw).  Returns float64 [M, D] before
    the final bf16 rounding."""
    x = bf16_bits_to_f64(hidden_bits)
    M, D = x.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    route_w = np.zeros((M, E, ids.shape[1]), np.float64)
    for t in range(M):
        for s in range(ids.shape[1]):
            e = int(ids[t, s])
            if 0 <= e < E:
                route_w[t, e, s] = float(tw[t, s])
    if act_quant:
        c, sc = quantize(x)
        xq = E2M1[c] * np.repeat(np.exp2(sc.astype(np.float64) - 127.0), 32, axis=-1)
    else:
        xq = x
    out = np.zeros((M, D), np.float64)
    for e in range(E):
        slots = route_w[:, e, :]
        if not np.any(slots != 0):
            continue
        W13 = dequant(w13[e], w13s[e])            # [2I, D]
        W2 = dequant(w2[e], w2s[e])               # [D, I]
        g = xq @ W13[:I].T
        u = xq @ W13[I:].T
        h = round_bf16(g / (1.0 + np.exp(-g)) * u)
        if act_quant:
            c2, s2 = quantize(h)
            h = E2M1[c2] * np.repeat(np.exp2(s2.astype(np.float64) - 127.0), 32, axis=-1)
        y = h @ W2.T                              # [M, D]
        out += slots.sum(axis=1)[:, None] * y
    return out
