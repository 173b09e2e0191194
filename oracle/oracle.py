"""ctypes front-end of the C oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Arrays are numpy; bf16 tensors travel as uint16
bit patterns.  The shared library is built by oracle/build.py on first use.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib_path() -> str:
    return _build.LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(os.path.dirname(_build.LIB), "moe_oracle.c")
    if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(src):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P = ctypes.c_void_p
    i32, i64, d = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_e2m1_value.argtypes, lib.oracle_e2m1_value.restype = [i32], d
    lib.oracle_e8m0_value.argtypes, lib.oracle_e8m0_value.restype = [i32], d
    lib.oracle_bf16_value.argtypes, lib.oracle_bf16_value.restype = [ctypes.c_uint16], d
    lib.oracle_bf16_round.argtypes, lib.oracle_bf16_round.restype = [d], ctypes.c_uint16
    lib.oracle_mx_quant_block_f64.argtypes = [P, P, P]
    lib.oracle_mx_quant_block_f64.restype = None
    lib.oracle_mx_quant_block_bf16.argtypes = [P, P, P]
    lib.oracle_mx_quant_block_bf16.restype = None
    lib.oracle_mx_quantize_rows.argtypes = [P, i64, i64, P, P, i32]
    lib.oracle_mx_quantize_rows.restype = i32
    lib.oracle_mx_dequantize_rows.argtypes = [P, P, i64, i64, P]
    lib.oracle_mx_dequantize_rows.restype = i32
    lib.oracle_mx_dot.argtypes, lib.oracle_mx_dot.restype = [P, P, P, P, i64], d
    lib.oracle_route.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, i64]
    lib.oracle_route.restype = i32
    lib.oracle_forward.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, i32,
                                   i32, i32, P, P, P]
    lib.oracle_forward.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _threads(n):
    if n is not None:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e8m0_value(s: int) -> float:
    return _load().oracle_e8m0_value(int(s))


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def bf16_round(x: float) -> int:
    return int(_load().oracle_bf16_round(float(x)))


def quant_block(x):
    """x: 32 values (float64 or uint16 bf16 bits).  Returns (codes[32] u8, scale u8)."""
    lib = _load()
    codes = np.zeros(32, np.uint8)
    scale = np.zeros(1, np.uint8)
    x = np.asarray(x)
    assert x.size == 32
    if x.dtype == np.uint16:
        xb = _c(x, np.uint16)
        lib.oracle_mx_quant_block_bf16(_ptr(xb), _ptr(codes), _ptr(scale))
    else:
        xd = _c(x, np.float64)
        lib.oracle_mx_quant_block_f64(_ptr(xd), _ptr(codes), _ptr(scale))
    return codes, int(scale[0])


def quantize_rows(x_bf16_bits, nthreads=None):
    """x: uint16 [rows, cols].  Returns (packed u8 [rows, cols/2], scales u8 [rows, cols/32])."""
    x = _c(x_bf16_bits, np.uint16)
    rows, cols = x.shape
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    rc = _load().oracle_mx_quantize_rows(_ptr(x), rows, cols, _ptr(packed), _ptr(scales),
                                         _threads(nthreads))
    if rc:
        raise ValueError("oracle_mx_quantize_rows failed")
    return packed, scales


def dequantize_rows(packed, scales):
    p = _c(packed, np.uint8)
    s = _c(scales, np.uint8)
    rows = p.shape[0]
    cols = p.shape[1] * 2
    out = np.empty((rows, cols), np.float64)
    if _load().oracle_mx_dequantize_rows(_ptr(p), _ptr(s), rows, cols, _ptr(out)):
        raise ValueError("oracle_mx_dequantize_rows failed")
    return out


def mx_dot(a_packed, a_scales, w_packed, w_scales) -> float:
    ap, as_ = _c(a_packed, np.uint8), _c(a_scales, np.uint8)
    wp, ws = _c(w_packed, np.uint8), _c(w_scales, np.uint8)
    K = ap.size * 2
    return _load().oracle_mx_dot(_ptr(ap), _ptr(as_), _ptr(wp), _ptr(ws), K)


def route_capacity(M, k, E, bm):
    """An upper bound of the padded sorted length: every expert that receives a
    route adds at most bm-1 padding rows."""
    R = M * k
    cap = R + min(E, R) * (bm - 1)
    return ((cap + bm - 1) // bm) * bm


def route(ids, tw, E, bm):
    """ids int32 [M,k], tw float32 [M,k].  Returns dict with the valid prefix of
    sorted_route, sorted_w, block_expert and num_valid (2,)."""
    ids = _c(ids, np.int32)
    tw = _c(tw, np.float32)
    M, k = ids.shape
    cap = route_capacity(M, k, E, bm)
    sr = np.empty(max(cap, 1), np.int32)
    sw = np.empty(max(cap, 1), np.float32)
    be = np.empty(max(cap // bm, 1), np.int32)
    nv = np.zeros(2, np.int32)
    if _load().oracle_route(_ptr(ids), _ptr(tw), M, k, E, bm, _ptr(sr), _ptr(sw), _ptr(be),
                            _ptr(nv), cap):
        raise ValueError("oracle_route: capacity exceeded")
    n = int(nv[0])
    return {"sorted_route": sr[:n].copy(), "sorted_w": sw[:n].copy(),
            "block_expert": be[: n // bm].copy(), "num_valid": nv.copy(), "cap": cap}


def forward(hidden_bits, w13, w13s, w2, w2s, ids, tw, tokens=None, act_quant=True,
            nthreads=None, want_f64=False, want_h=False):
    """Oracle forward on canonical (raw) layouts.

    hidden_bits uint16 [M,D]; w13 u8 [E,2I,D/2]; w13s u8 [E,2I,D/32];
    w2 u8 [E,D,I/2]; w2s u8 [E,D,I/32]; ids int32 [M,k]; tw float32 [M,k].
    tokens: optional list of token rows to compute (outputs in that order).
    Returns out uint16 [ntok, D] (+ fp64 accumulators, + h [ntok,k,I] if asked).
    """
    h = _c(hidden_bits, np.uint16)
    M, D = h.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    ids = _c(ids, np.int32)
    tw = _c(tw, np.float32)
    k = ids.shape[1]
    w13 = _c(w13, np.uint8)
    w13s = _c(w13s, np.uint8)
    w2 = _c(w2, np.uint8)
    w2s = _c(w2s, np.uint8)
    assert w13s.shape == (E, 2 * I, D // 32) and w2.shape == (E, D, I // 2)
    assert w2s.shape == (E, D, I // 32) and ids.shape == tw.shape == (M, k)
    tok = None if tokens is None else _c(tokens, np.int32)
    ntok = M if tok is None else tok.size
    out = np.empty((ntok, D), np.uint16)
    of = np.empty((ntok, D), np.float64) if want_f64 else None
    ho = np.empty((ntok, k, I), np.uint16) if want_h else None
    rc = _load().oracle_forward(_ptr(h), _ptr(w13), _ptr(w13s), _ptr(w2), _ptr(w2s), _ptr(ids),
                                _ptr(tw), M, D, I, E, k, _ptr(tok), ntok, 1 if act_quant else 0,
                                _threads(nthreads), _ptr(out), _ptr(of), _ptr(ho))
    if rc:
        raise ValueError("oracle_forward: bad arguments")
    res = [out]
    if want_f64:
        res.append(of)
    if want_h:
        res.append(ho)
    return res[0] if len(res) == 1 else tuple(res)
