"""The requant allowance of the GPU parity tests (tests/moe_cases.requant_moves
and requant_slack), checked on the CPU.

A GPU requant code may differ from the oracle's only where the two bf16 h
values sit on opposite sides of a decision boundary of the MXFP4 rounding:
the midpoint between two adjacent E2M1 magnitudes (same scale byte), or the
power of two where the scale byte steps (block maxima on either side).  The
tests plant each accepted kind and each rejected one on small hand-made
blocks (scale byte 127 unless stated), then check the output slack on a
whole case built from the oracle's own intermediates."""
import numpy as np
import pytest
import torch

import oracle
from tests.moe_cases import bf16_to_f64, custom_case, requant_moves, requant_slack


def _bits(vals):
    """float values (bf16-representable) -> bf16 bit patterns [1, n]."""
    a = np.asarray(vals, np.float32).view(np.uint32)
    assert np.all((a & 0xFFFF) == 0), vals
    return (a >> 16).astype(np.uint16).reshape(1, -1)


def _block(**changes):
    """32 values with block maximum 6 (scale byte 127): element 0 = 6, the
    others small distinct grid-interior values; `changes` {index: value}."""
    v = np.array([6.0] + [0.625, 1.125, 1.625, 2.25, 2.75, 3.25, 4.5] * 4 + [0.375, 0.875, 0.125],
                 np.float64)
    assert v.size == 32
    for i, x in changes.items():
        v[int(i)] = x
    return v


def _quant(vals):
    c, s = oracle.quantize_rows(_bits(vals))
    return c, s


def _moves(h_gpu_vals, h_or_vals, gc=None, gs=None):
    hg, ho = _bits(h_gpu_vals), _bits(h_or_vals)
    qc, qs = _quant(h_gpu_vals)
    oc, os_ = _quant(h_or_vals)
    return requant_moves(hg, ho, qc if gc is None else gc, qs if gs is None else gs, oc, os_)


def test_identical_codes_no_move():
    v = _block()
    dv = _moves(v, v)
    assert not dv.any()


def test_one_step_midpoint_crossing_accepted():
    # 0.625 rounds to 0.5; 0.7578125 (the bf16 above the midpoint 0.75) rounds to 1.0
    dv = _moves(_block(**{"1": 0.7578125}), _block(**{"1": 0.6875}))
    assert dv[0, 1] == 0.5 and np.count_nonzero(dv) == 1


def test_tie_on_the_midpoint_accepted():
    # exactly 0.75: ties to the even code (1.0); 0.7421875 rounds to 0.5
    dv = _moves(_block(**{"1": 0.75}), _block(**{"1": 0.7421875}))
    assert dv[0, 1] == 0.5


def test_zero_crossing_accepted_and_signed_zero_free():
    # +0.2 -> +0 against -0.3 -> -0.5: adjacent magnitudes across 0.25
    dv = _moves(_block(**{"30": 0.19921875}), _block(**{"30": -0.30078125}))
    assert dv[0, 30] == 0.5
    # +0.1 -> +0 against -0.1 -> -0: codes differ, values do not
    dv = _moves(_block(**{"31": 0.10009765625}), _block(**{"31": -0.10009765625}))
    assert not dv.any()


def test_two_step_move_rejected():
    # 1.3 rounds to 1.5 (magnitude index 3), 0.625 to 0.5 (index 1)
    with pytest.raises(AssertionError, match="one-step midpoint"):
        _moves(_block(**{"1": 1.296875}), _block(**{"1": 0.625}))


def test_one_step_without_bracketing_rejected():
    # both h are 0.625 (oracle code 0.5) but the GPU code says 1.0
    v = _block()
    qc, qs = _quant(v)
    bad = qc.copy()
    bad[0, 0] = (bad[0, 0] & 0x0F) | (0x2 << 4)        # element 1 (high nibble of byte 0) -> 1.0
    with pytest.raises(AssertionError, match="one-step midpoint"):
        _moves(v, v, gc=bad, gs=qs)


def test_sign_flip_of_a_nonzero_code_rejected():
    v = _block()
    qc, qs = _quant(v)
    bad = qc.copy()
    bad[0, 0] ^= 0x80                                   # element 1: +0.5 -> -0.5
    with pytest.raises(AssertionError):
        _moves(v, v, gc=bad, gs=qs)


def test_scale_step_with_bracketing_maxima_accepted():
    # amax 4.0 -> byte 127; amax 3.984375 (just below 4) -> byte 126
    small = _block() * 0.5                              # every other element below 2.25
    hg, ho = small.copy(), small.copy()
    hg[0], ho[0] = 4.0, 3.984375
    _, sg = _quant(hg)
    _, so = _quant(ho)
    assert int(sg[0, 0]) == 127 and int(so[0, 0]) == 126
    dv = _moves(hg, ho)
    assert dv.any()


def test_unexplained_scale_change_rejected():
    v = _block()
    qc, qs = _quant(v)
    with pytest.raises(AssertionError, match="scale step"):
        _moves(v, v, gc=qc, gs=(qs + 1).astype(np.uint8))


def test_scale_two_bytes_apart_rejected():
    small = _block() * 0.5
    hg, ho = small.copy(), small.copy()
    hg[0], ho[0] = 8.0, 3.984375
    with pytest.raises(AssertionError, match="scale step"):
        _moves(hg, ho)


# -------------------------------------------- output slack on a whole case ---

def _oracle_debug(case, h_gpu, bm=16):
    """Debug-shaped outputs built from the oracle alone: sorted rows, h_gpu
    (given, [M, k, I] bits) and its quantization as the GPU would store it."""
    rt = oracle.route(case.ids, case.tw, case.E, bm)
    sr = rt["sorted_route"]
    n = int(rt["num_valid"][0])
    R = case.M * case.topk
    codes = np.zeros((n, case.I // 2), np.uint8)
    scales = np.zeros((n, case.I // 32), np.uint8)
    hrows = np.zeros((n, case.I), np.uint16)
    rows = np.nonzero(sr[:n] < R)[0]
    r = sr[rows]
    hrows[rows] = h_gpu[r // case.topk, r % case.topk]
    c, s = oracle.quantize_rows(hrows[rows])
    codes[rows], scales[rows] = c, s
    return {"sorted_route": torch.from_numpy(sr.astype(np.int32)),
            "num_valid": torch.from_numpy(rt["num_valid"].astype(np.int32)),
            "h": torch.from_numpy(hrows.view(np.int16)).view(torch.bfloat16),
            "a2_codes": torch.from_numpy(codes), "a2_scales": torch.from_numpy(scales)}


def test_requant_slack_zero_when_codes_agree():
    case = custom_case(6, 256, 256, 4, 2, 5, device="cpu")
    _, h_or = case.run_oracle(want_h=True)
    slack, moved, total = requant_slack(case, _oracle_debug(case, h_or), h_or)
    assert slack is None and moved == 0 and total > 0


def _midpoint_element(h_or, case):
    """A (t, s, i) whose |h| / X lies in (0.5, 0.75) and is not its block's
    maximum, and the bf16 just above the midpoint 0.75 X with h's sign."""
    for t in range(case.M):
        for s in range(case.topk):
            if not (0 <= case.ids[t, s] < case.E):
                continue
            row = bf16_to_f64(h_or[t, s])
            for i in range(case.I):
                blk = np.abs(row[i // 32 * 32:(i // 32 + 1) * 32])
                amax = blk.max()
                if amax == 0:
                    continue
                X = 2.0 ** (np.floor(np.log2(amax)) - 2)
                v = abs(row[i]) / X
                if 0.5 < v < 0.75 and abs(row[i]) < amax:
                    up = np.float32(0.75 * X)
                    u = up.view(np.uint32) + np.uint32(1 << 16)       # next bf16 above
                    val = float(np.uint32(u).view(np.float32)) * np.sign(row[i])
                    return t, s, i, val, X
    raise AssertionError("no element in (0.5, 0.75) X")


def test_requant_slack_one_explained_move():
    case = custom_case(6, 256, 256, 4, 2, 6, device="cpu")
    _, h_or = case.run_oracle(want_h=True)
    t, s, i, val, X = _midpoint_element(h_or, case)
    h_gpu = h_or.copy()
    h_gpu[t, s, i] = _bits([val])[0, 0]
    slack, moved, _ = requant_slack(case, _oracle_debug(case, h_gpu), h_or)
    assert moved == 1
    e = int(case.ids[t, s])
    w2 = oracle.dequantize_rows(case.wq[2][e], case.wq[3][e])
    want = abs(float(case.tw[t, s])) * 0.5 * X * np.abs(w2[:, i])
    np.testing.assert_allclose(slack[t], want, rtol=1e-12)
    assert not np.delete(slack, t, axis=0).any()


def test_requant_slack_restricted_to_sampled_tokens():
    case = custom_case(6, 256, 256, 4, 2, 6, device="cpu")
    _, h_or = case.run_oracle(want_h=True)
    t, s, i, val, X = _midpoint_element(h_or, case)
    h_gpu = h_or.copy()
    h_gpu[t, s, i] = _bits([val])[0, 0]
    toks = np.array([t, (t + 2) % case.M])
    slack, moved, _ = requant_slack(case, _oracle_debug(case, h_gpu), h_or[toks], tokens=toks)
    assert moved == 1 and slack.shape == (2, case.D) and slack[0].any() and not slack[1].any()
    others = np.array([u for u in range(case.M) if u != t][:2])
    slack, moved, _ = requant_slack(case, _oracle_debug(case, h_gpu), h_or[others], tokens=others)
    assert slack is None and moved == 0


def test_requant_slack_rejects_codes_that_are_not_quant_of_gpu_h():
    case = custom_case(6, 256, 256, 4, 2, 6, device="cpu")
    _, h_or = case.run_oracle(want_h=True)
    dbg = _oracle_debug(case, h_or)
    rows = np.nonzero(dbg["sorted_route"].numpy()[: int(dbg["num_valid"][0])] < case.M * case.topk)[0]
    dbg["a2_codes"][int(rows[0]), 0] ^= 0x01
    with pytest.raises(AssertionError, match="not the MXFP4 quantization"):
        requant_slack(case, dbg, h_or)
