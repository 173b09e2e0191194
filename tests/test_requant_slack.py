"""The output slack that the GPU parity tests allow for requant codes one grid
step from the oracle's (tests/moe_cases.requant_slack), checked on the CPU with
the oracle's own intermediates standing in for the debug outputs: no slack when
every code agrees; moving one code gives slack on exactly that code's token, of
|w| * |dv| * |W2[e][:, i]|."""
import numpy as np
import torch

import oracle
from tests.moe_cases import custom_case, requant_slack


def _oracle_debug(case, bm=16):
    """Debug-shaped outputs built from the oracle alone (sorted rows, codes)."""
    rt = oracle.route(case.ids, case.tw, case.E, bm)
    sr = rt["sorted_route"]
    n = int(rt["num_valid"][0])
    R = case.M * case.topk
    _, h = case.run_oracle(want_h=True)
    codes = np.zeros((n, case.I // 2), np.uint8)
    scales = np.zeros((n, case.I // 32), np.uint8)
    rows = np.nonzero(sr[:n] < R)[0]
    r = sr[rows]
    c, s = oracle.quantize_rows(h[r // case.topk, r % case.topk])
    codes[rows], scales[rows] = c, s
    return {"sorted_route": torch.from_numpy(sr.astype(np.int32)),
            "num_valid": torch.from_numpy(rt["num_valid"].astype(np.int32)),
            "a2_codes": torch.from_numpy(codes), "a2_scales": torch.from_numpy(scales)}, rows, r


def test_requant_slack_zero_when_codes_agree():
    case = custom_case(6, 256, 256, 4, 2, 5, device="cpu")
    dbg, _, _ = _oracle_debug(case)
    slack, moved, total = requant_slack(case, dbg)
    assert slack is None and moved == 0 and total > 0


def test_requant_slack_one_moved_code():
    case = custom_case(6, 256, 256, 4, 2, 6, device="cpu")
    dbg, rows, r = _oracle_debug(case)
    j = 3                                    # one valid sorted row
    p, route = int(rows[j]), int(r[j])
    t, s = route // case.topk, route % case.topk
    codes = dbg["a2_codes"].numpy()
    i = 10                                   # h element 10 = low nibble of byte 5
    old = int(codes[p, i // 2]) & 0xF
    new = old ^ 0x1                          # the neighbouring E2M1 magnitude
    codes[p, i // 2] = (int(codes[p, i // 2]) & 0xF0) | new
    slack, moved, _ = requant_slack(case, dbg)
    assert moved == 1
    scale = oracle.e8m0_value(int(dbg["a2_scales"].numpy()[p, i // 32]))
    dv = abs(oracle.e2m1_value(new) - oracle.e2m1_value(old)) * scale
    e = int(case.ids[t, s])
    w2 = oracle.dequantize_rows(case.wq[2][e], case.wq[3][e])
    want = abs(float(case.tw[t, s])) * dv * np.abs(w2[:, i])
    np.testing.assert_allclose(slack[t], want, rtol=1e-12)
    others = np.delete(np.arange(case.M), t)
    assert not slack[others].any()
