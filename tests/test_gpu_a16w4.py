"""Parity of the A16W4 forward (bf16 activations, MXFP4 weights, no
activation quantization) with the CPU oracle's act_quant=off mode, through the
C ABI on an MI355X.

Same end-to-end tolerance as the MXFP4 forward (check_close).  h per route
against the oracle's h: within 2^-6 relative + 1e-3 rms, and at least 95 % of
the elements bit-identical (fp32 vs fp64 accumulation and the hardware exp2 /
reciprocal of silu move an occasional bf16 rounding by one unit).
"""
import numpy as np
import pytest
import torch

from mixture_experts_mxfp4_amd import inputs
from tests.moe_cases import bf16_to_f64, check_close, custom_case, log, workload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding(gpu_device):
    from mixture_experts_mxfp4_amd import binding as b
    return b


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check_h(case, h_gpu_rows):
    R = case.M * case.topk
    ok = (case.ids.reshape(-1) >= 0) & (case.ids.reshape(-1) < case.E)
    valid = np.nonzero(ok)[0]
    _, h_or = case.run_oracle(act_quant=False, want_h=True)
    g = bf16_to_f64(_bits(h_gpu_rows)[:R][valid])
    o = bf16_to_f64(h_or.reshape(R, case.I)[valid])
    rms = float(np.sqrt(np.mean(o * o)))
    assert np.all(np.abs(g - o) <= 2.0 ** -6 * np.abs(o) + 1e-3 * rms)
    exact = float(np.mean(g == o))
    log(f"a16w4 h exact-bits fraction {exact:.4f}")
    assert exact >= 0.95


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_a16w4_workload_full_and_h(binding, name):
    case = workload_case(name)
    log(f"a16w4 {name}: M={case.M} D={case.D} I={case.I} E={case.E} topk={case.topk}")
    dbg = case.run_gpu_a16w4(debug=True)
    check_close(_bits(dbg["out"]), case.run_oracle(act_quant=False), f"a16w4 {name}")
    _check_h(case, dbg["h"])


def test_a16w4_e33_sixteen_tokens_sampled(binding):
    """16 tokens on the E=33, I=2048 expert set (D=7168), 5 tokens checked."""
    w = inputs.WORKLOADS["small_batch"]
    case = workload_case("small_batch", M=16)
    out = _bits(case.run_gpu_a16w4())
    toks = np.array([0, 3, 7, 12, 15])
    log(f"a16w4 E={w.E} I={w.I} M=16: oracle on {toks.size} tokens")
    check_close(out[toks], case.run_oracle(tokens=toks, act_quant=False), "a16w4 E=33 M=16")


@pytest.mark.parametrize("M,D,I,E,n_routed,seed", [
    (1, 512, 256, 9, 2, 61),          # single token
    (32, 512, 256, 65, 8, 62),        # two row tiles in stage 2, shared expert over both
    (13, 768, 768, 5, 3, 63),         # ragged M, D and I not multiples of 512
    (3, 256, 256, 2, 1, 64),          # smallest dims
    (24, 256, 256, 1024, 8, 65),      # largest E
    (20, 512, 256, 9, 1, 69),         # two row tiles with h staged in LDS (40 routes, 20 KB)
])
def test_a16w4_shapes(binding, M, D, I, E, n_routed, seed):
    log(f"a16w4 shape M={M} D={D} I={I} E={E} topk={n_routed + 1}")
    case = custom_case(M, D, I, E, n_routed, seed)
    dbg = case.run_gpu_a16w4(debug=True)
    check_close(_bits(dbg["out"]), case.run_oracle(act_quant=False), f"a16w4 M={M} D={D} I={I}")
    _check_h(case, dbg["h"])


def test_a16w4_invalid_and_duplicate_ids(binding):
    """Invalid ids contribute nothing; a token naming one expert in several
    slots counts once per slot (stage 2's extra layers)."""
    M, E, D, I = 8, 40, 512, 256
    rng = np.random.default_rng(7)
    ids = rng.integers(0, E, (M, 5)).astype(np.int32)
    ids[:, 1] = ids[:, 0]
    ids[::3, 4] = ids[::3, 0]        # three slots on one expert
    ids[::2, 2] = -1
    ids[1::4, 3] = E + 3
    tw = rng.random((M, 5)).astype(np.float32)
    case = custom_case(M, D, I, E, 2, 66, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    check_close(_bits(case.run_gpu_a16w4()), case.run_oracle(act_quant=False),
                "a16w4 invalid/duplicate ids")


def test_a16w4_no_valid_routes_and_m_zero(binding):
    M, D, I, E = 4, 512, 256, 3
    ids = np.full((M, 2), -1, np.int32)
    case = custom_case(M, D, I, E, 1, 67, ids=torch.from_numpy(ids),
                       tw=torch.ones((M, 2), dtype=torch.float32))
    assert torch.all(case.run_gpu_a16w4().cpu().float() == 0)
    d = case.device_inputs()
    h0 = torch.zeros((0, D), dtype=torch.bfloat16, device="cuda")
    out = binding.moe_mxfp4_forward_a16w4(
        h0, *d["prepared"], torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
        torch.zeros((0, 2), dtype=torch.float32, device="cuda"),
        workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert out.shape == (0, D)


def test_a16w4_unsupported_shape_is_an_error(binding):
    case = custom_case(33, 512, 256, 9, 2, 68)
    d = case.device_inputs()
    with pytest.raises(binding.MoeMxfp4Error) as e:
        binding.moe_mxfp4_forward_a16w4(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                        workspace=torch.empty(1 << 20, dtype=torch.uint8,
                                                              device="cuda"))
    assert e.value.status == 2


def test_a16w4_deterministic_and_debug_matches(binding):
    """Two calls give identical bits; the timed/debug call gives the same
    bits and records its two launches and every stage-1 workgroup span."""
    import bench
    case = workload_case("decode")
    a = case.run_gpu_a16w4()
    b = case.run_gpu_a16w4()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    d = case.device_inputs()
    ev = bench.Events(8)
    n_wg = binding.a16w4_stage1_workgroups(case.M, case.I, case.E, case.topk)
    span = torch.zeros(2 * n_wg, dtype=torch.int64, device="cuda")
    r = binding.moe_mxfp4_forward_a16w4_debug(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                              kernel_events=ev.ev, stage1_clock=span)
    torch.cuda.synchronize()
    assert torch.equal(r["out"].view(torch.int16), a.view(torch.int16))
    rec = span.cpu().reshape(-1, 2)
    assert bool((rec > 0).all()) and bool((rec[:, 1] >= rec[:, 0]).all())
    for i in (1, 2):
        ms = ev.ms(2 * i, 2 * i + 1)
        log(f"a16w4 decode launch {binding.LAUNCHES[i]}: {1000 * ms:.2f} us")
        assert ms > 0.0
    ev.close()
