"""Parity of the split-K decode forward (stage 1's contraction over D split
across two workgroups per unit, fp32 halves merged by the second to finish)
with the CPU oracle, through the C ABI on an MI355X: h and the requant codes
per route (bit-exact requant of its own h), the output within the end-to-end
tolerance; repeated calls on one workspace (the part counters return to zero,
the bits repeat)."""
import numpy as np
import pytest
import torch

from tests.moe_cases import custom_case, log, workload_case
from tests.test_gpu_parity import _check_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding(gpu_device):
    from mixture_experts_mxfp4_amd import binding as b
    return b


def _run(binding, case, workspace=None):
    d = case.device_inputs()
    r = binding.moe_mxfp4_forward_splitk_debug(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                               workspace=workspace)
    torch.cuda.synchronize()
    R = case.M * case.topk
    ids = case.ids.reshape(-1)
    ok = (ids >= 0) & (ids < case.E)
    return {"out": r["out"], "h": r["h"], "a2_codes": r["a2_codes"], "a2_scales": r["a2_scales"],
            "sorted_route": torch.from_numpy(np.where(ok, np.arange(R), R).astype(np.int32)),
            "num_valid": torch.tensor([R, int(ok.sum())], dtype=torch.int32),
            "block_m": 16, "path": binding.PATH_DIRECT}


def test_splitk_decode_workload(binding):
    case = workload_case("decode")
    _check_forward(case, _run(binding, case), "split-K decode (all tokens)")


@pytest.mark.parametrize("M,D,I,E,n_routed,seed", [
    (1, 512, 256, 9, 2, 81),           # single token
    (32, 512, 256, 65, 8, 82),         # two row tiles in stage 2; 17-32 routes on the shared expert
    (20, 512, 256, 130, 15, 83),       # 16 slots per token
    (13, 768, 768, 5, 3, 84),          # K = D = 768: 6 K tiles, 3 per part (odd split over waves)
    (16, 7168, 2048, 33, 8, 85),       # the E=33, I=2048 expert set at 16 tokens
])
def test_splitk_shapes(binding, M, D, I, E, n_routed, seed):
    case = custom_case(M, D, I, E, n_routed, seed)
    _check_forward(case, _run(binding, case), f"split-K M={M} D={D} I={I} E={E} topk={n_routed + 1}")


def test_splitk_invalid_and_duplicate_ids(binding):
    M, D, I, E = 12, 512, 256, 40
    rng = np.random.default_rng(8)
    ids = rng.integers(0, E, (M, 5)).astype(np.int32)
    ids[:, 1] = ids[:, 0]
    ids[::2, 3] = -1
    ids[1::4, 4] = E + 2
    tw = rng.random((M, 5)).astype(np.float32)
    case = custom_case(M, D, I, E, 2, 86, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    _check_forward(case, _run(binding, case), "split-K invalid/duplicate ids")


def test_splitk_repeated_calls(binding):
    """Five calls on one workspace: identical bits, every part counter back at zero."""
    case = workload_case("decode")
    d = case.device_inputs()
    ws = binding.alloc_workspace_splitk(case.M, case.D, case.I, case.E, case.topk)
    outs = []
    for _ in range(5):
        out = binding.moe_mxfp4_forward_splitk(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                               workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().view(torch.int16).numpy().copy())
    n_ctr = min(case.E, case.M * case.topk) * (case.I // 64)
    ctr = ws[: 4 * n_ctr].view(torch.int32).cpu().numpy()
    log(f"split-K: {n_ctr} part counters after five calls, nonzero: {int(np.count_nonzero(ctr))}")
    assert not ctr.any()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
