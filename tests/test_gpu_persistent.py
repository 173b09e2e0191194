"""Parity of the persistent (single-launch) decode forward with the CPU oracle,
through the C ABI on an MI355X: the route list it implies, h and the requant
codes per route (bit-exact requant of its own h), and the output within the
end-to-end tolerance; repeated calls on one workspace (the grid barrier's
words return to zero, the error word stays zero, the bits repeat)."""
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
    r = binding.moe_mxfp4_forward_persistent_debug(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                                   workspace=workspace)
    torch.cuda.synchronize()
    R = case.M * case.topk
    ids = case.ids.reshape(-1)
    ok = (ids >= 0) & (ids < case.E)
    dbg = {"out": r["out"], "h": r["h"], "a2_codes": r["a2_codes"], "a2_scales": r["a2_scales"],
           "sorted_route": torch.from_numpy(np.where(ok, np.arange(R), R).astype(np.int32)),
           "num_valid": torch.tensor([R, int(ok.sum())], dtype=torch.int32),
           "block_m": 16, "path": binding.PATH_DIRECT}
    assert binding.persistent_error_word(r["workspace"]) == 0
    return dbg, r["workspace"]


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_persistent_decode_workload(binding):
    case = workload_case("decode")
    log(f"persistent decode: {binding.moe_mxfp4_persistent_workgroups(case.M)} workgroups")
    dbg, _ = _run(binding, case)
    _check_forward(case, dbg, "persistent decode (all tokens)")


@pytest.mark.parametrize("M,D,I,E,n_routed,seed", [
    (1, 512, 256, 9, 2, 71),           # single token
    (32, 512, 256, 65, 8, 72),         # 17-32 tokens: two row tiles
    (20, 512, 256, 130, 15, 73),       # 16 slots per token
    (13, 768, 768, 5, 3, 74),          # D and I not multiples of 512, few experts
    (3, 256, 256, 2, 1, 75),           # smallest dims
    (16, 7168, 2048, 33, 8, 76),       # the E=33, I=2048 expert set at 16 tokens
])
def test_persistent_shapes(binding, M, D, I, E, n_routed, seed):
    case = custom_case(M, D, I, E, n_routed, seed)
    dbg, _ = _run(binding, case)
    _check_forward(case, dbg, f"persistent M={M} D={D} I={I} E={E} topk={n_routed + 1}")


def test_persistent_invalid_and_duplicate_ids(binding):
    """A token naming one expert in several slots (further route-table
    layers), ids outside [0, E)."""
    M, D, I, E = 12, 512, 256, 40
    rng = np.random.default_rng(7)
    ids = rng.integers(0, E, (M, 5)).astype(np.int32)
    ids[:, 1] = ids[:, 0]
    ids[::3, 2] = ids[::3, 0]          # three slots of one expert
    ids[::2, 3] = -1
    ids[1::4, 4] = E + 2
    tw = rng.random((M, 5)).astype(np.float32)
    case = custom_case(M, D, I, E, 2, 77, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    dbg, _ = _run(binding, case)
    _check_forward(case, dbg, "persistent invalid/duplicate ids")


def test_persistent_repeated_calls(binding):
    """The barrier words return to zero after each call: five calls on one
    workspace give identical bits and leave the error word at zero."""
    case = workload_case("decode")
    d = case.device_inputs()
    ws = binding.alloc_workspace_persistent(case.M, case.D, case.I, case.E, case.topk)
    outs = []
    for _ in range(5):
        out = binding.moe_mxfp4_forward_persistent(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                                   workspace=ws)
        torch.cuda.synchronize()
        outs.append(_bits(out))
    words = ws[:2048].view(torch.int32).cpu().numpy()
    log(f"barrier generation and error word after five calls: {words[:2].tolist()}")
    assert words[0] == 5 and words[1] == 0
    counts = words[4 + 32 * np.arange(9)]      # the nine arrival counts, one per 128-byte line
    assert not counts.any(), counts
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_persistent_no_valid_routes(binding):
    M, D, I, E = 4, 512, 256, 3
    ids = np.full((M, 2), -1, np.int32)
    tw = np.ones((M, 2), np.float32)
    case = custom_case(M, D, I, E, 1, 78, ids=torch.from_numpy(ids), tw=torch.from_numpy(tw))
    d = case.device_inputs()
    out = binding.moe_mxfp4_forward_persistent(d["hidden"], *d["prepared"], d["ids"], d["tw"])
    torch.cuda.synchronize()
    assert torch.all(out.cpu().float() == 0)


def test_persistent_unsupported_shape(binding):
    case = custom_case(40, 512, 256, 9, 2, 79)
    assert binding.moe_mxfp4_persistent_workspace_bytes(40, 512, 256, 9, 3) == 0
    d = case.device_inputs()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.MoeMxfp4Error) as err:
        binding.moe_mxfp4_forward_persistent(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                             workspace=ws)
    assert err.value.status == 2
