"""The forward under HIP graph capture (torch.cuda.graph over the C ABI).

The forward enqueues kernel launches only (no allocation, memset, copy or
host synchronization), so it can be captured once and replayed.  Each case
replays three times with eager work and a synchronization between replays;
every replay must equal the eager forward bit for bit (the forward is
deterministic), and a replay after new inputs are copied into the captured
buffers must equal the eager forward on those inputs.
"""
import pytest
import torch

from tests.moe_cases import custom_case, log, workload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding(gpu_device):
    from mixture_experts_mxfp4_amd import binding as b
    return b


def _case(kind):
    if kind == "decode":
        return workload_case("decode")
    if kind == "small_batch":
        return workload_case("small_batch", M=40)
    if kind == "prefill":
        return workload_case("prefill")                 # paired 32-row blocks, chunked sort
    return custom_case(1400, 512, 256, 5, 2, 25)       # LDS-tiled path


@pytest.mark.parametrize("kind,a16", [("decode", False), ("decode", True), ("small_batch", False),
                                      ("prefill", False), ("tiled", False)])
def test_forward_graph_replay(binding, kind, a16):
    case = _case(kind)
    d = case.device_inputs()
    M, D, I, E, k = case.M, case.D, case.I, case.E, case.topk
    path = "a16w4" if a16 else binding.PATH_NAMES[binding.moe_mxfp4_path(M, D, I, E, k)]
    log(f"graph capture: {kind} M={M} path {path}")
    fwd = binding.moe_mxfp4_forward_a16w4 if a16 else binding.moe_mxfp4_forward
    alloc = binding.alloc_workspace_a16w4 if a16 else binding.alloc_workspace
    ws = alloc(M, D, I, E, k)
    hidden = d["hidden"].clone()
    out = torch.empty_like(hidden)

    def run(h, o, w):
        fwd(h, *d["prepared"], d["ids"], d["tw"], out=o, workspace=w)

    run(hidden, out, ws)                       # eager (also the first call on the device)
    torch.cuda.synchronize()
    ref = out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(hidden, out, ws)
    for rep in range(3):
        out.fill_(0)                           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"

    # new activations in the captured buffer: the replay reads them
    gen = torch.Generator().manual_seed(99)
    new_h = torch.randn(hidden.shape, generator=gen).to(torch.bfloat16).cuda()
    ref2 = torch.empty_like(out)
    run(new_h, ref2, alloc(M, D, I, E, k))
    hidden.copy_(new_h)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref2.view(torch.int16))
    assert not torch.equal(ref2.view(torch.int16), ref.view(torch.int16))
