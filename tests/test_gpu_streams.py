"""Forwards in flight together on several streams (default priority), each
with its own workspace: the library keeps no per-call state outside the
caller's workspace and output, so every result equals its eager forward on
the current stream bit for bit (the forward is deterministic)."""
import pytest
import torch

from tests.moe_cases import custom_case, log, workload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding(gpu_device):
    from mixture_experts_mxfp4_amd import binding as b
    return b


def _bits(t):
    return t.view(torch.int16)


def _eager(binding, d, hidden):
    M, D = hidden.shape
    out = torch.empty_like(hidden)
    binding.moe_mxfp4_forward(hidden, *d["prepared"], d["ids"], d["tw"], out=out)
    torch.cuda.synchronize()
    return out


def test_forwards_of_three_paths_on_three_streams(binding):
    cases = [workload_case("decode"), workload_case("small_batch", M=40),
             custom_case(1400, 512, 256, 5, 2, 25)]
    runs = []
    for c in cases:
        d = c.device_inputs()
        path = binding.PATH_NAMES[binding.moe_mxfp4_path(c.M, c.D, c.I, c.E, c.topk)]
        log(f"streams: M={c.M} D={c.D} I={c.I} E={c.E} topk={c.topk} path {path}")
        ref = _eager(binding, d, d["hidden"])
        ws = binding.alloc_workspace(c.M, c.D, c.I, c.E, c.topk)
        outs = [torch.full_like(d["hidden"], float("nan")) for _ in range(4)]
        runs.append((d, ref, ws, outs))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    # interleave the launches: the streams' forwards overlap on the device
    for rep in range(4):
        for (d, ref, ws, outs), s in zip(runs, streams):
            with torch.cuda.stream(s):
                binding.moe_mxfp4_forward(d["hidden"], *d["prepared"], d["ids"], d["tw"],
                                          out=outs[rep], workspace=ws, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for i, (d, ref, ws, outs) in enumerate(runs):
        for rep, o in enumerate(outs):
            assert torch.equal(_bits(o), _bits(ref)), f"case {i} repeat {rep}"


def test_same_shape_on_two_streams_different_inputs(binding):
    c = workload_case("prefill")
    d = c.device_inputs()
    gen = torch.Generator().manual_seed(7)
    h2 = torch.randn(d["hidden"].shape, generator=gen).to(torch.bfloat16).cuda()
    log(f"streams: two prefill forwards (M={c.M}, E={c.E}) with different activations")
    ref1 = _eager(binding, d, d["hidden"])
    ref2 = _eager(binding, d, h2)
    assert not torch.equal(_bits(ref1), _bits(ref2))
    ws = [binding.alloc_workspace(c.M, c.D, c.I, c.E, c.topk) for _ in range(2)]
    outs = [torch.full_like(d["hidden"], float("nan")) for _ in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for j, (h, s) in enumerate(zip((d["hidden"], h2), streams)):
            with torch.cuda.stream(s):
                binding.moe_mxfp4_forward(h, *d["prepared"], d["ids"], d["tw"], out=outs[j],
                                          workspace=ws[j], stream=s.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(_bits(outs[0]), _bits(ref1))
    assert torch.equal(_bits(outs[1]), _bits(ref2))
