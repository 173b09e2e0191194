"""The forward that allocates nothing (moe_mxfp4_forward_noalloc, through the
C ABI) against the forward with a caller's workspace, on an MI355X: identical
bits on two calls in a row on the same device, the second with a smaller
input (its scratch array then still holds the first call's intermediates),
and a shape whose workspace exceeds the array refused with the workspace
status.  The forward is deterministic, so equality is bit for bit."""
import numpy as np
import pytest
import torch

from mixture_experts_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _prepared(binding, w, dev):
    w13f, w2f = inputs.make_weights(w.E, w.D, w.I, w.seed, device=dev)
    c13, s13 = binding.moe_mxfp4_quantize(w13f.reshape(-1, w.D))
    c2, s2 = binding.moe_mxfp4_quantize(w2f.reshape(-1, w.I))
    return binding.moe_mxfp4_prepare_weights(
        c13.view(w.E, 2 * w.I, w.D // 2), s13.view(w.E, 2 * w.I, w.D // 32),
        c2.view(w.E, w.D, w.I // 2), s2.view(w.E, w.D, w.I // 32))


def test_noalloc_matches_forward_two_calls(gpu_device):
    from mixture_experts_mxfp4_amd import binding
    w = inputs.WORKLOADS["small_batch"]          # D=7168, I=2048, E=33, top-9
    dev = gpu_device
    prep = _prepared(binding, w, dev)
    results = []
    for M in (64, 16):                           # sorted streaming path, then route-indexed path
        hidden, ids, tw = inputs.make_activations(M, w.D, w.E, w.n_routed, w.routing, 100 + M)
        h, i, t = hidden.to(dev), ids.to(dev), tw.to(dev)
        path = binding.moe_mxfp4_path(M, w.D, w.I, w.E, w.topk)
        assert binding.moe_mxfp4_workspace_bytes(M, w.D, w.I, w.E, w.topk) <= \
            binding.NOALLOC_SCRATCH_BYTES
        out_na = binding.moe_mxfp4_forward_noalloc(h, *prep, i, t)
        torch.cuda.synchronize()
        ref = binding.moe_mxfp4_forward(h, *prep, i, t)
        torch.cuda.synchronize()
        a, b = _bits(out_na), _bits(ref)
        print(f"[moe-test] noalloc M={M} path={binding.PATH_NAMES[path]}: "
              f"{int(np.count_nonzero(a != b))} of {a.size} elements differ", flush=True)
        assert np.isfinite(out_na.float().cpu().numpy()).all()
        assert np.array_equal(a, b)
        results.append(path)
    assert results == [binding.PATH_STREAM, binding.PATH_DIRECT]


def test_noalloc_refuses_shapes_beyond_its_scratch(gpu_device):
    from mixture_experts_mxfp4_amd import binding
    M, D, I, E, k = 1024, 7168, 256, 257, 9
    assert binding.moe_mxfp4_workspace_bytes(M, D, I, E, k) > binding.NOALLOC_SCRATCH_BYTES
    u8 = torch.uint8
    w = [torch.zeros(s, dtype=u8, device=gpu_device)
         for s in ((E, 2 * I, D // 2), (E, 2 * I, D // 32), (E, D, I // 2), (E, D, I // 32))]
    h = torch.zeros((M, D), dtype=torch.bfloat16, device=gpu_device)
    ids = torch.zeros((M, k), dtype=torch.int32, device=gpu_device)
    tw = torch.zeros((M, k), dtype=torch.float32, device=gpu_device)
    with pytest.raises(binding.MoeMxfp4Error) as err:
        binding.moe_mxfp4_forward_noalloc(h, *w, ids, tw)
    assert err.value.status == 3
