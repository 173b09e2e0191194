"""The seeded synthetic inputs (mixture_experts_mxfp4_amd/inputs.py), on the CPU:
the recipe the workloads are stated with, reproducible from the seed."""
import numpy as np
import torch

from mixture_experts_mxfp4_amd import inputs


def test_activations_are_reproducible_and_shaped():
    a = inputs.make_activations(12, 256, 9, 2, "uniform", 5)
    b = inputs.make_activations(12, 256, 9, 2, "uniform", 5)
    c = inputs.make_activations(12, 256, 9, 2, "uniform", 6)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    hidden, ids, tw = a
    assert hidden.shape == (12, 256) and hidden.dtype == torch.bfloat16
    assert ids.shape == (12, 3) and ids.dtype == torch.int32
    assert tw.shape == (12, 3) and tw.dtype == torch.float32


def test_routing_recipe():
    """Routed ids distinct per token from 0..E-2, softmax weights summing to
    one over the routed slots, the shared expert E-1 last with weight 1."""
    for routing in ("uniform", "zipf"):
        _, ids, tw = inputs.make_activations(200, 256, 33, 8, routing, 3)
        ids, tw = ids.numpy(), tw.numpy()
        assert np.all(ids[:, -1] == 32) and np.all(tw[:, -1] == 1.0)
        routed = ids[:, :-1]
        assert routed.min() >= 0 and routed.max() <= 31
        assert all(len(set(r)) == 8 for r in routed)
        assert np.allclose(tw[:, :-1].sum(axis=1), 1.0, atol=1e-5)
        assert np.all(tw[:, :-1] > 0)


def test_zipf_routing_is_skewed_and_uniform_is_not():
    """Zipf(1.1) over the routed ids: the most popular expert is picked far more
    often than the median one; uniform routing keeps counts near the mean."""
    _, zi, _ = inputs.make_activations(1024, 256, 257, 8, "zipf", 3)
    _, un, _ = inputs.make_activations(1024, 256, 257, 8, "uniform", 3)
    cz = np.bincount(zi.numpy()[:, :-1].reshape(-1), minlength=256)
    cu = np.bincount(un.numpy()[:, :-1].reshape(-1), minlength=256)
    assert cz.sum() == cu.sum() == 1024 * 8
    assert cz.max() > 20 * max(np.median(cz), 1)
    assert cu.max() < 3 * cu.mean()


def test_weights_scale_with_the_contraction_length():
    """N(0, 1/K) entries (std 1/sqrt(K)) for both projections, seeded."""
    w13, w2 = inputs.make_weights(3, 1024, 256, 7)
    assert w13.shape == (3, 512, 1024) and w2.shape == (3, 1024, 256)
    s13 = float(w13.float().std())
    s2 = float(w2.float().std())
    assert abs(s13 * np.sqrt(1024) - 1) < 0.05
    assert abs(s2 * np.sqrt(256) - 1) < 0.05
    w13b, _ = inputs.make_weights(3, 1024, 256, 7)
    assert torch.equal(w13, w13b)
