"""Seeded synthetic inputs for the fused MXFP4 MoE forward.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantization, no GEMM).  Both the HIP path and the CPU oracle
take their inputs from here; each side quantizes the float weights with its
own code.

Workloads (DeepSeek-R1-shaped routed-expert block, D = 7168, top-9 with the
shared expert in the last slot, as in the self-test generator of kernelindex
submission 723815 and the shapes of submission 754773's tuning table):

  tiny           M=8,    D=512,  I=256,  E=9,   2 routed of 0..7   + shared 8
  decode         M=16,   D=7168, I=256,  E=257, 8 routed of 0..255 + shared 256
  small_batch    M=64,   D=7168, I=2048, E=33,  8 routed of 0..31  + shared 32
  prefill        M=1024, D=7168, I=256,  E=257, 8 routed Zipf(1.1) + shared 256
  large_prefill  M=4096, D=7168, I=2048, E=33,  8 routed of 0..31  + shared 32

Recipe: hidden bf16 N(0,1); gate_up weight [E, 2I, D] and down weight [E, D, I]
bf16 N(0, 1/sqrt(K)) with K the contraction length (D for gate_up, I for down);
routed ids distinct per token; routed weights softmax of N(0,1) over the routed
slots; shared expert E-1 with weight 1.0 in the last slot.
"""
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    D: int
    I: int
    E: int
    n_routed: int      # routed slots per token; topk = n_routed + 1 (shared)
    routing: str       # "uniform" or "zipf"
    seed: int

    @property
    def topk(self) -> int:
        return self.n_routed + 1


WORKLOADS = {
    "tiny": Workload("tiny", 8, 512, 256, 9, 2, "uniform", 0),
    "decode": Workload("decode", 16, 7168, 256, 257, 8, "uniform", 1),
    "small_batch": Workload("small_batch", 64, 7168, 2048, 33, 8, "uniform", 2),
    "prefill": Workload("prefill", 1024, 7168, 256, 257, 8, "zipf", 3),
    "large_prefill": Workload("large_prefill", 4096, 7168, 2048, 33, 8, "uniform", 4),
}

ZIPF_S = 1.1


def make_routing(M, E, n_routed, routing, gen):
    """Routed ids (distinct per token) from 0..E-2, softmax(N(0,1)) weights,
    and the shared expert E-1 with weight 1.0 in the last slot."""
    n_choices = E - 1
    if n_routed > n_choices:
        raise ValueError("more routed slots than routed experts")
    if routing == "uniform":
        keys = torch.rand(M, n_choices, generator=gen)
        routed = torch.argsort(keys, dim=1)[:, :n_routed]
    elif routing == "zipf":
        p = torch.arange(1, n_choices + 1, dtype=torch.float64).pow(-ZIPF_S)
        p = (p / p.sum()).expand(M, n_choices).contiguous()
        routed = torch.multinomial(p, n_routed, replacement=False, generator=gen)
    else:
        raise ValueError(routing)
    logits = torch.randn(M, n_routed, generator=gen)
    w = torch.softmax(logits, dim=1)
    ids = torch.cat([routed.to(torch.int32),
                     torch.full((M, 1), E - 1, dtype=torch.int32)], dim=1)
    tw = torch.cat([w.to(torch.float32), torch.ones(M, 1, dtype=torch.float32)], dim=1)
    return ids.contiguous(), tw.contiguous()


def make_weights(E, D, I, seed, device="cpu", chunk=8):
    """Float weights, bf16: gate_up [E, 2I, D] ~ N(0, 1/D), down [E, D, I] ~ N(0, 1/I).
    Drawn expert-chunk by expert-chunk on `device` with a generator seeded by
    `seed`; the stream (hence the values) depends on the device."""
    gen = torch.Generator(device=device).manual_seed(seed * 7919 + 17)
    w13 = torch.empty((E, 2 * I, D), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((E, D, I), dtype=torch.bfloat16, device=device)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        w13[e0:e1] = (torch.randn((e1 - e0, 2 * I, D), generator=gen, device=device)
                      * (1.0 / np.sqrt(D))).to(torch.bfloat16)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        w2[e0:e1] = (torch.randn((e1 - e0, D, I), generator=gen, device=device)
                     * (1.0 / np.sqrt(I))).to(torch.bfloat16)
    return w13, w2


def make_activations(M, D, E, n_routed, routing, seed):
    """hidden bf16 [M, D] ~ N(0,1) and the routing, all from one CPU generator."""
    gen = torch.Generator().manual_seed(seed)
    hidden = torch.randn((M, D), generator=gen).to(torch.bfloat16)
    ids, tw = make_routing(M, E, n_routed, routing, gen)
    return hidden, ids, tw


def make_case(w: Workload, weight_device="cpu", M=None):
    """All float inputs of a workload (optionally with a different token count)."""
    M = w.M if M is None else M
    hidden, ids, tw = make_activations(M, w.D, w.E, w.n_routed, w.routing, w.seed)
    w13, w2 = make_weights(w.E, w.D, w.I, w.seed, device=weight_device)
    return {"hidden": hidden, "ids": ids, "tw": tw, "w13": w13, "w2": w2}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw bit patterns of a bf16 tensor as numpy uint16 (CPU copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16)
