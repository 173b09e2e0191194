"""Builds parity cases for the GPU tests (test code).

Float inputs come from mixture_experts_mxfp4_amd.inputs; the MXFP4 weights fed
to BOTH sides are quantized by the CPU oracle, so the HIP path and the oracle
run on identical codes and scales.  Nothing here feeds a HIP result to the
oracle.
"""
import sys

import numpy as np
import torch

import oracle
from mixture_experts_mxfp4_amd import inputs


def log(msg):
    print(f"[moe-test] {msg}", flush=True)
    sys.stdout.flush()


def oracle_quant_weights(w13f, w2f):
    """bf16 float weights (any device) -> oracle MXFP4 codes/scales as numpy."""
    E, twoI, D = w13f.shape
    I = twoI // 2
    w13, w13s = oracle.quantize_rows(inputs.bf16_bits(w13f).reshape(E * twoI, D))
    w2, w2s = oracle.quantize_rows(inputs.bf16_bits(w2f).reshape(E * D, I))
    return (w13.reshape(E, twoI, D // 2), w13s.reshape(E, twoI, D // 32),
            w2.reshape(E, D, I // 2), w2s.reshape(E, D, I // 32))


class Case:
    """One parity case: host numpy arrays for the oracle, device tensors for HIP."""

    def __init__(self, hidden, ids, tw, w13f, w2f, device="cuda"):
        self.hidden_t = hidden.contiguous()
        self.ids_t = ids.contiguous()
        self.tw_t = tw.contiguous()
        self.M, self.D = hidden.shape
        self.E, twoI, _ = w13f.shape
        self.I = twoI // 2
        self.topk = ids.shape[1]
        self.hb = inputs.bf16_bits(hidden)
        self.ids = ids.numpy()
        self.tw = tw.numpy()
        self.wq = oracle_quant_weights(w13f, w2f)
        self.device = device
        self._dev = None

    def device_inputs(self):
        if self._dev is None:
            from mixture_experts_mxfp4_amd import binding
            dev = self.device
            raw = [torch.from_numpy(a).to(dev) for a in self.wq]
            prepared = binding.moe_mxfp4_prepare_weights(*raw)
            self._dev = {
                "hidden": self.hidden_t.to(dev),
                "ids": self.ids_t.to(dev),
                "tw": self.tw_t.to(dev),
                "raw": raw,
                "prepared": prepared,
            }
        return self._dev

    def run_gpu(self, debug=False):
        from mixture_experts_mxfp4_amd import binding
        d = self.device_inputs()
        if debug:
            r = binding.moe_mxfp4_forward_debug(d["hidden"], *d["prepared"], d["ids"], d["tw"])
            torch.cuda.synchronize()
            return r
        out = binding.moe_mxfp4_forward(d["hidden"], *d["prepared"], d["ids"], d["tw"])
        torch.cuda.synchronize()
        return out

    def run_gpu_a16w4(self, debug=False):
        """The A16W4 forward (bf16 activations); with debug, dict(out, h)."""
        from mixture_experts_mxfp4_amd import binding
        d = self.device_inputs()
        if debug:
            r = binding.moe_mxfp4_forward_a16w4_debug(d["hidden"], *d["prepared"], d["ids"],
                                                      d["tw"], h=True)
            torch.cuda.synchronize()
            return r
        out = binding.moe_mxfp4_forward_a16w4(d["hidden"], *d["prepared"], d["ids"], d["tw"])
        torch.cuda.synchronize()
        return out

    def run_oracle(self, tokens=None, **kw):
        return oracle.forward(self.hb, *self.wq, self.ids, self.tw, tokens=tokens, **kw)


def workload_case(name, device="cuda", M=None):
    w = inputs.WORKLOADS[name]
    log(f"building case {name} (M={M or w.M}, D={w.D}, I={w.I}, E={w.E}, topk={w.topk})")
    hidden, ids, tw = inputs.make_activations(M or w.M, w.D, w.E, w.n_routed, w.routing, w.seed)
    w13f, w2f = inputs.make_weights(w.E, w.D, w.I, w.seed, device=device)
    return Case(hidden, ids, tw, w13f, w2f, device)


def custom_case(M, D, I, E, n_routed, seed, routing="uniform", device="cuda", ids=None, tw=None):
    hidden, ids0, tw0 = inputs.make_activations(M, D, E, n_routed, routing, seed)
    w13f, w2f = inputs.make_weights(E, D, I, seed, device=device)
    return Case(hidden, ids0 if ids is None else ids, tw0 if tw is None else tw, w13f, w2f, device)


def bf16_to_f64(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def check_close(gpu_bits, oracle_bits, what=""):
    """The end-to-end tolerance: |gpu - oracle| <= 2e-2 * rms(oracle) + 2^-7 * |oracle|
    on >= 99.9% of the elements, and no element beyond 0.1 * rms(oracle)."""
    g = bf16_to_f64(gpu_bits)
    o = bf16_to_f64(oracle_bits)
    assert g.shape == o.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    rms = float(np.sqrt(np.mean(o * o)))
    err = np.abs(g - o)
    bound = 2e-2 * rms + 2.0 ** -7 * np.abs(o)
    frac = float(np.mean(err <= bound))
    worst = float(err.max()) if err.size else 0.0
    log(f"{what}: rms={rms:.4g} within-bound={frac * 100:.4f}% worst={worst / max(rms, 1e-30):.4g}*rms "
        f"exact-bf16={float(np.mean(g == o)) * 100:.2f}%")
    assert frac >= 0.999, f"{what}: only {frac:.5f} of elements within tolerance"
    assert worst <= 0.1 * rms, f"{what}: worst error {worst} > 0.1*rms ({rms})"
    return frac, worst / max(rms, 1e-30)
