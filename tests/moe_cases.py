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


def requant_slack(case, dbg):
    """Output slack explained by requant codes that differ from the oracle's.

    Stage 1 accumulates in fp32 and the oracle in fp64, so a bf16 h may differ
    by an ulp; where that ulp straddles a rounding midpoint of the E2M1 grid
    (or a power of two of the block maximum) the requantized code moves by a
    whole grid step, up to a third of the block maximum.  Both codes are the
    correct quantization of their own h (the GPU's is checked bit for bit
    against the oracle quantizer applied to the GPU h, and the GPU h against
    the oracle's h, in _check_intermediates), so the output may differ from the
    oracle's by what the step carries through stage 2:
    slack[t, d] = sum over the token's routes of |w| * sum_i |dv_i| * |W2[e][d, i]|,
    dv the difference of the dequantized codes.  Returns (slack [M, D] or None,
    number of differing h elements, number of h elements)."""
    sr = dbg["sorted_route"].cpu().numpy()
    n = int(dbg["num_valid"].cpu().numpy()[0])
    R = case.M * case.topk
    rows = np.nonzero(sr[:n] < R)[0]
    r = sr[rows]
    if rows.size == 0:
        return None, 0, 0
    t, s = r // case.topk, r % case.topk
    _, h_or = case.run_oracle(want_h=True)
    oc, os_ = oracle.quantize_rows(h_or[t, s])
    gc = dbg["a2_codes"].cpu().numpy()[rows]
    gs = dbg["a2_scales"].cpu().numpy()[rows]
    dv = np.abs(oracle.dequantize_rows(gc, gs) - oracle.dequantize_rows(oc, os_))
    moved = np.nonzero(dv.max(axis=1) > 0)[0]
    if moved.size == 0:
        return None, 0, dv.size
    slack = np.zeros((case.M, case.D))
    experts = case.ids[t[moved], s[moved]]
    for e in np.unique(experts):
        w2 = np.abs(oracle.dequantize_rows(case.wq[2][e], case.wq[3][e]))    # [D, I]
        for j in moved[experts == e]:
            slack[t[j]] += abs(float(case.tw[t[j], s[j]])) * (w2 @ dv[j])
    return slack, int(np.count_nonzero(dv)), dv.size


def check_close(gpu_bits, oracle_bits, what="", slack=None):
    """The end-to-end tolerance: |gpu - oracle| <= 2e-2 * rms(oracle) + 2^-7 * |oracle|
    on >= 99.9% of the elements, and no element beyond 0.1 * rms(oracle); with
    `slack` (requant_slack), each element's bound grows by its slack."""
    g = bf16_to_f64(gpu_bits)
    o = bf16_to_f64(oracle_bits)
    assert g.shape == o.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    rms = float(np.sqrt(np.mean(o * o)))
    err = np.abs(g - o)
    extra = 0.0 if slack is None else slack
    bound = 2e-2 * rms + 2.0 ** -7 * np.abs(o) + extra
    frac = float(np.mean(err <= bound))
    over = err - extra
    worst = float(over.max()) if err.size else 0.0
    log(f"{what}: rms={rms:.4g} within-bound={frac * 100:.4f}% worst={worst / max(rms, 1e-30):.4g}*rms "
        f"exact-bf16={float(np.mean(g == o)) * 100:.2f}%"
        + ("" if slack is None else f" slack on {int(np.count_nonzero(slack.max(axis=1)))} tokens"))
    assert frac >= 0.999, f"{what}: only {frac:.5f} of elements within tolerance"
    assert worst <= 0.1 * rms, f"{what}: worst error {worst} > 0.1*rms ({rms})"
    return frac, worst / max(rms, 1e-30)
