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


def covering_tokens(ids, tw, E, block_m, must=()):
    """Tokens whose routes touch every part of the sorted route list that a
    kernel tiles differently: every used block, and in every 64-row group of
    a block (the whole block when block_m < 64) the first 16-row slice and the
    16-row slice holding the group's last route.  The list is the oracle's
    (oracle.route, the list the forward is checked against bit for bit);
    greedy set cover, then `must` added.  Returns sorted token indices."""
    M, topk = ids.shape
    R = M * topk
    rt = oracle.route(ids, tw, E, block_m)
    sr = rt["sorted_route"]
    n = int(rt["num_valid"][0])
    group = min(block_m, 64)
    cells = []
    for b0 in range(0, n, block_m):
        for g0 in range(b0, b0 + block_m, group):
            rows = sr[g0:g0 + group]
            valid = np.nonzero(rows < R)[0]
            if valid.size == 0:
                continue
            for sl in sorted({0, int(valid[-1]) // 16}):
                part = rows[sl * 16:(sl + 1) * 16]
                cells.append(set((part[part < R] // topk).tolist()))
    by_token = {}
    for c, toks in enumerate(cells):
        for t in toks:
            by_token.setdefault(t, []).append(c)
    covered = np.zeros(len(cells), bool)
    chosen = set(int(t) for t in must)
    for t in chosen:
        covered[by_token.get(t, [])] = True
    while not covered.all():
        best = max(by_token, key=lambda t: int(np.count_nonzero(~covered[by_token[t]])))
        chosen.add(best)
        covered[by_token[best]] = True
    return np.array(sorted(chosen), np.int64)


def bf16_to_f64(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# E2M1 magnitudes by the low three code bits (the OCP MX v1.0 FP4 table).
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _spacing(v):
    """Spacing of the E2M1 grid (in units of the block scale) around |v|."""
    a = np.abs(v)
    return np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))


def requant_moves(h_gpu, h_or, gc, gs, oc, os_):
    """Per-element |difference| of the dequantized requant codes of the GPU
    (gc, gs: its own h_gpu quantized) and of the oracle (oc, os_: the
    oracle's h_or quantized), rows [n, I]; h as bf16 bit patterns.

    Stage 1 accumulates in fp32 and the oracle in fp64, so a bf16 h may differ
    by an ulp, and where that ulp crosses a decision boundary of the MXFP4
    rounding the two codes differ although each is the exact quantization of
    its own h.  Exactly two such boundaries exist, and only differences they
    explain are accepted (anything else raises AssertionError):

    1. same scale byte, one element: the two magnitudes are adjacent E2M1
       grid points (or both zero: a sign-only change of a zero) and |h_gpu|
       and |h_or| lie on opposite sides of (or on) the midpoint between them;
       the element moves by one grid step;
    2. scale bytes one apart: the two block maxima lie on opposite sides of
       the power of two 4 * 2^(s_hi - 127) where the scale rule steps (the
       larger maximum with the larger byte); every element of the block then
       re-rounds on a grid of twice the spacing, which moves it by at most
       twice the local spacing of the coarser grid plus |h_gpu - h_or|.

    Returns dv [n, I] (float64, zero where the dequantized values agree)."""
    n, I = h_gpu.shape
    hg = bf16_to_f64(h_gpu).reshape(n, I // 32, 32)
    ho = bf16_to_f64(h_or).reshape(n, I // 32, 32)
    dg = oracle.dequantize_rows(gc, gs).reshape(n, I // 32, 32)
    do = oracle.dequantize_rows(oc, os_).reshape(n, I // 32, 32)
    dv = np.abs(dg - do)
    gs = np.asarray(gs, np.int64).reshape(n, I // 32)
    os_ = np.asarray(os_, np.int64).reshape(n, I // 32)
    # codes per element, low nibble first
    def codes(packed):
        p = np.asarray(packed, np.uint8).reshape(n, I // 2)
        return np.stack([p & 0xF, p >> 4], -1).reshape(n, I // 32, 32)
    cg, co = codes(gc), codes(oc)

    same = gs == os_
    # kind 1: same scale byte, adjacent magnitudes bracketing their midpoint
    r, b, j = np.nonzero(same[..., None] & ((cg != co)))
    if r.size:
        mg, mo = cg[r, b, j] & 7, co[r, b, j] & 7
        X = np.exp2(gs[r, b].astype(np.float64) - 127.0)
        lo, hi = np.minimum(mg, mo), np.maximum(mg, mo)
        zero_sign = (mg == 0) & (mo == 0)                   # +0 against -0: no value change
        adjacent = hi - lo == 1
        sign_ok = ((cg[r, b, j] >> 3) == (co[r, b, j] >> 3)) | (lo == 0)
        mid = 0.5 * (E2M1_MAGS[lo] + E2M1_MAGS[np.minimum(hi, 7)]) * X
        ag, ao = np.abs(hg[r, b, j]), np.abs(ho[r, b, j])
        brackets = (ag - mid) * (ao - mid) <= 0.0
        ok = zero_sign | (adjacent & sign_ok & brackets)
        if not ok.all():
            k = int(np.nonzero(~ok)[0][0])
            raise AssertionError(
                f"requant code of row {r[k]}, element {b[k] * 32 + j[k]} differs from the "
                f"oracle's without a one-step midpoint crossing: gpu code {cg[r[k], b[k], j[k]]:#x} "
                f"(h {hg[r[k], b[k], j[k]]!r}), oracle code {co[r[k], b[k], j[k]]:#x} "
                f"(h {ho[r[k], b[k], j[k]]!r}), scale byte {gs[r[k], b[k]]}")
    # kind 2: scale bytes one apart, block maxima bracketing the step
    rb, bb = np.nonzero(~same)
    for r2, b2 in zip(rb, bb):
        sg, so = int(gs[r2, b2]), int(os_[r2, b2])
        amg, amo = np.abs(hg[r2, b2]).max(), np.abs(ho[r2, b2]).max()
        s_hi = max(sg, so)
        P = 4.0 * 2.0 ** (s_hi - 127)
        hi_max, lo_max = (amg, amo) if sg > so else (amo, amg)
        if abs(sg - so) != 1 or not (lo_max < P <= hi_max):
            raise AssertionError(
                f"requant scale of row {r2}, block {b2} differs from the oracle's without the "
                f"block maximum crossing a scale step: gpu byte {sg} (amax {amg!r}), oracle byte "
                f"{so} (amax {amo!r})")
        Xc = 2.0 ** (s_hi - 127)
        v = np.maximum(np.abs(hg[r2, b2]), np.abs(ho[r2, b2])) / Xc
        allowed = 2.0 * _spacing(v) * Xc + np.abs(hg[r2, b2] - ho[r2, b2])
        if not np.all(dv[r2, b2] <= allowed):
            raise AssertionError(f"requant block {b2} of row {r2}: an element moved by more than "
                                 f"the coarser grid allows after a scale step")
    return dv.reshape(n, I)


def requant_slack(case, dbg, h_or, tokens=None):
    """Output slack from requant codes that differ from the oracle's for the
    two reasons requant_moves accepts (and only those).

    dbg: the debug forward's outputs (sorted_route, num_valid, h, a2_codes,
    a2_scales); h_or: the oracle's h [ntok, topk, I] for `tokens` (all
    tokens when None), from the same oracle run whose output is compared.
    slack[t, d] = sum over the token's routes of |w| * sum_i |dv_i| * |W2[e][d, i]|.
    Returns (slack [ntok, D] or None, number of moved h elements, number of h
    elements compared)."""
    sr = dbg["sorted_route"].cpu().numpy()
    n = int(dbg["num_valid"].cpu().numpy()[0])
    R = case.M * case.topk
    rows = np.nonzero(sr[:n] < R)[0]
    r = sr[rows]
    tok_list = np.arange(case.M) if tokens is None else np.asarray(tokens)
    pos = np.full(case.M, -1, np.int64)
    pos[tok_list] = np.arange(tok_list.size)
    keep = pos[r // case.topk] >= 0
    rows, r = rows[keep], r[keep]
    if rows.size == 0:
        return None, 0, 0
    t, s = r // case.topk, r % case.topk
    h_ref = h_or[pos[t], s]
    h_gpu = dbg["h"].cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    oc, os_ = oracle.quantize_rows(h_ref)
    gc = dbg["a2_codes"].cpu().numpy()[rows]
    gs = dbg["a2_scales"].cpu().numpy()[rows]
    # the GPU's codes must be the exact quantization of the GPU's own h
    qc, qs = oracle.quantize_rows(h_gpu)
    assert np.array_equal(gs, qs) and np.array_equal(gc, qc), \
        "GPU requant codes are not the MXFP4 quantization of the GPU h"
    dv = requant_moves(h_gpu, h_ref, gc, gs, oc, os_)
    moved = np.nonzero(dv.max(axis=1) > 0)[0]
    if moved.size == 0:
        return None, 0, dv.size
    slack = np.zeros((tok_list.size, case.D))
    experts = case.ids[t[moved], s[moved]]
    for e in np.unique(experts):
        w2 = np.abs(oracle.dequantize_rows(case.wq[2][e], case.wq[3][e]))    # [D, I]
        for j in moved[experts == e]:
            slack[pos[t[j]]] += abs(float(case.tw[t[j], s[j]])) * (w2 @ dv[j])
    return slack, int(np.count_nonzero(dv)), dv.size


def check_close(gpu_bits, oracle_bits, what="", slack=None):
    """The end-to-end tolerance: |gpu - oracle| <= 2e-2 * rms(oracle) + 2^-7 * |oracle|
    on >= 99.9% of the elements, and no element beyond 0.1 * rms(oracle).

    The strict result (no slack) is always computed and logged.  Without
    `slack` it is what is asserted.  With `slack` (requant_slack: requant
    codes one explained step from the oracle's), each element's bound grows by
    its slack and the strict result is only reported.  Returns dict(strict,
    frac, worst) with worst in units of rms."""
    g = bf16_to_f64(gpu_bits)
    o = bf16_to_f64(oracle_bits)
    assert g.shape == o.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    err = np.abs(g - o)
    base = 2e-2 * rms + 2.0 ** -7 * np.abs(o)
    s_frac = float(np.mean(err <= base)) if err.size else 1.0
    s_worst = float(err.max()) if err.size else 0.0
    strict = s_frac >= 0.999 and s_worst <= 0.1 * rms
    scale = max(rms, 1e-30)
    msg = (f"{what}: rms={rms:.4g} strict: within-bound={s_frac * 100:.4f}% "
           f"worst={s_worst / scale:.4g}*rms -> {'PASS' if strict else 'FAIL'}; "
           f"exact-bf16={float(np.mean(g == o)) * 100 if o.size else 100.0:.2f}%")
    if slack is None:
        log(msg)
        assert s_frac >= 0.999, f"{what}: only {s_frac:.5f} of elements within tolerance"
        assert s_worst <= 0.1 * rms, f"{what}: worst error {s_worst} > 0.1*rms ({rms})"
        return {"strict": True, "frac": s_frac, "worst": s_worst / scale}
    frac = float(np.mean(err <= base + slack))
    over = err - slack
    worst = float(over.max()) if err.size else 0.0
    log(msg + f"; with requant slack on {int(np.count_nonzero(slack.max(axis=1)))} tokens: "
        f"within-bound={frac * 100:.4f}% worst={worst / scale:.4g}*rms")
    assert frac >= 0.999, f"{what}: only {frac:.5f} of elements within tolerance (with slack)"
    assert worst <= 0.1 * rms, f"{what}: worst error beyond slack {worst} > 0.1*rms ({rms})"
    return {"strict": strict, "frac": frac, "worst": worst / scale}
