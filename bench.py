#!/usr/bin/env python3
"""Benchmark of the fused MXFP4 MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode] [--a16w4]

One step = one full forward through the C ABI on a seeded synthetic
DeepSeek-R1-shaped batch whose inputs are already resident in HBM: on the
route-indexed path (few tokens) stage 1 (own route scan + activation quant +
gate_up + SwiGLU + requant) and stage 2 (down projection x routing weight,
per-token sum); on the sorted paths the prologue (route sort + activation
quant), stage 1, stage 2 and the per-token slot reduction.  Prepared weights are kept in
several copies and rotated step by step, so that every forward streams its
experts' weights from HBM rather than from the 256 MB Infinity Cache.
--a16w4 runs the same workload through the A16W4 forward (bf16 activations,
no activation quantization; route-indexed kernels, up to 32 tokens).

Prints ONE JSON line: the metric (algorithmic GB/s for HBM-bound workloads,
TFLOP/s for MFMA-bound ones), microseconds per forward, the roofline of the
dominant kernel (stage 1) timed on the device over the same K steps (in a
second pass: its timing records would perturb the timed one), and the CPU
oracle timed on a bounded sample of the same workload.  With the default
decode workload the line also carries a `workloads` map: the other D = 7168
workloads (small_batch, prefill, large_prefill), each timed the same way with
the same K and W (--headline-only leaves them out).

Helper modes (used to make the committed rocprofv3 summaries):
    --copy-calibration         run a plain 1 GiB device copy (counter scale)
    --summarize-stats DIR      print the kernel-time summary of a rocprofv3 run
    --summarize-pmc DIR        print per-kernel counter means of a --pmc run
    --traffic-summary WORKLOAD FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
                               print the stage-1 HBM traffic summary (the
                               profiles/<kernel>_<workload>_hbm_traffic.txt
                               format) from FETCH_SIZE / WRITE_SIZE passes of
                               the workload and of --copy-calibration
    --mfma-summary WORKLOAD PMC_DIR
                               print the MFMA counter summary of both GEMM
                               stages (profiles/<kernel>_<workload>_mfma.txt)
                               from a `--pmc SQ_INSTS_VALU_MFMA_MOPS_F6F4
                               MfmaUtil` pass of the workload
    --mfma-ceiling             the library's register-only FP4 MFMA probe
                               (moe_mxfp4_mfma_probe) with random and with
                               single-bit operands: the practical ceiling of
                               the MFMA-bound kernels next to the published peak
"""
import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/forward + HBM GB/s (M≤16) / MXFP4 MFMA TFLOPS (M≥1024), D=7168"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense MXFP4 MFMA
MALL_BYTES = 256 << 20
NS_A16 = 13.0                   # oracle ns per multiply-add with bf16 activations
# the stage-1 (dominant) kernel and the sources that define it, per path
_CSRC = "mixture_experts_mxfp4_amd/csrc/"
STAGE1 = {
    "direct": ("gemm1_direct_kernel", (_CSRC + "direct.hip", _CSRC + "direct_common.h",
                                       _CSRC + "moe_common.h", _CSRC + "moe_kernels.h")),
    "persistent": ("decode_fused_kernel", (_CSRC + "decode_fused.hip", _CSRC + "direct_common.h",
                                           _CSRC + "moe_common.h", _CSRC + "moe_kernels.h")),
    "stream": ("gemm1_swiglu_quant_kernel", (_CSRC + "gemm1.hip", _CSRC + "moe_common.h",
                                             _CSRC + "moe_kernels.h")),
    "tiled": ("gemm1_tile_kernel", (_CSRC + "gemm_tile.hip", _CSRC + "moe_common.h",
                                    _CSRC + "moe_kernels.h")),
}


# ---------------------------------------------------------------- helpers ---

def _hip():
    for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
        try:
            lib = ctypes.CDLL(name)
            break
        except OSError:
            continue
    else:
        raise RuntimeError("libamdhip64.so not found")
    lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


class Events:
    """Raw hipEvent_t handles created through the HIP runtime, for the
    library's kernel-attached timing (moe_mxfp4_forward_profiled), which
    records them on the stream the kernels are launched on."""

    def __init__(self, n):
        self.hip = _hip()
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), 0) == 0
            self.ev.append(h.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]),
                                            ctypes.c_void_p(self.ev[b])) == 0
        return float(out.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(w, ids_np, tokens=None):
    """Algorithmic bytes / FLOPs of a forward over `tokens` (default all):
    the active experts' weights and scales (1.59375*I*D bytes each: w13 codes
    I*D + scales I*D/16, w2 codes I*D/2 + scales I*D/32), hidden and output
    (2*M*D bytes each), ids and weights (8*M*topk); 6*I*D FLOPs per valid
    (token, slot).  Stage 1 alone: 1.0625*I*D bytes per active expert,
    4*I*D FLOPs per valid (token, slot)."""
    import numpy as np
    ids = ids_np if tokens is None else ids_np[tokens]
    M, k = ids.shape
    valid = (ids >= 0) & (ids < w.E)
    n_active = len(np.unique(ids[valid]))
    n_valid = int(valid.sum())
    ID = w.I * w.D
    return {
        "n_active": n_active, "n_valid": n_valid,
        "bytes": n_active * ID * 1.59375 + 4.0 * M * w.D + 8.0 * M * k,
        "flops": 6.0 * ID * n_valid,
        "stage1_bytes": n_active * ID * 1.0625,
        "stage1_flops": 4.0 * ID * n_valid,
    }


def load_traffic(workload, path_name):
    """HBM traffic of the stage-1 kernel from the committed rocprofv3 counter
    summary, if it was taken on the current stage-1 source; else None."""
    kernel, sources = STAGE1[path_name]
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("stage1_source_sha256_16") != source_hash(sources):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------- CPU leg ---

def cpu_baseline(w, hidden, ids, tw, w13f, w2f, target_cpu_s=16.0, act_quant=True):
    """The CPU oracle on a bounded sample of the same workload (its first
    tokens), weights quantized by the oracle itself (untimed, like the GPU's
    weight preparation)."""
    import numpy as np

    import oracle
    from mixture_experts_mxfp4_amd import inputs

    threads = max(1, min(16, os.cpu_count() or 1))
    # measured oracle cost per multiply-add: ~16 ns (MXFP4 operands), ~NS_A16 ns (bf16)
    per_tok_cpu_s = (16e-9 if act_quant else NS_A16 * 1e-9) * 3 * w.I * w.D * w.topk
    n = int(max(1, min(w.M, round(target_cpu_s / per_tok_cpu_s))))
    toks = np.arange(n)
    ids_np = ids.numpy()
    used = np.unique(ids_np[toks][(ids_np[toks] >= 0) & (ids_np[toks] < w.E)])
    remap = np.full(w.E, -1, np.int64)
    remap[used] = np.arange(used.size)
    sub_ids = np.where((ids_np >= 0) & (ids_np < w.E), remap[np.clip(ids_np, 0, w.E - 1)], -1)
    sub_ids = sub_ids.astype(np.int32)
    sel = torch_index(used)
    w13, w13s = oracle.quantize_rows(inputs.bf16_bits(w13f[sel]).reshape(-1, w.D), threads)
    w2, w2s = oracle.quantize_rows(inputs.bf16_bits(w2f[sel]).reshape(-1, w.I), threads)
    Eu = used.size
    wq = (w13.reshape(Eu, 2 * w.I, w.D // 2), w13s.reshape(Eu, 2 * w.I, w.D // 32),
          w2.reshape(Eu, w.D, w.I // 2), w2s.reshape(Eu, w.D, w.I // 32))
    hb = inputs.bf16_bits(hidden)
    threads = min(threads, n)          # the oracle runs one token per thread
    t0 = time.perf_counter()
    oracle.forward(hb, *wq, sub_ids, tw.numpy(), tokens=toks, nthreads=threads,
                   act_quant=act_quant)
    dt = time.perf_counter() - t0
    alg = algorithmic(w, ids_np, toks)
    return {"seconds": dt, "tokens": n, "threads": threads, "alg": alg}


def torch_index(np_idx):
    import torch
    return torch.from_numpy(np_idx.astype("int64"))


# ------------------------------------------------------------- GPU leg ----

def workload_of(args):
    """The named workload, or with --shape M,E,I a DeepSeek-R1-shaped one
    (D=7168, 8 routed ids uniform without replacement + the shared expert E-1,
    as in the self-test generator of kernelindex submission 723815)."""
    from mixture_experts_mxfp4_amd import inputs
    if not args.shape:
        return inputs.WORKLOADS[args.workload]
    M, E, I = (int(v) for v in args.shape.split(","))
    return inputs.Workload(f"shape_M{M}_E{E}_I{I}", M, 7168, I, E, 8, "uniform", 7)


def measure(w, args, a16=False, persistent=False, splitk=False):
    """One workload on the GPU: K timed forwards after W untimed ones, then the
    kernel-timing pass.  Returns the timing and roofline figures (and the
    float inputs, for the CPU leg)."""
    import numpy as np
    import torch

    from mixture_experts_mxfp4_amd import binding, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hidden, ids, tw = inputs.make_activations(w.M, w.D, w.E, w.n_routed, w.routing, w.seed)
    w13f, w2f = inputs.make_weights(w.E, w.D, w.I, w.seed, device=dev)

    # MXFP4 weights from the library's own quantizer, then the kernel layout
    raw = [binding.moe_mxfp4_quantize(w13f.reshape(-1, w.D)),
           binding.moe_mxfp4_quantize(w2f.reshape(-1, w.I))]
    w13 = raw[0][0].view(w.E, 2 * w.I, w.D // 2)
    w13s = raw[0][1].view(w.E, 2 * w.I, w.D // 32)
    w2 = raw[1][0].view(w.E, w.D, w.I // 2)
    w2s = raw[1][1].view(w.E, w.D, w.I // 32)
    prepared = binding.moe_mxfp4_prepare_weights(w13, w13s, w2, w2s)
    del raw, w13, w13s, w2, w2s
    ids_np = ids.numpy()
    alg = algorithmic(w, ids_np)
    per_copy_active = alg["n_active"] * w.I * w.D * 1.59375
    copies = args.copies or int(max(2, min(8, np.ceil(3 * (MALL_BYTES + (64 << 20)) / per_copy_active))))
    weight_sets = [prepared] + [tuple(t.clone() for t in prepared) for _ in range(copies - 1)]

    h_d, ids_d, tw_d = hidden.to(dev), ids.to(dev), tw.to(dev)
    out = torch.empty_like(h_d)
    if persistent:
        if binding.moe_mxfp4_persistent_workspace_bytes(w.M, w.D, w.I, w.E, w.topk) == 0:
            raise SystemExit(f"bench.py: the persistent forward does not run {w.name} (M={w.M})")
        ws = binding.alloc_workspace_persistent(w.M, w.D, w.I, w.E, w.topk, dev)
        path = binding.PATH_DIRECT
        n_wg = binding.moe_mxfp4_persistent_workgroups(w.M)

        def forward(wset):
            binding.moe_mxfp4_forward_persistent(h_d, *wset, ids_d, tw_d, out, ws)

        def forward_timed(wset, ev, clk=None):
            binding.moe_mxfp4_forward_persistent_debug(h_d, *wset, ids_d, tw_d, out, ws,
                                                       intermediates=False, kernel_events=ev,
                                                       clock=clk)
    elif splitk:
        if binding.moe_mxfp4_splitk_workspace_bytes(w.M, w.D, w.I, w.E, w.topk) == 0:
            raise SystemExit(f"bench.py: the split-K forward does not run {w.name} (M={w.M})")
        ws = binding.alloc_workspace_splitk(w.M, w.D, w.I, w.E, w.topk, dev)
        path = binding.PATH_DIRECT
        n_wg = binding.splitk_stage1_workgroups(w.M, w.I, w.E, w.topk)

        def forward(wset):
            binding.moe_mxfp4_forward_splitk(h_d, *wset, ids_d, tw_d, out, ws)

        def forward_timed(wset, ev, clk=None):
            binding.moe_mxfp4_forward_splitk_debug(h_d, *wset, ids_d, tw_d, out, ws,
                                                   intermediates=False, kernel_events=ev,
                                                   stage1_clock=clk)
    elif a16:
        if binding.moe_mxfp4_a16w4_workspace_bytes(w.M, w.D, w.I, w.E, w.topk) == 0:
            raise SystemExit(f"bench.py: the A16W4 forward does not run {w.name} (M={w.M})")
        ws = binding.alloc_workspace_a16w4(w.M, w.D, w.I, w.E, w.topk, dev)
        path = binding.PATH_DIRECT
        n_wg = binding.a16w4_stage1_workgroups(w.M, w.I, w.E, w.topk)

        def forward(wset):
            binding.moe_mxfp4_forward_a16w4(h_d, *wset, ids_d, tw_d, out, ws)

        def forward_timed(wset, ev, clk=None):
            binding.moe_mxfp4_forward_a16w4_debug(h_d, *wset, ids_d, tw_d, out, ws,
                                                  kernel_events=ev, stage1_clock=clk)
    else:
        ws = binding.alloc_workspace(w.M, w.D, w.I, w.E, w.topk, dev)
        path = binding.moe_mxfp4_path(w.M, w.D, w.I, w.E, w.topk)
        n_wg = binding.moe_mxfp4_stage1_workgroups(w.M, w.D, w.I, w.E, w.topk)

        def forward(wset):
            binding.moe_mxfp4_forward(h_d, *wset, ids_d, tw_d, out, ws)

        def forward_timed(wset, ev, clk=None):
            binding.moe_mxfp4_forward_profiled(h_d, *wset, ids_d, tw_d, out, ws, ev, clk)
    torch.cuda.synchronize()
    path_name = "persistent" if persistent else binding.PATH_NAMES[path]
    launches = (1,) if persistent else binding.PATH_LAUNCHES[path]
    workload_id = (w.name + ("_a16w4" if a16 else "") + ("_persistent" if persistent else "")
                   + ("_splitk" if splitk else ""))

    # buffers of the kernel-timing pass, allocated up front so that no host
    # work separates the passes
    khz = binding.moe_mxfp4_wall_clock_khz()
    spans = torch.zeros((args.steps + 1, 2 * n_wg), dtype=torch.int64, device=dev)
    step_ev = Events(2 * (args.steps + 1))

    # untimed warm-up; the last warm-up pass also times every launch.  Under
    # sustained matrix-core load the chip's power controller overshoots after
    # any pause: the first ~20 forwards of large_prefill run up to 40% slower
    # than the steady state (per-dispatch kernel traces).
    stage_ev = Events(8)
    for i in range(args.warmup):
        ev = stage_ev.ev if i == args.warmup - 1 else [None] * 8
        forward_timed(weight_sets[i % copies], ev)
    torch.cuda.synchronize()
    stages_us = None
    if args.warmup > 0:
        stages_us = {binding.LAUNCHES[j]: round(1000 * stage_ev.ms(2 * j, 2 * j + 1), 2)
                     for j in launches}

    # timed region: exactly K forwards, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        forward(weight_sets[i % copies])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = 1000.0 * (t1 - t0) / args.steps

    # kernel-timing pass: the same K forwards again, on the same stream, each
    # with (a) stage 1's span on the device clock (its earliest workgroup
    # start to its latest workgroup end, recorded by the kernel itself) and (b)
    # HIP stop events attached to the dispatches of stage 1 and of the launch
    # before it.  Back-to-back launches start as the previous one ends, so
    # stop minus previous stop is stage 1's time as the queue sees it; the
    # runtime's marker for a launch carrying events adds a few microseconds
    # in front of it, which the span excludes.  Launches with events or spans
    # are not the plain timed ones, so this is a pass of its own, preceded by
    # the same W untimed forwards as the timed region.
    prev = 0 if 0 in launches else launches[-1]          # launch before stage 1
    same_forward = prev < 1
    for i in range(args.warmup):
        forward(weight_sets[i % copies])
    for i in range(args.steps + 1):
        ev = [None] * 8
        if prev != 1:                  # one launch per forward: its own previous stop
            ev[2 * prev + 1] = step_ev.ev[2 * i]
        ev[3] = step_ev.ev[2 * i + 1]
        forward_timed(weight_sets[i % copies], ev, spans[i])
    torch.cuda.synchronize()
    if same_forward:
        ev_times = [step_ev.ms(2 * i, 2 * i + 1) for i in range(1, args.steps + 1)]
    elif prev == 1:
        ev_times = [step_ev.ms(2 * (i - 1) + 1, 2 * i + 1) for i in range(1, args.steps + 1)]
    else:
        ev_times = [step_ev.ms(2 * (i - 1), 2 * i + 1) for i in range(1, args.steps + 1)]
    sp = spans[1:].cpu()
    span_ms = [binding.stage1_span_ms(sp[i], khz) for i in range(args.steps)]
    stage1_ms = sum(span_ms) / len(span_ms)
    stage1_event_ms = sum(ev_times) / len(ev_times)
    step_ev.close()
    stage_ev.close()

    sec = ms_per_step / 1000.0
    # roofline: which peak bounds the whole forward of this workload
    hbm_bound = alg["bytes"] / (HBM_PEAK_GBS * 1e9) >= alg["flops"] / (FP4_PEAK_TFLOPS * 1e12)
    if hbm_bound:
        value, unit = alg["bytes"] / sec / 1e9, "GB/s"
        # the persistent kernel is the whole forward: all of its bytes
        kbytes = alg["bytes"] if persistent else alg["stage1_bytes"]
        achieved = kbytes / (stage1_ms / 1000.0) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        value, unit = alg["flops"] / sec / 1e12, "TFLOP/s"
        achieved = alg["stage1_flops"] / (stage1_ms / 1000.0) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP4_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP4_PEAK_TFLOPS, 4)}
    roof["traffic"] = load_traffic(workload_id, path_name)
    roof["kernel"] = STAGE1[path_name][0]
    roof["source_sha256_16"] = source_hash(STAGE1[path_name][1])
    if persistent:
        roof["algorithmic_bytes"] = "the whole forward (one launch)"
    roof["kernel_us"] = round(stage1_ms * 1000.0, 2)
    roof["kernel_us_events"] = round(stage1_event_ms * 1000.0, 2)
    roof["kernel_timing"] = ("kernel span on the device clock; events: stop-to-stop "
                             "with the runtime's launch marker")
    res = {
        "w": w, "alg": alg, "hbm_bound": hbm_bound, "value": value, "unit": unit,
        "ms_per_step": ms_per_step, "sec": sec, "path_name": path_name, "copies": copies,
        "stages_us": stages_us, "roof": roof,
        "inputs": (hidden, ids, tw, w13f, w2f),
    }
    del weight_sets, prepared, ws, out, h_d, spans
    return res


def forward_fraction(r):
    """The whole forward's roofline fraction: the larger of its HBM and MFMA
    floors over its measured time."""
    alg = r["alg"]
    return max(alg["bytes"] / (HBM_PEAK_GBS * 1e9), alg["flops"] / (FP4_PEAK_TFLOPS * 1e12)) / r["sec"]


def workload_summary(r):
    """The figures of one further workload for the `workloads` map."""
    alg, sec = r["alg"], r["sec"]
    return {
        "us_per_forward": round(r["ms_per_step"] * 1000.0, 2),
        "value": round(r["value"], 3 if r["unit"] == "TFLOP/s" else 1),
        "unit": r["unit"],
        "tokens_per_s": round(r["w"].M / sec, 1),
        "hbm_gbs": round(alg["bytes"] / sec / 1e9, 1),
        "mfma_tflops": round(alg["flops"] / sec / 1e12, 3),
        "roofline_frac_forward": round(forward_fraction(r), 4),
        "stage1": {k: r["roof"][k] for k in ("bound", "kernel", "achieved", "unit", "frac",
                                             "kernel_us")},
        "path": r["path_name"],
        "launches_per_forward": _launches(r["w"]),
        "kernel_us_warmup": r["stages_us"],
    }


def _launches(w):
    from mixture_experts_mxfp4_amd import binding
    return binding.moe_mxfp4_launch_count(w.M, w.D, w.I, w.E, w.topk)


def host_cpu():
    """The host's logical CPU count and CPU model (from /proc/cpuinfo)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def run(args):
    import torch

    from mixture_experts_mxfp4_amd import binding

    w = workload_of(args)
    a16 = args.a16w4
    r = measure(w, args, a16, persistent=args.persistent, splitk=args.splitk)
    hidden, ids, tw, w13f, w2f = r.pop("inputs")
    alg, sec, unit = r["alg"], r["sec"], r["unit"]

    cpu = None
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, hidden, ids, tw, w13f, w2f, args.cpu_sample_s, act_quant=not a16)
        ca = cb["alg"]
        cval = ca["bytes"] / cb["seconds"] / 1e9 if r["hbm_bound"] else ca["flops"] / cb["seconds"] / 1e12
        n_cpu, model = host_cpu()
        cpu = {"value": round(cval, 4), "unit": unit, "cores": cb["threads"], "kind": "oracle",
               "host_logical_cpus": n_cpu, "host_cpu_model": model,
               "sample": f"first {cb['tokens']} of {w.M} tokens of the {w.name} workload "
                         f"({cb['seconds']:.2f} s wall, fp64 C oracle"
                         f"{', activations unquantized' if a16 else ''}, {cb['threads']} threads "
                         f"on a host with {n_cpu} logical CPUs)"}
    del hidden, ids, tw, w13f, w2f

    # the other D = 7168 workloads of the metric, timed with the same K and W
    extra = {}
    if not args.headline_only and not args.shape and not a16 and not args.persistent and not args.splitk:
        from mixture_experts_mxfp4_amd import inputs
        for name in ("small_batch", "prefill", "large_prefill"):
            if name == w.name:
                continue
            torch.cuda.empty_cache()
            ro = measure(inputs.WORKLOADS[name], args)
            ro.pop("inputs")
            extra[name] = workload_summary(ro)
            extra[name]["config"] = (f"M={ro['w'].M} D={ro['w'].D} I={ro['w'].I} E={ro['w'].E} "
                                     f"top{ro['w'].topk} ({ro['w'].n_routed} routed "
                                     f"{ro['w'].routing} + shared expert {ro['w'].E - 1})")
            del ro

    line = {
        "metric": METRIC,
        "value": round(r["value"], 3 if unit == "TFLOP/s" else 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if a16 else "mxfp4",
        "data": "synthetic",
        "config": {"workload": f"{w.name}{' A16W4 (bf16 activations, MXFP4 weights)' if a16 else ''}"
                               f": M={w.M} D={w.D} I={w.I} E={w.E} top{w.topk} "
                               f"({w.n_routed} routed {w.routing} + shared expert {w.E - 1})",
                   "mode": "a16w4" if a16 else "a4w4",
                   "variant": ("persistent (one launch)" if args.persistent else
                               "split-K stage 1" if args.splitk else "default"),
                   "M": w.M, "D": w.D, "I": w.I, "E": w.E, "topk": w.topk,
                   "routing": w.routing, "seed": w.seed, "global_batch": w.M,
                   "parallelism": "single GPU", "path": r["path_name"],
                   "block_m": 16 if a16 else binding.moe_mxfp4_block_m(w.M, w.D, w.I, w.E, w.topk),
                   "weight_copies": r["copies"]},
        "us_per_forward": round(r["ms_per_step"] * 1000.0, 2),
        "tokens_per_s": round(w.M / sec, 1),
        "hbm_gbs": round(alg["bytes"] / sec / 1e9, 1),
        "mfma_tflops": round(alg["flops"] / sec / 1e12, 3),
        "roofline_frac_forward": round(forward_fraction(r), 4),
        "active_experts": alg["n_active"],
        "launches_per_forward": 2 if a16 else 1 if args.persistent else _launches(w),
        "kernel_us_warmup": r["stages_us"],
        "roofline": r["roof"],
        "cpu_baseline": cpu,
    }
    if extra:
        line["workloads"] = extra
    print(json.dumps(line, ensure_ascii=False), flush=True)


# ------------------------------------------------------- profiling helpers ---

def mfma_ceiling(iters=2_000_000):
    """The FP4 MFMA rate on register operands (no memory traffic), with random
    and with single-bit operands, for the 32x32x64 instruction of the tiled
    kernels and the 16x16x128 one of the streaming kernels, against the
    published dense peak."""
    import torch

    from mixture_experts_mxfp4_amd import binding
    torch.cuda.set_device(0)
    out = {"published_peak_tflops": FP4_PEAK_TFLOPS, "iters_per_wave": iters}
    for name, rnd, small in (("random_operands", True, False), ("single_bit_operands", False, False),
                             ("random_operands_16x16x128", True, True),
                             ("single_bit_operands_16x16x128", False, True)):
        r = binding.moe_mxfp4_mfma_probe(rnd, iters, small_tile=small)
        out[name] = {"tflops": round(r["tflops"], 1), "shader_mhz": round(r["shader_mhz"], 1),
                     "per_clock_frac": round(r["per_clock_frac"], 4),
                     "frac_of_peak": round(r["tflops"] / FP4_PEAK_TFLOPS, 4)}
    print(json.dumps(out), flush=True)


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": n}), flush=True)


def _rows(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    return rows


def summarize_stats(d):
    rows = _rows(os.path.join(d, "**", "*kernel_stats.csv"))
    print(f"{'kernel':80s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        name = r.get("Name", "")[:80]
        print(f"{name:80s} {r.get('Calls', ''):>6s} {float(r.get('AverageNs', 0)) / 1000:10.2f} "
              f"{float(r.get('MinNs', 0)) / 1000:10.2f} {float(r.get('MaxNs', 0)) / 1000:10.2f} "
              f"{float(r.get('Percentage', 0)):6.2f}")


def summarize_pmc(d):
    rows = _rows(os.path.join(d, "**", "*counter_collection.csv"))
    acc = {}
    for r in rows:
        key = (r.get("Kernel_Name", "")[:80], r.get("Counter_Name", ""))
        acc.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
    print(f"{'kernel':80s} {'counter':>12s} {'dispatches':>10s} {'mean_per_dispatch':>18s}")
    for (k, c), v in sorted(acc.items()):
        print(f"{k:80s} {c:>12s} {len(v):10d} {sum(v) / len(v):18.1f}")


def _pmc_mean(d, kernel_prefix):
    """Mean per dispatch of the one counter of a --pmc run, over the kernels
    whose name (template arguments included) starts with `kernel_prefix`."""
    vals = []
    for r in _rows(os.path.join(d, "**", "*counter_collection.csv")):
        name = r.get("Kernel_Name", "").replace("void ", "")
        if name.startswith(kernel_prefix):
            vals.append(float(r.get("Counter_Value", 0)))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel_prefix} in {d}")
    return sum(vals) / len(vals), len(vals)


def traffic_summary(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    from mixture_experts_mxfp4_amd import binding, inputs
    a16 = workload.endswith("_a16w4")          # the A16W4 forward on that workload
    w = inputs.WORKLOADS[workload[:-len("_a16w4")] if a16 else workload]
    path = binding.PATH_DIRECT if a16 else binding.moe_mxfp4_path(w.M, w.D, w.I, w.E, w.topk)
    path_name = binding.PATH_NAMES[path]
    kernel, sources = STAGE1[path_name]
    copy_kib = float(1 << 30) / 1024.0
    cf, _ = _pmc_mean(copy_fetch_dir, "__amd_rocclr_copyBuffer")
    cw, _ = _pmc_mean(copy_write_dir, "__amd_rocclr_copyBuffer")
    f, nf = _pmc_mean(fetch_dir, "moe::" + kernel)
    wr, nw = _pmc_mean(write_dir, "moe::" + kernel)
    ff, fw = copy_kib / cf, copy_kib / cw
    traffic = (f * ff + wr * fw) * 1024.0
    print(f"# HBM traffic of {kernel} on the {workload} workload (path {path_name})")
    print(f"# FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by what the same counters")
    print(f"# read for a plain 1 GiB device copy (bench.py --copy-calibration)")
    print(f"workload: {workload}")
    print(f"kernel: {kernel}")
    print(f"stage1_source_sha256_16: {source_hash(sources)}")
    print(f"fetch_size_kib_per_dispatch: {f:.1f}  ({nf} dispatches)")
    print(f"write_size_kib_per_dispatch: {wr:.1f}  ({nw} dispatches)")
    print(f"copy_fetch_size_kib: {cf:.1f}  (1 GiB = {copy_kib:.0f} KiB)")
    print(f"copy_write_size_kib: {cw:.1f}")
    print(f"fetch_scale: {ff:.4f}")
    print(f"write_scale: {fw:.4f}")
    print(f"traffic_bytes_per_launch: {traffic:.0f}")


def _pmc_rows(d, kernel_prefix):
    """Per-dispatch counter rows of the kernels whose name starts with the prefix."""
    out = {}
    for r in _rows(os.path.join(d, "**", "*counter_collection.csv")):
        name = r.get("Kernel_Name", "").replace("void ", "")
        if name.startswith(kernel_prefix):
            key = (r["Dispatch_Id"], int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
            out.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def mfma_summary(workload, pmc_dir):
    """FP4 MFMA work the hardware counted (SQ_INSTS_VALU_MFMA_MOPS_F6F4 x 512
    FLOP) and the MFMA busy share (MfmaUtil) per dispatch of both GEMM
    stages, against the algorithmic FLOPs of the valid routes."""
    import numpy as np

    from mixture_experts_mxfp4_amd import binding, inputs
    w = inputs.WORKLOADS[workload]
    path_name = binding.PATH_NAMES[binding.moe_mxfp4_path(w.M, w.D, w.I, w.E, w.topk)]
    _, ids, _ = inputs.make_activations(w.M, w.D, w.E, w.n_routed, w.routing, w.seed)
    alg = algorithmic(w, ids.numpy())
    kernel1, _ = STAGE1[path_name]
    kernel2 = kernel1.replace("gemm1", "gemm2").replace("_swiglu_quant", "_simple")
    print(f"# FP4 MFMA counters of the {workload} workload (path {path_name}), per dispatch")
    print(f"# issued = SQ_INSTS_VALU_MFMA_MOPS_F6F4 x 512 FLOP; busy = MfmaUtil (MFMA busy cycles")
    print(f"# over active cycles x SIMDs); durations from the same counter run (kernels serialized)")
    print(f"workload: {workload}")
    print(f"stage1_source_sha256_16: {source_hash(STAGE1[path_name][1])}")
    for stage, kernel, fl in (("stage1", kernel1, alg["stage1_flops"]),
                              ("stage2", kernel2, alg["flops"] - alg["stage1_flops"])):
        rows = _pmc_rows(pmc_dir, "moe::" + kernel)
        if not rows:
            continue
        mops = np.mean([v.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0) for v in rows.values()])
        util = np.mean([v.get("MfmaUtil", 0.0) for v in rows.values()])
        dur = np.mean([(k[2] - k[1]) * 1e-9 for k in rows])
        issued = mops * 512.0
        print(f"{stage}_kernel: {kernel}  ({len(rows)} dispatches)")
        print(f"{stage}_issued_flop_per_dispatch: {issued:.4e}")
        print(f"{stage}_algorithmic_flop: {fl:.4e}")
        print(f"{stage}_issued_over_algorithmic: {issued / fl:.3f}")
        print(f"{stage}_mfma_busy_pct: {util:.1f}")
        print(f"{stage}_duration_us_counter_run: {dur * 1e6:.1f}")
        print(f"{stage}_issued_tflops_counter_run: {issued / dur / 1e12:.1f}")


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode",
                   choices=["tiny", "decode", "small_batch", "prefill", "large_prefill"])
    p.add_argument("--shape", metavar="M,E,I", default=None,
                   help="a D=7168 top-9 workload of this shape instead of --workload")
    p.add_argument("--a16w4", action="store_true",
                   help="the A16W4 forward (bf16 activations; up to 32 tokens)")
    p.add_argument("--persistent", action="store_true",
                   help="the persistent forward (one launch; up to 32 tokens)")
    p.add_argument("--splitk", action="store_true",
                   help="the forward with a split-K stage 1 (up to 32 tokens)")
    p.add_argument("--copies", type=int, default=0, help="weight copies rotated (0: auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="time only the named workload (no `workloads` map of the others)")
    p.add_argument("--cpu-sample-s", type=float, default=16.0,
                   help="CPU-seconds of oracle work in the baseline sample")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--mfma-ceiling", action="store_true")
    p.add_argument("--mfma-summary", nargs=2, metavar=("WORKLOAD", "PMC_DIR"))
    p.add_argument("--summarize-stats", metavar="DIR")
    p.add_argument("--summarize-pmc", metavar="DIR")
    p.add_argument("--traffic-summary", nargs=5,
                   metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    args = p.parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    if args.mfma_summary:
        return mfma_summary(*args.mfma_summary)
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats)
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the forward is measured on exactly one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported.", file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        return copy_calibration()
    if args.mfma_ceiling:
        return mfma_ceiling()
    if args.steps < 1:
        p.error("--steps must be >= 1")
    run(args)


if __name__ == "__main__":
    main()
