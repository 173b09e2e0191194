"""The benchmark's reporting logic, on the CPU: the algorithmic bytes and
FLOPs behind `value` and `roofline.achieved`, the source-hash guard on the
committed traffic summaries, and the refusal of more than one GPU."""
import os
import shutil
import subprocess
import sys

import numpy as np

import bench
from mixture_experts_mxfp4_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_counts_active_experts_and_valid_routes():
    """2 tokens, 3 slots, E=5: experts {1, 4} active (id 1 twice), one id
    out of range; 5 valid routes."""
    w = inputs.Workload("t", 2, 512, 256, 5, 2, "uniform", 0)
    ids = np.array([[1, 1, 4], [4, -1, 1]], np.int32)
    a = bench.algorithmic(w, ids)
    ID = 256 * 512
    assert a["n_active"] == 2 and a["n_valid"] == 5
    # weights and scales of both GEMMs per active expert, hidden + out, ids + weights
    assert a["bytes"] == 2 * ID * (1 + 1 / 16 + 1 / 2 + 1 / 32) + 2 * (2 * 2 * 512) + 8 * 2 * 3
    assert a["flops"] == 5 * (2 * 2 * 256 * 512 + 2 * 256 * 512)
    assert a["stage1_bytes"] == 2 * ID * (1 + 1 / 16)
    assert a["stage1_flops"] == 5 * 2 * 2 * 256 * 512
    # a token subset counts only its own routes and experts
    b = bench.algorithmic(w, ids, tokens=np.array([0]))
    assert b["n_active"] == 2 and b["n_valid"] == 3


def test_traffic_summary_requires_matching_sources(tmp_path, monkeypatch):
    """A traffic summary taken on other stage-1 sources is not reported."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    kernel, sources = bench.STAGE1["direct"]
    good = bench.source_hash(sources)
    text = f"stage1_source_sha256_16: {good}\ntraffic_bytes_per_launch: 123456\n"
    (prof / f"{kernel}_decode_hbm_traffic.txt").write_text(text)
    for src in sources:                     # the hashed sources, copied unchanged
        dst = tmp_path / src
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, src), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("decode", "direct") == 123456.0
    with open(tmp_path / sources[0], "a") as f:
        f.write("\n// changed\n")
    assert bench.load_traffic("decode", "direct") is None
    assert bench.load_traffic("prefill", "stream") is None       # no summary at all


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_host_cpu_and_workload_summary():
    """The CPU leg states the host's logical CPU count and model; a further
    workload's entry carries its time, rate and both roofline fractions."""
    n, model = bench.host_cpu()
    assert n == os.cpu_count() and (model is None or isinstance(model, str))
    w = inputs.WORKLOADS["large_prefill"]
    ids = np.tile(np.arange(9, dtype=np.int32) + 24, (w.M, 1))
    alg = bench.algorithmic(w, ids)
    r = {"w": w, "alg": alg, "sec": 1e-3, "ms_per_step": 1.0, "value": alg["flops"] / 1e-3 / 1e12,
         "unit": "TFLOP/s", "path_name": "tiled", "stages_us": None,
         "roof": {"bound": "mfma", "kernel": "gemm1_tile_kernel", "achieved": 4000.0,
                  "unit": "TFLOP/s", "frac": 0.396, "kernel_us": 540.0}}
    s = bench.workload_summary(r)
    assert s["us_per_forward"] == 1000.0 and s["unit"] == "TFLOP/s"
    assert abs(s["roofline_frac_forward"] - alg["flops"] / (bench.FP4_PEAK_TFLOPS * 1e12) / 1e-3) < 1e-4
    assert s["stage1"]["frac"] == 0.396 and s["path"] == "tiled"
