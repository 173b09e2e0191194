"""Ahead-of-time build of libmoe_mxfp4.so for gfx950 (hipcc, in-tree).

    python -m mixture_experts_mxfp4_amd.build [-v]
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_mxfp4.so")
SOURCES = ["api.hip", "prologue.hip", "prepare.hip", "gemm1.hip", "gemm2.hip", "gemm_tile.hip", "direct.hip",
           "decode_fused.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else (shutil.which("hipcc") or "hipcc")


def compile_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-fvisibility=hidden",
        # no packed-fp32 VALU instructions (v_pk_{add,mul,fma}_f32) anywhere
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-munsafe-fp-atomics",
        "-Wall", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + compile_flags()
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature flag; that warning is harmless
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
