"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, run on
the CPU (no GPU, nothing here launches a kernel):

- the CPU oracle (oracle/moe_oracle.c), built with gcc and driven by
  tests/sanitize/oracle_driver.c through every function it exports;
- the library's host code (csrc/api.hip: argument validation, shape queries,
  workspace layout), instrumented on its host side only and linked with the
  library's other objects, loaded into a Python child process with the
  sanitizer runtime preloaded, and called with shapes across the limits and
  with arguments that every entry point must refuse before it touches a
  device.
"""
import glob
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    subprocess.run([gcc, "-std=c11", "-O1", "-g", *SAN_FLAGS, "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "oracle", "moe_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    "-o", exe, "-lm", "-lpthread"], check=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


_DRIVER = textwrap.dedent('''
    import ctypes, sys
    lib = ctypes.CDLL(sys.argv[1])
    I, I64, P, SZ = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    for f in ("moe_mxfp4_path", "moe_mxfp4_block_m", "moe_mxfp4_launch_count"):
        getattr(lib, f).argtypes, getattr(lib, f).restype = [I] * 5, I
    for f in ("moe_mxfp4_workspace_bytes", "moe_mxfp4_a16w4_workspace_bytes"):
        getattr(lib, f).argtypes, getattr(lib, f).restype = [I] * 5, SZ
    lib.moe_mxfp4_stage1_workgroups.argtypes, lib.moe_mxfp4_stage1_workgroups.restype = [I] * 5, I64
    lib.moe_mxfp4_route_capacity.argtypes, lib.moe_mxfp4_route_capacity.restype = [I] * 4, I64
    lib.moe_mxfp4_status_string.argtypes, lib.moe_mxfp4_status_string.restype = [I], ctypes.c_char_p
    fwd = [P] * 8 + [I] * 5 + [P, SZ]
    lib.moe_mxfp4_forward.argtypes = fwd + [P]
    lib.moe_mxfp4_forward_a16w4.argtypes = fwd + [P]
    lib.moe_mxfp4_forward_debug.argtypes = fwd + [P] * 5 + [P]
    lib.moe_mxfp4_forward_profiled.argtypes = fwd + [P, P, P]
    lib.moe_mxfp4_quantize.argtypes = [P, I64, I64, P, P, P]
    lib.moe_mxfp4_route.argtypes = [P, P] + [I] * 4 + [P] * 4 + [P]
    lib.moe_mxfp4_prepare_weights.argtypes = [P] * 4 + [I] * 3 + [P] * 5
    lib.moe_mxfp4_forward_noalloc.argtypes = [P] * 8 + [I] * 5 + [P]
    lib.moe_mxfp4_forward_persistent.argtypes = fwd + [P]
    lib.moe_mxfp4_persistent_workspace_bytes.argtypes = [I] * 5
    lib.moe_mxfp4_persistent_workspace_bytes.restype = SZ
    lib.moe_mxfp4_workspace_init.argtypes = [P, SZ, P]
    lib.moe_mxfp4_forward_splitk.argtypes = fwd + [P]
    lib.moe_mxfp4_splitk_workspace_bytes.argtypes = [I] * 5
    lib.moe_mxfp4_splitk_workspace_bytes.restype = SZ
    shapes = []
    for M in (0, 1, 7, 16, 32, 33, 64, 1024, 4096, 1 << 21, 1 << 24):
        for D, Id in ((256, 256), (7168, 256), (7168, 2048), (65536, 65536), (500, 256)):
            for E in (1, 9, 33, 257, 1024, 1025):
                for k in (1, 9, 16, 17, 32, 33):
                    shapes.append((M, D, Id, E, k))
    for s in shapes:
        path = lib.moe_mxfp4_path(*s)
        ws = lib.moe_mxfp4_workspace_bytes(*s)
        lib.moe_mxfp4_a16w4_workspace_bytes(*s)
        lib.moe_mxfp4_block_m(*s)
        lib.moe_mxfp4_launch_count(*s)
        lib.moe_mxfp4_stage1_workgroups(*s)
        lib.moe_mxfp4_persistent_workspace_bytes(*s)
        lib.moe_mxfp4_splitk_workspace_bytes(*s)
        assert (path == 0) == (ws == 0) or s[0] == 0, s
        for bm in (1, 16, 256):
            lib.moe_mxfp4_route_capacity(s[0], s[3], s[4], bm)
    for st in range(-2, 7):
        assert lib.moe_mxfp4_status_string(st)
    null, ok, odd = P(0), P(0x1000), P(0x1008)
    # every call below must be refused by host validation (no device call)
    for f in (lib.moe_mxfp4_forward, lib.moe_mxfp4_forward_a16w4):
        assert f(*([null] * 8), 4, 512, 256, 9, 3, null, 1 << 30, null) == 1
        assert f(*([ok] * 8), 4, 500, 256, 9, 3, ok, 1 << 30, null) == 1
        assert f(*([odd] + [ok] * 7), 4, 512, 256, 9, 3, ok, 1 << 30, null) == 1
        assert f(*([ok] * 8), 4, 512, 256, 9, 3, ok, 16, null) == 3
        assert f(*([ok] * 8), 0, 512, 256, 9, 3, ok, 0, null) == 0
    assert lib.moe_mxfp4_forward_a16w4(*([ok] * 8), 64, 512, 256, 9, 3, ok, 1 << 30, null) == 2
    assert lib.moe_mxfp4_forward(*([ok] * 8), 4096, 65536, 65536, 33, 9, ok, 1 << 40, null) == 2
    assert lib.moe_mxfp4_forward_debug(*([ok] * 8), 4, 512, 256, 9, 3, ok, 16, *([null] * 5), null) == 3
    assert lib.moe_mxfp4_forward_debug(*([ok] * 8), 4, 512, 256, 9, 3, ok, 1 << 30, odd,
                                       *([null] * 4), null) == 1
    assert lib.moe_mxfp4_forward_profiled(*([ok] * 8), 4, 512, 256, 9, 3, ok, 1 << 30, null,
                                          P(0x1004), null) == 1
    assert lib.moe_mxfp4_forward_noalloc(*([null] * 8), 4, 512, 256, 9, 3, null) == 1
    assert lib.moe_mxfp4_forward_noalloc(*([ok] * 8), 1024, 7168, 256, 257, 9, null) == 3
    assert lib.moe_mxfp4_forward_persistent(*([null] * 8), 4, 512, 256, 9, 3, null, 1 << 30, null) == 1
    assert lib.moe_mxfp4_forward_persistent(*([ok] * 8), 64, 512, 256, 9, 3, ok, 1 << 30, null) == 2
    assert lib.moe_mxfp4_forward_persistent(*([ok] * 8), 4, 512, 256, 9, 3, ok, 16, null) == 3
    assert lib.moe_mxfp4_forward_splitk(*([null] * 8), 4, 512, 256, 9, 3, null, 1 << 30, null) == 1
    assert lib.moe_mxfp4_forward_splitk(*([ok] * 8), 64, 512, 256, 9, 3, ok, 1 << 30, null) == 2
    assert lib.moe_mxfp4_forward_splitk(*([ok] * 8), 4, 512, 256, 9, 3, ok, 16, null) == 3
    assert lib.moe_mxfp4_workspace_init(null, 256, null) == 1
    assert lib.moe_mxfp4_workspace_init(ok, 100, null) == 1
    assert lib.moe_mxfp4_workspace_init(ok, 0, null) == 0
    assert lib.moe_mxfp4_quantize(ok, 4, 33, ok, ok, null) == 1
    assert lib.moe_mxfp4_quantize(null, 4, 64, ok, ok, null) == 1
    assert lib.moe_mxfp4_quantize(ok, 0, 64, ok, ok, null) == 0
    assert lib.moe_mxfp4_route(ok, ok, 4, 8, 2, 24, ok, ok, ok, ok, null) == 1
    assert lib.moe_mxfp4_route(ok, ok, 4, 2000, 2, 16, ok, ok, ok, ok, null) == 2
    assert lib.moe_mxfp4_prepare_weights(*([ok] * 4), 2, 512, 256, *([null] * 4), null) == 1
    assert lib.moe_mxfp4_prepare_weights(*([ok] * 4), 2, 512, 256, *([ok] * 4), null) == 1
    print("library host code: all checks passed")
''')


def test_library_host_code_under_asan_ubsan(tmp_path):
    from mixture_experts_mxfp4_amd import build as hip_build
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(hip_build.hipcc()):
        pytest.skip("hipcc or its sanitizer runtime not found")
    others = [os.path.join(hip_build.BUILD, os.path.splitext(s)[0] + ".o")
              for s in hip_build.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        hip_build.build()
    obj, lib = str(tmp_path / "api_san.o"), str(tmp_path / "libmoe_mxfp4_san.so")
    host_san = []
    for f in SAN_FLAGS:
        host_san += ["-Xarch_host", f]       # host side only: no GPU code is instrumented
    flags = [f for f in hip_build.compile_flags() if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([hip_build.hipcc(), "-c", os.path.join(hip_build.CSRC, "api.hip"), "-o", obj,
                        *flags, *host_san], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([hip_build.hipcc(), "-shared", "-fPIC", f"--offload-arch={hip_build.ARCH}",
                        "-o", lib, obj, *others, "-Xarch_host", "-fsanitize=address,undefined",
                        "-shared-libsan"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    drv = tmp_path / "drive.py"
    drv.write_text(_DRIVER)
    env = dict(os.environ, LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, str(drv), lib], capture_output=True, text=True,
                       timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
