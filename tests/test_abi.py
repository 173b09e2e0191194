"""The C-ABI library loads and exports every declared symbol; host-side sizing
and validation behave as documented.  No kernel is launched (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")


@pytest.fixture(scope="module")
def binding():
    from mixture_experts_mxfp4_amd import binding as b
    return b


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_mxfp4_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_mxfp4_prepare_weights", "moe_mxfp4_forward",
                     "moe_mxfp4_workspace_bytes", "moe_mxfp4_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(binding):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(binding.LIB_PATH)
    for n in declared_functions():
        assert getattr(lib, n) is not None
    assert set(binding.EXPORTS) == set(declared_functions())


def test_library_links_no_torch(binding):
    # the library's own dependency list (DT_NEEDED), read statically
    out = subprocess.run(["readelf", "-d", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out)
    assert any(n.startswith("libamdhip64") for n in needed), needed
    assert not any("torch" in n or "c10" in n for n in needed), needed


def test_status_strings(binding):
    for s in range(5):
        assert binding.moe_mxfp4_status_string(s)
    assert binding.moe_mxfp4_status_string(99) == "unknown status"


def test_block_m_and_capacity(binding):
    assert binding.moe_mxfp4_block_m(16, 7168, 256, 257, 9) == 16
    assert binding.moe_mxfp4_block_m(64, 7168, 2048, 33, 9) == 32
    assert binding.moe_mxfp4_block_m(4096, 7168, 2048, 33, 9) == 256
    assert binding.moe_mxfp4_block_m(1024, 7168, 256, 257, 9) == 32    # paired blocks
    assert binding.moe_mxfp4_block_m(1024, 7168, 2048, 257, 9) == 64
    assert binding.moe_mxfp4_block_m(1700, 7168, 256, 257, 9) == 64
    assert binding.moe_mxfp4_block_m(16, 7168, 100, 257, 9) == 0       # I % 256 != 0
    for M, E, k, bm in [(16, 257, 9, 16), (1, 1, 1, 16), (4096, 33, 9, 64), (3, 500, 2, 32)]:
        cap = binding.moe_mxfp4_route_capacity(M, E, k, bm)
        assert cap % bm == 0
        # every expert with n routes pads to ceil(n/bm)*bm: worst case bounded by cap
        assert cap >= M * k + min(E, M * k) * (bm - 1)
    assert binding.moe_mxfp4_route_capacity(0, 8, 2, 16) == 0


def test_path_choice(binding):
    assert binding.moe_mxfp4_path(16, 7168, 256, 257, 9) == binding.PATH_DIRECT
    assert binding.moe_mxfp4_path(8, 512, 256, 9, 3) == binding.PATH_DIRECT
    assert binding.moe_mxfp4_path(64, 7168, 2048, 33, 9) == binding.PATH_STREAM
    assert binding.moe_mxfp4_path(1024, 7168, 256, 257, 9) == binding.PATH_STREAM
    assert binding.moe_mxfp4_path(200, 512, 256, 257, 9) == binding.PATH_STREAM
    assert binding.moe_mxfp4_path(4096, 7168, 2048, 33, 9) == binding.PATH_TILED
    # from 64 routes per expert on average the tiled kernels are chosen
    assert binding.moe_mxfp4_path(512, 7168, 2048, 33, 9) == binding.PATH_TILED
    assert binding.moe_mxfp4_path(128, 7168, 512, 33, 9) == binding.PATH_STREAM
    assert binding.moe_mxfp4_path(16, 7000, 256, 257, 9) == 0


def test_workspace_bytes(binding):
    # route-indexed path: at least h in MXFP4 for every route
    assert binding.moe_mxfp4_workspace_bytes(16, 7168, 256, 257, 9) >= 16 * 9 * (128 + 8)
    # sorted paths: at least the bf16 contribution of every route
    assert binding.moe_mxfp4_workspace_bytes(64, 7168, 2048, 33, 9) >= 64 * 9 * 7168 * 2
    assert binding.moe_mxfp4_workspace_bytes(16, 7000, 256, 257, 9) == 0
    assert binding.moe_mxfp4_workspace_bytes(16, 7168, 256, 2000, 9) == 0     # E > 1024


def test_tiled_path_offset_limits(binding):
    """The LDS-tiled kernels use 32-bit per-lane offsets: an expert's gate_up
    codes (I*D bytes) below 2^31 and the sorted operands' scale words below
    2^32; beyond that every shape query reports the shape unsupported and the
    forward refuses it before touching the device."""
    M, E, k = 4096, 33, 9
    assert binding.moe_mxfp4_path(M, 7168, 2048, E, k) == binding.PATH_TILED
    assert binding.moe_mxfp4_path(M, 65536, 65536, E, k) == 0              # I*D = 2^32
    assert binding.moe_mxfp4_workspace_bytes(M, 65536, 65536, E, k) == 0
    assert binding.moe_mxfp4_path(M, 65536, 32512, E, k) == binding.PATH_TILED   # I*D < 2^31
    assert binding.moe_mxfp4_path(M, 65536, 32768, E, k) == 0              # I*D = 2^31
    # the other paths keep 64-bit addressing: a streaming shape of the same dims is fine
    assert binding.moe_mxfp4_path(64, 65536, 65536, E, k) == binding.PATH_STREAM
    # scale words: 65536/128 K tiles x cap rows x 4 bytes >= 2^32 for a very long route list
    big = 1 << 21
    assert binding.moe_mxfp4_path(big, 65536, 256, E, 8) == 0
    assert binding.moe_mxfp4_path(big, 7168, 256, E, 8) == binding.PATH_TILED
    lib = ctypes.CDLL(binding.LIB_PATH)
    lib.moe_mxfp4_forward.argtypes = binding._lib.moe_mxfp4_forward.argtypes
    lib.moe_mxfp4_forward.restype = ctypes.c_int
    ok = ctypes.c_void_p(0x1000)
    assert lib.moe_mxfp4_forward(*([ok] * 8), M, 65536, 65536, E, k, ok, 1 << 40,
                                 ctypes.c_void_p(0)) == 2


def test_noalloc_host_validation_without_device(binding):
    """The forward without a workspace refuses bad arguments, and shapes whose
    workspace exceeds its static scratch array, before touching a device."""
    lib = ctypes.CDLL(binding.LIB_PATH)
    lib.moe_mxfp4_forward_noalloc.argtypes = binding._lib.moe_mxfp4_forward_noalloc.argtypes
    lib.moe_mxfp4_forward_noalloc.restype = ctypes.c_int
    null, ok = ctypes.c_void_p(0), ctypes.c_void_p(0x1000)
    assert lib.moe_mxfp4_forward_noalloc(*([null] * 8), 4, 512, 256, 9, 3, null) == 1
    assert lib.moe_mxfp4_forward_noalloc(*([ok] * 8), 4, 500, 256, 9, 3, null) == 1
    assert lib.moe_mxfp4_forward_noalloc(*([ok] * 8), 0, 512, 256, 9, 3, null) == 0
    limit = binding.NOALLOC_SCRATCH_BYTES
    assert binding.moe_mxfp4_workspace_bytes(1024, 7168, 256, 257, 9) > limit
    assert lib.moe_mxfp4_forward_noalloc(*([ok] * 8), 1024, 7168, 256, 257, 9, null) == 3
    assert binding.moe_mxfp4_workspace_bytes(16, 7168, 256, 257, 9) <= limit
    assert binding.moe_mxfp4_workspace_bytes(64, 7168, 2048, 33, 9) <= limit
    text = open(HEADER).read()
    assert f"MOE_MXFP4_NOALLOC_SCRATCH_BYTES (32u << 20)" in text and limit == 32 << 20


def test_host_validation_without_device(binding):
    lib = ctypes.CDLL(binding.LIB_PATH)
    lib.moe_mxfp4_forward.argtypes = binding._lib.moe_mxfp4_forward.argtypes
    lib.moe_mxfp4_forward.restype = ctypes.c_int
    null = ctypes.c_void_p(0)
    # null pointers with M > 0 -> invalid argument, before touching the device
    assert lib.moe_mxfp4_forward(*([null] * 8), 4, 512, 256, 9, 3, null, 1 << 30, null) == 1
    # bad dims
    assert lib.moe_mxfp4_forward(*([null] * 8), 4, 500, 256, 9, 3, null, 1 << 30, null) == 1
    assert lib.moe_mxfp4_forward(*([null] * 8), 4, 512, 256, 0, 3, null, 1 << 30, null) == 1
    assert lib.moe_mxfp4_forward(*([null] * 8), 4, 512, 256, 9, 33, null, 1 << 30, null) == 1
    # M = 0 is a no-op
    assert lib.moe_mxfp4_forward(*([null] * 8), 0, 512, 256, 9, 3, null, 0, null) == 0
    # misaligned pointers
    fake = ctypes.c_void_p(0x1000 + 8)
    ok = ctypes.c_void_p(0x1000)
    args = [fake] + [ok] * 7
    assert lib.moe_mxfp4_forward(*args, 4, 512, 256, 9, 3, ok, 1 << 30, null) == 1
    # workspace too small
    args = [ok] * 8
    assert lib.moe_mxfp4_forward(*args, 4, 512, 256, 9, 3, ok, 16, null) == 3
    lib.moe_mxfp4_quantize.argtypes = binding._lib.moe_mxfp4_quantize.argtypes
    assert lib.moe_mxfp4_quantize(ok, 4, 33, ok, ok, null) == 1
    lib.moe_mxfp4_route.argtypes = binding._lib.moe_mxfp4_route.argtypes
    assert lib.moe_mxfp4_route(ok, ok, 4, 8, 2, 24, ok, ok, ok, ok, null) == 1    # block_m 24
    lib.moe_mxfp4_prepare_weights.argtypes = binding._lib.moe_mxfp4_prepare_weights.argtypes
    assert lib.moe_mxfp4_prepare_weights(*([ok] * 4), 2, 512, 256, *([null] * 4), null) == 1
    # in-place (aliasing) prepare is rejected
    assert lib.moe_mxfp4_prepare_weights(*([ok] * 4), 2, 512, 256, *([ok] * 4), null) == 1
    # the MFMA probe: unknown flag bits, iteration counts out of range and null outputs
    lib.moe_mxfp4_mfma_probe.argtypes = binding._lib.moe_mxfp4_mfma_probe.argtypes
    d = [ctypes.c_double() for _ in range(3)]
    outs = [ctypes.byref(x) for x in d]
    for flags, iters in ((4, 100), (-1, 100), (0, 0), (3, (1 << 24) + 1)):
        assert lib.moe_mxfp4_mfma_probe(flags, iters, *outs, null) == 1
    assert lib.moe_mxfp4_mfma_probe(1, 100, null, outs[1], outs[2], null) == 1


def test_a16w4_sizing_and_validation(binding):
    # bf16 h for every route plus the expert slot tables; 0 where the A16W4
    # forward does not run (M > 32, M*topk > 1024, topk > 16) or a bad shape
    assert binding.moe_mxfp4_a16w4_workspace_bytes(16, 7168, 256, 257, 9) >= 16 * 9 * 256 * 2
    assert binding.moe_mxfp4_a16w4_workspace_bytes(32, 7168, 2048, 33, 9) >= 32 * 9 * 2048 * 2
    assert binding.moe_mxfp4_a16w4_workspace_bytes(33, 7168, 256, 257, 9) == 0
    assert binding.moe_mxfp4_a16w4_workspace_bytes(8, 512, 256, 9, 17) == 0
    assert binding.moe_mxfp4_a16w4_workspace_bytes(16, 7000, 256, 257, 9) == 0
    assert binding.a16w4_stage1_workgroups(16, 256, 257, 9) == 4 * 144
    lib = ctypes.CDLL(binding.LIB_PATH)
    f = lib.moe_mxfp4_forward_a16w4
    f.argtypes = binding._lib.moe_mxfp4_forward_a16w4.argtypes
    f.restype = ctypes.c_int
    null, ok = ctypes.c_void_p(0), ctypes.c_void_p(0x1000)
    assert f(*([null] * 8), 4, 512, 256, 9, 3, null, 1 << 30, null) == 1      # null pointers
    assert f(*([null] * 8), 33, 512, 256, 9, 3, null, 1 << 30, null) == 2     # M > 32
    assert f(*([null] * 8), 0, 512, 256, 9, 3, null, 0, null) == 0            # M = 0
    assert f(*([ok] * 8), 4, 512, 256, 9, 3, ok, 16, null) == 3               # short workspace
    g = lib.moe_mxfp4_forward_a16w4_debug
    g.argtypes = binding._lib.moe_mxfp4_forward_a16w4_debug.argtypes
    g.restype = ctypes.c_int
    odd = ctypes.c_void_p(0x1000 + 8)
    assert g(*([ok] * 8), 4, 512, 256, 9, 3, ok, 1 << 30, odd, null, null, null) == 1


def test_binding_refuses_wrong_dtypes(binding):
    import torch
    h = torch.zeros(2, 512, dtype=torch.float32)
    with pytest.raises(TypeError):
        binding._ptr(h, torch.bfloat16, (2, 512), "hidden")


def test_binding_refuses_host_tensors():
    """Tensors on the host would give the kernels host addresses: the binding
    raises before any call into the library."""
    import pytest
    import torch
    from mixture_experts_mxfp4_amd import binding
    M, D, I, E, k = 4, 512, 256, 9, 3
    u8 = torch.uint8
    w = [torch.zeros(s, dtype=u8) for s in ((E, 2 * I, D // 2), (E, 2 * I, D // 32),
                                            (E, D, I // 2), (E, D, I // 32))]
    hidden = torch.zeros((M, D), dtype=torch.bfloat16)
    ids = torch.zeros((M, k), dtype=torch.int32)
    tw = torch.ones((M, k), dtype=torch.float32)
    ws = torch.empty(binding.moe_mxfp4_workspace_bytes(M, D, I, E, k), dtype=u8)
    with pytest.raises(ValueError, match="GPU tensor"):
        binding.moe_mxfp4_forward(hidden, *w, ids, tw, workspace=ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        binding.moe_mxfp4_prepare_weights(*w)
    with pytest.raises(ValueError, match="GPU tensor"):
        binding.moe_mxfp4_quantize(hidden)


def test_launch_count():
    """Launches per forward by path: 2 route-indexed; 4 streaming (one
    prologue launch: the sort, on a workgroup per 2,048-route chunk above 768 routes, and the activation
    quantization); tiled one more (the sorted copy of the activations)."""
    from mixture_experts_mxfp4_amd import binding
    assert binding.moe_mxfp4_launch_count(16, 7168, 256, 257, 9) == 2        # decode
    assert binding.moe_mxfp4_launch_count(64, 7168, 2048, 33, 9) == 4        # small batch
    assert binding.moe_mxfp4_launch_count(1024, 7168, 256, 257, 9) == 4      # prefill
    assert binding.moe_mxfp4_launch_count(4096, 7168, 2048, 33, 9) == 5      # large prefill
    assert binding.moe_mxfp4_launch_count(1000, 768, 512, 3, 2) == 5         # tiled, one chunk
    assert binding.moe_mxfp4_launch_count(0, 7168, 256, 257, 9) == 0
    assert binding.moe_mxfp4_launch_count(16, 7000, 256, 257, 9) == 0        # D % 256 != 0
