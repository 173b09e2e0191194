"""ctypes binding of libmoe_mxfp4.so (the C ABI in include/moe_mxfp4.h).

Argument marshalling only: every function takes torch tensors, checks their
dtype/shape/device, and passes raw device pointers, sizes and the current HIP
stream to the library function of the same name.  There is no fallback: if
the library is missing this module raises on import, and a non-zero status
raises MoeMxfp4Error.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mxfp4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_mxfp4_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t

_lib.moe_mxfp4_status_string.argtypes, _lib.moe_mxfp4_status_string.restype = [_I], ctypes.c_char_p
_lib.moe_mxfp4_workspace_bytes.argtypes = [_I] * 5
_lib.moe_mxfp4_workspace_bytes.restype = _SZ
_lib.moe_mxfp4_block_m.argtypes, _lib.moe_mxfp4_block_m.restype = [_I] * 5, _I
_lib.moe_mxfp4_path.argtypes, _lib.moe_mxfp4_path.restype = [_I] * 5, _I
_lib.moe_mxfp4_launch_count.argtypes, _lib.moe_mxfp4_launch_count.restype = [_I] * 5, _I
_lib.moe_mxfp4_route_capacity.argtypes = [_I] * 4
_lib.moe_mxfp4_route_capacity.restype = _I64
for _name in ("moe_mxfp4_prepare_weights", "moe_mxfp4_unprepare_weights"):
    getattr(_lib, _name).argtypes = [_P] * 4 + [_I] * 3 + [_P] * 4 + [_P]
    getattr(_lib, _name).restype = _I
_lib.moe_mxfp4_forward.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ, _P]
_lib.moe_mxfp4_forward.restype = _I
_lib.moe_mxfp4_forward_noalloc.argtypes = [_P] * 8 + [_I] * 5 + [_P]
_lib.moe_mxfp4_forward_noalloc.restype = _I
_lib.moe_mxfp4_forward_debug.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ] + [_P] * 5 + [_P]
_lib.moe_mxfp4_forward_debug.restype = _I
_lib.moe_mxfp4_forward_profiled.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ, _P, _P, _P]
_lib.moe_mxfp4_wall_clock_khz.argtypes, _lib.moe_mxfp4_wall_clock_khz.restype = [], _I
_lib.moe_mxfp4_mfma_probe.argtypes = [_I, _I, _P, _P, _P, _P]
_lib.moe_mxfp4_mfma_probe.restype = _I
_lib.moe_mxfp4_debug_mfma.argtypes = [_I, _I] + [_P] * 5 + [_P]
_lib.moe_mxfp4_debug_mfma.restype = _I
_lib.moe_mxfp4_stage1_workgroups.argtypes = [_I] * 5
_lib.moe_mxfp4_stage1_workgroups.restype = _I64
_lib.moe_mxfp4_forward_profiled.restype = _I
_lib.moe_mxfp4_quantize.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.moe_mxfp4_quantize.restype = _I
_lib.moe_mxfp4_route.argtypes = [_P, _P] + [_I] * 4 + [_P] * 4 + [_P]
_lib.moe_mxfp4_route.restype = _I
_lib.moe_mxfp4_a16w4_workspace_bytes.argtypes = [_I] * 5
_lib.moe_mxfp4_a16w4_workspace_bytes.restype = _SZ
_lib.moe_mxfp4_forward_a16w4.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ, _P]
_lib.moe_mxfp4_forward_a16w4.restype = _I
_lib.moe_mxfp4_forward_a16w4_debug.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ, _P, _P, _P, _P]
_lib.moe_mxfp4_forward_a16w4_debug.restype = _I
_lib.moe_mxfp4_persistent_workspace_bytes.argtypes = [_I] * 5
_lib.moe_mxfp4_persistent_workspace_bytes.restype = _SZ
_lib.moe_mxfp4_workspace_init.argtypes, _lib.moe_mxfp4_workspace_init.restype = [_P, _SZ, _P], _I
_lib.moe_mxfp4_persistent_workgroups.argtypes = [_I]
_lib.moe_mxfp4_persistent_workgroups.restype = _I64
_lib.moe_mxfp4_forward_persistent.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ, _P]
_lib.moe_mxfp4_forward_persistent.restype = _I
_lib.moe_mxfp4_forward_persistent_debug.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ] + [_P] * 5 + [_P]
_lib.moe_mxfp4_forward_persistent_debug.restype = _I
_lib.moe_mxfp4_splitk_workspace_bytes.argtypes = [_I] * 5
_lib.moe_mxfp4_splitk_workspace_bytes.restype = _SZ
_lib.moe_mxfp4_forward_splitk.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ, _P]
_lib.moe_mxfp4_forward_splitk.restype = _I
_lib.moe_mxfp4_forward_splitk_debug.argtypes = [_P] * 8 + [_I] * 5 + [_P, _SZ] + [_P] * 5 + [_P]
_lib.moe_mxfp4_forward_splitk_debug.restype = _I

EXPORTS = ("moe_mxfp4_status_string", "moe_mxfp4_workspace_bytes", "moe_mxfp4_block_m",
           "moe_mxfp4_path", "moe_mxfp4_launch_count",
           "moe_mxfp4_route_capacity", "moe_mxfp4_prepare_weights",
           "moe_mxfp4_unprepare_weights", "moe_mxfp4_forward", "moe_mxfp4_forward_noalloc",
           "moe_mxfp4_forward_debug",
           "moe_mxfp4_quantize", "moe_mxfp4_route", "moe_mxfp4_forward_profiled",
           "moe_mxfp4_wall_clock_khz", "moe_mxfp4_stage1_workgroups",
           "moe_mxfp4_a16w4_workspace_bytes", "moe_mxfp4_forward_a16w4",
           "moe_mxfp4_forward_a16w4_debug", "moe_mxfp4_persistent_workspace_bytes",
           "moe_mxfp4_workspace_init", "moe_mxfp4_persistent_workgroups",
           "moe_mxfp4_forward_persistent", "moe_mxfp4_forward_persistent_debug",
           "moe_mxfp4_splitk_workspace_bytes", "moe_mxfp4_forward_splitk",
           "moe_mxfp4_forward_splitk_debug", "moe_mxfp4_mfma_probe", "moe_mxfp4_debug_mfma")


class MoeMxfp4Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: status {status}: {moe_mxfp4_status_string(status)}")
        self.status = status


def _check(fn, status):
    if status != 0:
        raise MoeMxfp4Error(fn, status)


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(0)


def _ptr(t, dtype=None, shape=None, name="tensor", device=None):
    """Device pointer of t after checking what the kernels assume: a GPU tensor
    (on `device` when given), dtype, shape, contiguity.  A host tensor would
    hand a host address to a GPU kernel, so it is refused here."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor, got device {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device} like the other operands")
    return ctypes.c_void_p(t.data_ptr())


def moe_mxfp4_status_string(status: int) -> str:
    return _lib.moe_mxfp4_status_string(int(status)).decode()


def moe_mxfp4_workspace_bytes(M, D, I, E, topk) -> int:
    return int(_lib.moe_mxfp4_workspace_bytes(M, D, I, E, topk))


def moe_mxfp4_block_m(M, D, I, E, topk) -> int:
    return int(_lib.moe_mxfp4_block_m(M, D, I, E, topk))


PATH_DIRECT, PATH_STREAM, PATH_TILED = 1, 2, 3
PATH_NAMES = {PATH_DIRECT: "direct", PATH_STREAM: "stream", PATH_TILED: "tiled"}


def moe_mxfp4_path(M, D, I, E, topk) -> int:
    """Kernel path of the forward for this shape (PATH_DIRECT / _STREAM / _TILED; 0 if invalid)."""
    return int(_lib.moe_mxfp4_path(M, D, I, E, topk))


def moe_mxfp4_launch_count(M, D, I, E, topk) -> int:
    """Kernel launches of one forward for this shape (0 if invalid or M = 0)."""
    return int(_lib.moe_mxfp4_launch_count(M, D, I, E, topk))


def moe_mxfp4_route_capacity(M, E, topk, block_m) -> int:
    return int(_lib.moe_mxfp4_route_capacity(M, E, topk, block_m))


def _weight_dims(w13, w2):
    E, twoI, Dh = w13.shape
    return E, Dh * 2, twoI // 2


def _weight_ptrs(w13, w13s, w2, w2s, E, D, I, tag, device=None):
    u8 = torch.uint8
    return (_ptr(w13, u8, (E, 2 * I, D // 2), tag + "w13", device),
            _ptr(w13s, u8, (E, 2 * I, D // 32), tag + "w13_scale", device),
            _ptr(w2, u8, (E, D, I // 2), tag + "w2", device),
            _ptr(w2s, u8, (E, D, I // 32), tag + "w2_scale", device))


def moe_mxfp4_prepare_weights(w13, w13_scale, w2, w2_scale, w13_out=None, w13_scale_out=None,
                              w2_out=None, w2_scale_out=None, stream=None):
    """Raw MXFP4 weights -> kernel layout (same shapes).  Returns the 4 outputs."""
    E, D, I = _weight_dims(w13, w2)
    outs = [o if o is not None else torch.empty_like(i)
            for o, i in zip((w13_out, w13_scale_out, w2_out, w2_scale_out),
                            (w13, w13_scale, w2, w2_scale))]
    src = _weight_ptrs(w13, w13_scale, w2, w2_scale, E, D, I, "", w13.device)
    dst = _weight_ptrs(*outs, E, D, I, "out ", w13.device)
    _check("moe_mxfp4_prepare_weights",
           _lib.moe_mxfp4_prepare_weights(*src, E, D, I, *dst, _stream(stream)))
    return tuple(outs)


def moe_mxfp4_unprepare_weights(w13p, w13p_scale, w2p, w2p_scale, stream=None):
    E, D, I = _weight_dims(w13p, w2p)
    outs = [torch.empty_like(t) for t in (w13p, w13p_scale, w2p, w2p_scale)]
    src = _weight_ptrs(w13p, w13p_scale, w2p, w2p_scale, E, D, I, "", w13p.device)
    dst = _weight_ptrs(*outs, E, D, I, "out ", w13p.device)
    _check("moe_mxfp4_unprepare_weights",
           _lib.moe_mxfp4_unprepare_weights(*src, E, D, I, *dst, _stream(stream)))
    return tuple(outs)


def alloc_workspace(M, D, I, E, topk, device="cuda"):
    n = moe_mxfp4_workspace_bytes(M, D, I, E, topk)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace):
    E, D, I = _weight_dims(w13, w2)
    M = hidden.shape[0]
    topk = topk_ids.shape[1]
    dev = hidden.device
    args = (_ptr(hidden, torch.bfloat16, (M, D), "hidden"),
            *_weight_ptrs(w13, w13_scale, w2, w2_scale, E, D, I, "", dev),
            _ptr(topk_ids, torch.int32, (M, topk), "topk_ids", dev),
            _ptr(topk_w, torch.float32, (M, topk), "topk_w", dev),
            _ptr(out, torch.bfloat16, (M, D), "out", dev),
            M, D, I, E, topk, _ptr(workspace, torch.uint8, None, "workspace", dev),
            workspace.numel())
    return args, (M, D, I, E, topk)


def moe_mxfp4_forward(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out=None,
                      workspace=None, stream=None):
    """Fused MXFP4 MoE forward on prepared weights; returns out (bf16 [M, D])."""
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        E, D, I = _weight_dims(w13, w2)
        workspace = alloc_workspace(hidden.shape[0], D, I, E, topk_ids.shape[1], hidden.device)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward", _lib.moe_mxfp4_forward(*args, _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20      # MOE_MXFP4_NOALLOC_SCRATCH_BYTES


def moe_mxfp4_forward_noalloc(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out=None,
                              stream=None):
    """The forward on the library's static scratch array (no workspace, no
    allocation by the library; `out` is allocated here only when not given).
    Shapes whose workspace exceeds NOALLOC_SCRATCH_BYTES raise
    (MOE_MXFP4_ERR_WORKSPACE)."""
    if out is None:
        out = torch.empty_like(hidden)
    E, D, I = _weight_dims(w13, w2)
    M = hidden.shape[0]
    topk = topk_ids.shape[1]
    dev = hidden.device
    args = (_ptr(hidden, torch.bfloat16, (M, D), "hidden"),
            *_weight_ptrs(w13, w13_scale, w2, w2_scale, E, D, I, "", dev),
            _ptr(topk_ids, torch.int32, (M, topk), "topk_ids", dev),
            _ptr(topk_w, torch.float32, (M, topk), "topk_w", dev),
            _ptr(out, torch.bfloat16, (M, D), "out", dev), M, D, I, E, topk)
    _check("moe_mxfp4_forward_noalloc", _lib.moe_mxfp4_forward_noalloc(*args, _stream(stream)))
    return out


LAUNCHES = ("prologue", "stage1", "stage2", "reduce")
PATH_LAUNCHES = {PATH_DIRECT: (1, 2), PATH_STREAM: (0, 1, 2, 3), PATH_TILED: (0, 1, 2, 3)}


def moe_mxfp4_wall_clock_khz() -> int:
    """Frequency of the device clock that stage-1 spans are counted in."""
    return int(_lib.moe_mxfp4_wall_clock_khz())


def moe_mxfp4_mfma_probe(random_operands: bool, iters: int, stream=None, small_tile=False,
                         flags=None) -> dict:
    """Register-only FP4 MFMA rate on the current device: TFLOP/s, mean
    shader clock (MHz) and share of the per-clock FP4 peak.  small_tile: the
    16x16x128 instruction instead of 32x32x64.  flags, when given, is passed
    to the C call as it is (bit 0 random operands, bit 1 small tile)."""
    if flags is None:
        flags = int(bool(random_operands)) | (2 if small_tile else 0)
    tf, mhz, frac = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check("moe_mxfp4_mfma_probe",
           _lib.moe_mxfp4_mfma_probe(int(flags), int(iters), ctypes.byref(tf),
                                     ctypes.byref(mhz), ctypes.byref(frac), _stream(stream)))
    return {"tflops": tf.value, "shader_mhz": mhz.value, "per_clock_frac": frac.value}


def moe_mxfp4_debug_mfma(a, a_scales, b, b_scales, sel=0, stream=None):
    """One block-scaled FP4 MFMA: a, b uint8 [R, K/2] E2M1 codes, a_scales,
    b_scales uint8 [R, K/32] e8m0 (R x K = 16 x 128 or 32 x 64), on the GPU;
    returns A . B^T as float32 [R, R], the scales passed in byte `sel` of
    their words."""
    R = a.shape[0]
    if R not in (16, 32):
        raise ValueError("rows must be 16 or 32")
    K = 128 if R == 16 else 64
    dev = a.device
    pa = _ptr(a, torch.uint8, (R, K // 2), "a", dev)
    ps = _ptr(a_scales, torch.uint8, (R, K // 32), "a_scales", dev)
    pb = _ptr(b, torch.uint8, (R, K // 2), "b", dev)
    pbs = _ptr(b_scales, torch.uint8, (R, K // 32), "b_scales", dev)
    out = torch.empty((R, R), dtype=torch.float32, device=dev)
    _check("moe_mxfp4_debug_mfma",
           _lib.moe_mxfp4_debug_mfma(R, int(sel), pa, ps, pb, pbs, _ptr(out), _stream(stream)))
    return out


def moe_mxfp4_stage1_workgroups(M, D, I, E, topk) -> int:
    return int(_lib.moe_mxfp4_stage1_workgroups(M, D, I, E, topk))


def stage1_span_ms(records, khz):
    """Span (ms) of stage 1 from its per-workgroup [start, end] clock records."""
    r = records.reshape(-1, 2)
    return float((r[:, 1].max() - r[:, 0].min()).item()) / khz


def moe_mxfp4_forward_profiled(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out,
                               workspace, kernel_events, stage1_clock=None, stream=None):
    """Forward whose launches carry HIP events (raw hipEvent_t handles, ints or
    None): kernel_events[2*i], [2*i+1] = start, stop of launch i (LAUNCHES);
    see include/moe_mxfp4.h.  Launches a path does not make (PATH_LAUNCHES)
    leave their events unrecorded.  stage1_clock: None or a contiguous device
    int64 tensor of 2 * moe_mxfp4_stage1_workgroups(...) elements that
    receives every stage-1 workgroup's [start, end] clock (stage1_span_ms)."""
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    if len(kernel_events) != 2 * len(LAUNCHES):
        raise ValueError(f"kernel_events: expected {2 * len(LAUNCHES)} entries")
    ev = (ctypes.c_void_p * len(kernel_events))(
        *[ctypes.c_void_p(e) if e else None for e in kernel_events])
    clk = None
    if stage1_clock is not None:
        M, topk = topk_ids.shape
        E, D, I = _weight_dims(w13, w2)
        need = 2 * moe_mxfp4_stage1_workgroups(M, D, I, E, topk)
        if (stage1_clock.dtype != torch.int64 or stage1_clock.numel() < need
                or not stage1_clock.is_cuda or not stage1_clock.is_contiguous()):
            raise TypeError(f"stage1_clock: expected a contiguous device int64 tensor of {need}")
        clk = _ptr(stage1_clock, name="stage1_clock", device=hidden.device)
    _check("moe_mxfp4_forward_profiled",
           _lib.moe_mxfp4_forward_profiled(*args, ev, clk, _stream(stream)))
    return out


def moe_mxfp4_forward_debug(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out=None,
                            workspace=None, stream=None):
    """Forward that also returns its route list and intermediates (canonical layouts):
    dict(out, sorted_route, num_valid, h, a2_codes, a2_scales, block_m)."""
    E, D, I = _weight_dims(w13, w2)
    M, topk = topk_ids.shape
    dev = hidden.device
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        workspace = alloc_workspace(M, D, I, E, topk, dev)
    bm = moe_mxfp4_block_m(M, D, I, E, topk)
    cap = moe_mxfp4_route_capacity(M, E, topk, bm)
    sr = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    nv = torch.empty(4, dtype=torch.int32, device=dev)
    h = torch.empty((max(cap, 1), I), dtype=torch.bfloat16, device=dev)
    a2c = torch.empty((max(cap, 1), I // 2), dtype=torch.uint8, device=dev)
    a2s = torch.empty((max(cap, 1), I // 32), dtype=torch.uint8, device=dev)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward_debug",
           _lib.moe_mxfp4_forward_debug(*args, _ptr(sr), _ptr(nv), _ptr(h), _ptr(a2c), _ptr(a2s),
                                        _stream(stream)))
    return {"out": out, "sorted_route": sr[:cap], "num_valid": nv[:2], "h": h[:cap],
            "a2_codes": a2c[:cap], "a2_scales": a2s[:cap], "block_m": bm, "cap": cap,
            "path": moe_mxfp4_path(M, D, I, E, topk)}


def moe_mxfp4_quantize(x, codes=None, scales=None, stream=None):
    """bf16 [rows, cols] -> (codes u8 [rows, cols/2], scales u8 [rows, cols/32])."""
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check("moe_mxfp4_quantize",
           _lib.moe_mxfp4_quantize(_ptr(x, torch.bfloat16, (rows, cols), "x"), rows, cols,
                                   _ptr(codes, torch.uint8, (rows, cols // 2), "codes"),
                                   _ptr(scales, torch.uint8, (rows, cols // 32), "scales"),
                                   _stream(stream)))
    return codes, scales


def moe_mxfp4_route(topk_ids, topk_w, E, block_m, stream=None):
    """Route sort alone.  Returns dict(sorted_route, sorted_w, block_expert, num_valid, cap)."""
    M, topk = topk_ids.shape
    dev = topk_ids.device
    cap = moe_mxfp4_route_capacity(M, E, topk, block_m)
    sr = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    sw = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
    be = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    nv = torch.empty(2, dtype=torch.int32, device=dev)
    _check("moe_mxfp4_route",
           _lib.moe_mxfp4_route(_ptr(topk_ids, torch.int32, (M, topk), "topk_ids"),
                                _ptr(topk_w, torch.float32, (M, topk), "topk_w"),
                                M, E, topk, block_m, _ptr(sr), _ptr(sw), _ptr(be), _ptr(nv),
                                _stream(stream)))
    return {"sorted_route": sr[:cap], "sorted_w": sw[:cap], "block_expert": be[:cap // block_m],
            "num_valid": nv, "cap": cap}


def moe_mxfp4_a16w4_workspace_bytes(M, D, I, E, topk) -> int:
    """Workspace of the A16W4 forward (0: shape not supported by it)."""
    return int(_lib.moe_mxfp4_a16w4_workspace_bytes(M, D, I, E, topk))


def a16w4_stage1_workgroups(M, I, E, topk) -> int:
    return (I // 64) * min(E, M * topk) if M > 0 else 0


def alloc_workspace_a16w4(M, D, I, E, topk, device="cuda"):
    n = moe_mxfp4_a16w4_workspace_bytes(M, D, I, E, topk)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_mxfp4_forward_a16w4(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out=None,
                            workspace=None, stream=None):
    """A16W4 forward (bf16 activations, no activation quantization) on
    prepared weights; returns out (bf16 [M, D])."""
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        E, D, I = _weight_dims(w13, w2)
        workspace = alloc_workspace_a16w4(hidden.shape[0], D, I, E, topk_ids.shape[1],
                                          hidden.device)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward_a16w4", _lib.moe_mxfp4_forward_a16w4(*args, _stream(stream)))
    return out


def moe_mxfp4_forward_a16w4_debug(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w,
                                  out=None, workspace=None, h=None, kernel_events=None,
                                  stage1_clock=None, stream=None):
    """A16W4 forward with exports: h (bf16 [M*topk, I], by route; a tensor to
    fill, True to allocate one, or None), kernel_events (8 raw hipEvent_t
    handles or None, as in moe_mxfp4_forward_profiled) and stage1_clock
    (device int64 of 2 * a16w4_stage1_workgroups(...) or None).
    Returns dict(out, h)."""
    E, D, I = _weight_dims(w13, w2)
    M, topk = topk_ids.shape
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        workspace = alloc_workspace_a16w4(M, D, I, E, topk, hidden.device)
    if h is True:
        h = torch.empty((max(M * topk, 1), I), dtype=torch.bfloat16, device=hidden.device)
    hp = None
    if h is not None:
        if h.dtype != torch.bfloat16 or h.numel() < M * topk * I or not h.is_contiguous():
            raise TypeError(f"h: expected a contiguous bf16 tensor of {M * topk * I} elements")
        hp = _ptr(h, name="h", device=hidden.device)
    ev = None
    if kernel_events is not None:
        if len(kernel_events) != 2 * len(LAUNCHES):
            raise ValueError(f"kernel_events: expected {2 * len(LAUNCHES)} entries")
        ev = (ctypes.c_void_p * len(kernel_events))(
            *[ctypes.c_void_p(e) if e else None for e in kernel_events])
    clk = None
    if stage1_clock is not None:
        need = 2 * a16w4_stage1_workgroups(M, I, E, topk)
        if (stage1_clock.dtype != torch.int64 or stage1_clock.numel() < need
                or not stage1_clock.is_cuda or not stage1_clock.is_contiguous()):
            raise TypeError(f"stage1_clock: expected a contiguous device int64 tensor of {need}")
        clk = _ptr(stage1_clock, name="stage1_clock", device=hidden.device)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward_a16w4_debug",
           _lib.moe_mxfp4_forward_a16w4_debug(*args, hp, ev, clk, _stream(stream)))
    return {"out": out, "h": h[:M * topk] if h is not None else None}


def moe_mxfp4_persistent_workspace_bytes(M, D, I, E, topk) -> int:
    """Workspace of the persistent forward (0: shape not supported by it)."""
    return int(_lib.moe_mxfp4_persistent_workspace_bytes(M, D, I, E, topk))


def moe_mxfp4_workspace_init(workspace, stream=None):
    """Fill a workspace with zeros (enqueued): the persistent forward's set-up."""
    _check("moe_mxfp4_workspace_init",
           _lib.moe_mxfp4_workspace_init(_ptr(workspace, torch.uint8, None, "workspace"),
                                         workspace.numel(), _stream(stream)))


def moe_mxfp4_persistent_workgroups(M) -> int:
    return int(_lib.moe_mxfp4_persistent_workgroups(M))


def alloc_workspace_persistent(M, D, I, E, topk, device="cuda", stream=None):
    """A persistent-forward workspace, initialized."""
    n = moe_mxfp4_persistent_workspace_bytes(M, D, I, E, topk)
    if n == 0:
        raise MoeMxfp4Error("moe_mxfp4_persistent_workspace_bytes", 2)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_mxfp4_workspace_init(ws, stream)
    return ws


def persistent_error_word(workspace) -> int:
    """The workspace's barrier error word (nonzero after a timed-out wait)."""
    return int(workspace[4:8].view(torch.int32).item())


def moe_mxfp4_forward_persistent(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w,
                                 out=None, workspace=None, stream=None):
    """The forward in one persistent launch (few tokens); returns out."""
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        E, D, I = _weight_dims(w13, w2)
        workspace = alloc_workspace_persistent(hidden.shape[0], D, I, E, topk_ids.shape[1],
                                               hidden.device, stream)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward_persistent",
           _lib.moe_mxfp4_forward_persistent(*args, _stream(stream)))
    return out


def moe_mxfp4_forward_persistent_debug(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w,
                                       out=None, workspace=None, intermediates=True,
                                       kernel_events=None, clock=None, stream=None):
    """The persistent forward with exports: dict(out, h, a2_codes, a2_scales)
    by route (intermediates=True), kernel_events (8 raw hipEvent_t handles or
    None; the launch is entry pair 1) and clock (device int64 of
    2 * moe_mxfp4_persistent_workgroups(M), or None)."""
    E, D, I = _weight_dims(w13, w2)
    M, topk = topk_ids.shape
    dev = hidden.device
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        workspace = alloc_workspace_persistent(M, D, I, E, topk, dev, stream)
    R = max(M * topk, 1)
    h = a2c = a2s = None
    if intermediates:
        h = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        a2c = torch.empty((R, I // 2), dtype=torch.uint8, device=dev)
        a2s = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
    ev = None
    if kernel_events is not None:
        if len(kernel_events) != 2 * len(LAUNCHES):
            raise ValueError(f"kernel_events: expected {2 * len(LAUNCHES)} entries")
        ev = (ctypes.c_void_p * len(kernel_events))(
            *[ctypes.c_void_p(e) if e else None for e in kernel_events])
    clk = None
    if clock is not None:
        need = 2 * moe_mxfp4_persistent_workgroups(M)
        if (clock.dtype != torch.int64 or clock.numel() < need or not clock.is_cuda
                or not clock.is_contiguous()):
            raise TypeError(f"clock: expected a contiguous device int64 tensor of {need}")
        clk = _ptr(clock, name="clock", device=dev)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward_persistent_debug",
           _lib.moe_mxfp4_forward_persistent_debug(*args, _ptr(h), _ptr(a2c), _ptr(a2s), ev, clk,
                                                   _stream(stream)))
    return {"out": out, "h": h, "a2_codes": a2c, "a2_scales": a2s, "workspace": workspace}


def moe_mxfp4_splitk_workspace_bytes(M, D, I, E, topk) -> int:
    """Workspace of the split-K forward (0: shape not supported by it)."""
    return int(_lib.moe_mxfp4_splitk_workspace_bytes(M, D, I, E, topk))


def splitk_stage1_workgroups(M, I, E, topk) -> int:
    return 2 * (I // 64) * min(E, M * topk) if M > 0 else 0


def alloc_workspace_splitk(M, D, I, E, topk, device="cuda", stream=None):
    """A split-K forward workspace, zero-filled (its part counters start at zero)."""
    n = moe_mxfp4_splitk_workspace_bytes(M, D, I, E, topk)
    if n == 0:
        raise MoeMxfp4Error("moe_mxfp4_splitk_workspace_bytes", 2)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_mxfp4_workspace_init(ws, stream)
    return ws


def moe_mxfp4_forward_splitk(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out=None,
                             workspace=None, stream=None):
    """The forward with a split-K stage 1 (few tokens); returns out."""
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        E, D, I = _weight_dims(w13, w2)
        workspace = alloc_workspace_splitk(hidden.shape[0], D, I, E, topk_ids.shape[1],
                                           hidden.device, stream)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward_splitk", _lib.moe_mxfp4_forward_splitk(*args, _stream(stream)))
    return out


def moe_mxfp4_forward_splitk_debug(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w,
                                   out=None, workspace=None, intermediates=True,
                                   kernel_events=None, stage1_clock=None, stream=None):
    """The split-K forward with exports: dict(out, h, a2_codes, a2_scales,
    workspace); kernel_events / stage1_clock as in moe_mxfp4_forward_profiled
    (stage1_clock of 2 * splitk_stage1_workgroups(...) int64)."""
    E, D, I = _weight_dims(w13, w2)
    M, topk = topk_ids.shape
    dev = hidden.device
    if out is None:
        out = torch.empty_like(hidden)
    if workspace is None:
        workspace = alloc_workspace_splitk(M, D, I, E, topk, dev, stream)
    R = max(M * topk, 1)
    h = a2c = a2s = None
    if intermediates:
        h = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        a2c = torch.empty((R, I // 2), dtype=torch.uint8, device=dev)
        a2s = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
    ev = None
    if kernel_events is not None:
        if len(kernel_events) != 2 * len(LAUNCHES):
            raise ValueError(f"kernel_events: expected {2 * len(LAUNCHES)} entries")
        ev = (ctypes.c_void_p * len(kernel_events))(
            *[ctypes.c_void_p(e) if e else None for e in kernel_events])
    clk = None
    if stage1_clock is not None:
        need = 2 * splitk_stage1_workgroups(M, I, E, topk)
        if (stage1_clock.dtype != torch.int64 or stage1_clock.numel() < need
                or not stage1_clock.is_cuda or not stage1_clock.is_contiguous()):
            raise TypeError(f"stage1_clock: expected a contiguous device int64 tensor of {need}")
        clk = _ptr(stage1_clock, name="stage1_clock", device=dev)
    args, _ = _forward_args(hidden, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, workspace)
    _check("moe_mxfp4_forward_splitk_debug",
           _lib.moe_mxfp4_forward_splitk_debug(*args, _ptr(h), _ptr(a2c), _ptr(a2s), ev, clk,
                                               _stream(stream)))
    return {"out": out, "h": h, "a2_codes": a2c, "a2_scales": a2s, "workspace": workspace}


class MoeMxfp4:
    """Holds prepared weights and a workspace; calling it runs the forward."""

    def __init__(self, w13, w13_scale, w2, w2_scale, stream=None):
        self.E, self.D, self.I = _weight_dims(w13, w2)
        self.weights = moe_mxfp4_prepare_weights(w13, w13_scale, w2, w2_scale, stream=stream)
        self._ws = None

    def workspace(self, M, topk, device):
        n = moe_mxfp4_workspace_bytes(M, self.D, self.I, self.E, topk)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
        return self._ws

    def __call__(self, hidden, topk_ids, topk_w, out=None, stream=None):
        ws = self.workspace(hidden.shape[0], topk_ids.shape[1], hidden.device)
        return moe_mxfp4_forward(hidden, *self.weights, topk_ids, topk_w, out=out, workspace=ws,
                                 stream=stream)
