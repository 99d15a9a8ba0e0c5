"""Python binding of libgrinqh.so (the C ABI in include/grinqh.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libgrinqh.so.  PyTorch supplies device memory and the stream.
The functions with the C names take a grinqh_layout and caller-allocated
tensors, exactly like the C calls; the short names (pack, assign_bits, gemv,
debug_codes) allocate their outputs with torch and call the same entry points.
There is no CPU fallback: a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgrinqh.so")

GRINQH_OK, GRINQH_EINVAL, GRINQH_EALIGN, GRINQH_ENOSPACE, GRINQH_ENODEV, GRINQH_EDEVICE = range(6)
GRINQH_BF16, GRINQH_F32 = 0, 1


class GrinqhError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} (status {status})")


class Layout(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32), ("b_max", ctypes.c_int32),
                ("n_planes", ctypes.c_int32), ("row_words", ctypes.c_int32)]

    def __repr__(self):
        return (f"Layout(d_in={self.d_in}, d_out={self.d_out}, b_max={self.b_max}, "
                f"n_planes={self.n_planes}, row_words={self.row_words})")


class Operands(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("theta", ctypes.c_void_p), ("planes", ctypes.c_void_p),
                ("s", ctypes.c_void_p), ("z", ctypes.c_void_p), ("y", ctypes.c_void_p)]


MAX_GROUP = 8

EXPORTS = ("grinqh_version", "grinqh_status_string", "grinqh_layout_init", "grinqh_packed_bytes",
           "grinqh_gemv_workspace_bytes", "grinqh_pack", "grinqh_assign_bits", "grinqh_gemv",
           "grinqh_gemv_group_workspace_bytes", "grinqh_gemv_group", "grinqh_debug_codes",
           "grinqh_debug_force_launch", "grinqh_gemv_noalloc",
           "grinqh_calibrate_workspace_bytes", "grinqh_calibrate_thresholds", "grinqh_quantize_rtn",
           "grinqh_prefill_workspace_bytes", "grinqh_prefill_gemm")

_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libgrinqh.so (built in-tree by input_adaptive_bit_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # Bind to the HIP runtime torch already uses (same soname), so that streams
    # and device pointers handed over by torch belong to the runtime we call.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m input_adaptive_bit_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    LP = ctypes.POINTER(Layout)
    lib.grinqh_version.argtypes = []
    lib.grinqh_version.restype = i32
    lib.grinqh_status_string.argtypes = [ctypes.c_int]
    lib.grinqh_status_string.restype = ctypes.c_char_p
    lib.grinqh_layout_init.argtypes = [i32, i32, i32, LP]
    lib.grinqh_layout_init.restype = ctypes.c_int
    lib.grinqh_packed_bytes.argtypes = [LP]
    lib.grinqh_packed_bytes.restype = sz
    lib.grinqh_gemv_workspace_bytes.argtypes = [LP]
    lib.grinqh_gemv_workspace_bytes.restype = sz
    lib.grinqh_pack.argtypes = [LP, vp, vp, vp]
    lib.grinqh_pack.restype = ctypes.c_int
    lib.grinqh_assign_bits.argtypes = [LP, vp, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.grinqh_assign_bits.restype = ctypes.c_int
    lib.grinqh_gemv.argtypes = [LP, vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.grinqh_gemv.restype = ctypes.c_int
    OP = ctypes.POINTER(Operands)
    lib.grinqh_gemv_group_workspace_bytes.argtypes = [LP, i32]
    lib.grinqh_gemv_group_workspace_bytes.restype = sz
    lib.grinqh_gemv_group.argtypes = [LP, OP, i32, ctypes.c_int, ctypes.c_int, vp, sz, vp]
    lib.grinqh_gemv_group.restype = ctypes.c_int
    lib.grinqh_debug_codes.argtypes = [LP, vp, vp, vp, vp]
    lib.grinqh_debug_codes.restype = ctypes.c_int
    lib.grinqh_gemv_noalloc.argtypes = [LP, vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.grinqh_gemv_noalloc.restype = ctypes.c_int
    lib.grinqh_debug_force_launch.argtypes = [i32, i32, i32]
    lib.grinqh_debug_force_launch.restype = ctypes.c_int
    lib.grinqh_calibrate_workspace_bytes.argtypes = []
    lib.grinqh_calibrate_workspace_bytes.restype = sz
    lib.grinqh_calibrate_thresholds.argtypes = [vp, ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_double),
                                                i32, vp, vp, sz, vp]
    lib.grinqh_calibrate_thresholds.restype = ctypes.c_int
    lib.grinqh_quantize_rtn.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.grinqh_quantize_rtn.restype = ctypes.c_int
    lib.grinqh_prefill_workspace_bytes.argtypes = [i32]
    lib.grinqh_prefill_workspace_bytes.restype = sz
    lib.grinqh_prefill_gemm.argtypes = [LP, vp, ctypes.c_int, i32, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.grinqh_prefill_gemm.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().grinqh_status_string(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != GRINQH_OK:
        raise GrinqhError(status, call)


# ------------------------------------------------------------------ host ----

def grinqh_layout_init(d_in: int, d_out: int, b_max: int) -> Layout:
    L = Layout()
    _check(load().grinqh_layout_init(int(d_in), int(d_out), int(b_max), ctypes.byref(L)),
           "grinqh_layout_init")
    return L


def grinqh_packed_bytes(L: Layout) -> int:
    return int(load().grinqh_packed_bytes(ctypes.byref(L)))


def grinqh_gemv_workspace_bytes(L: Layout) -> int:
    return int(load().grinqh_gemv_workspace_bytes(ctypes.byref(L)))


# --------------------------------------------------------------- device -----

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GRINQH_BF16
    if t.dtype == torch.float32:
        return GRINQH_F32
    raise TypeError(f"x/y must be bfloat16 or float32, not {t.dtype}")


def _need(t, name, dtypes, numel=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() * t.element_size() < numel:
        raise ValueError(f"{name} is too small ({t.numel() * t.element_size()} < {numel} bytes)")


def grinqh_pack(L: Layout, q, planes, stream=None) -> None:
    import torch
    _need(q, "q", (torch.uint8,), L.d_out * L.d_in)
    _need(planes, "planes", (torch.int32, torch.uint32), grinqh_packed_bytes(L))
    _check(load().grinqh_pack(ctypes.byref(L), _ptr(q), _ptr(planes), _stream(stream)), "grinqh_pack")


def grinqh_assign_bits(L: Layout, x, theta, bits, active_idx=None, n_active=None, stream=None) -> None:
    import torch
    _need(x, "x", (torch.bfloat16, torch.float32), L.d_in * x.element_size())
    _need(theta, "theta", (torch.float32,), 4 * L.n_planes)
    _need(bits, "bits", (torch.uint8,), L.d_in)
    if active_idx is not None:
        _need(active_idx, "active_idx", (torch.int32,), 4 * L.d_in)
    if n_active is not None:
        _need(n_active, "n_active", (torch.int32,), 4)
    _check(load().grinqh_assign_bits(ctypes.byref(L), _ptr(x), _dtype_code(x), _ptr(theta), _ptr(bits),
                                     _ptr(active_idx), _ptr(n_active), _stream(stream)),
           "grinqh_assign_bits")


def grinqh_gemv(L: Layout, x, theta, planes, s, z, y, workspace, stream=None) -> None:
    import torch
    _need(x, "x", (torch.bfloat16, torch.float32), L.d_in * x.element_size())
    _need(theta, "theta", (torch.float32,), 4 * L.n_planes)
    _need(planes, "planes", (torch.int32, torch.uint32), grinqh_packed_bytes(L))
    _need(s, "s", (torch.float16,), 2 * L.d_out)
    _need(z, "z", (torch.float16,), 2 * L.d_out)
    _need(y, "y", (torch.bfloat16, torch.float32), L.d_out * y.element_size())
    _need(workspace, "workspace", None)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().grinqh_gemv(ctypes.byref(L), _ptr(x), _dtype_code(x), _ptr(theta), _ptr(planes),
                              _ptr(s), _ptr(z), _ptr(y), _dtype_code(y), _ptr(workspace), ws_bytes,
                              _stream(stream)),
           "grinqh_gemv")


NOALLOC_SCRATCH_BYTES = 1 << 20


def grinqh_gemv_noalloc(L: Layout, x, theta, planes, s, z, y, stream=None) -> None:
    """grinqh_gemv with the library's static device workspace (no workspace
    argument; the call allocates nothing)."""
    import torch
    _need(x, "x", (torch.bfloat16, torch.float32), L.d_in * x.element_size())
    _need(theta, "theta", (torch.float32,), 4 * L.n_planes)
    _need(planes, "planes", (torch.int32, torch.uint32), grinqh_packed_bytes(L))
    _need(s, "s", (torch.float16,), 2 * L.d_out)
    _need(z, "z", (torch.float16,), 2 * L.d_out)
    _need(y, "y", (torch.bfloat16, torch.float32), L.d_out * y.element_size())
    _check(load().grinqh_gemv_noalloc(ctypes.byref(L), _ptr(x), _dtype_code(x), _ptr(theta), _ptr(planes),
                                      _ptr(s), _ptr(z), _ptr(y), _dtype_code(y), _stream(stream)),
           "grinqh_gemv_noalloc")


def grinqh_gemv_group_workspace_bytes(layouts) -> int:
    arr = (Layout * len(layouts))(*layouts)
    return int(load().grinqh_gemv_group_workspace_bytes(arr, len(layouts)))


def grinqh_gemv_group(layouts, operands, workspace, stream=None) -> None:
    """operands: one (x, theta, planes, s, z, y) tuple of tensors per layout."""
    import torch
    n = len(layouts)
    if n != len(operands):
        raise ValueError("one operand tuple per layout")
    ops = (Operands * n)()
    for k, (L, (x, theta, planes, s, z, y)) in enumerate(zip(layouts, operands)):
        _need(x, "x", (torch.bfloat16, torch.float32), L.d_in * x.element_size())
        _need(theta, "theta", (torch.float32,), 4 * L.n_planes)
        _need(planes, "planes", (torch.int32, torch.uint32), grinqh_packed_bytes(L))
        _need(s, "s", (torch.float16,), 2 * L.d_out)
        _need(z, "z", (torch.float16,), 2 * L.d_out)
        _need(y, "y", (torch.bfloat16, torch.float32), L.d_out * y.element_size())
        if _dtype_code(x) != _dtype_code(operands[0][0]) or _dtype_code(y) != _dtype_code(operands[0][5]):
            raise TypeError("every member of a group shares the x and y dtypes")
        ops[k] = Operands(_ptr(x), _ptr(theta), _ptr(planes), _ptr(s), _ptr(z), _ptr(y))
    _need(workspace, "workspace", None)
    arr = (Layout * n)(*layouts)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().grinqh_gemv_group(arr, ops, n, _dtype_code(operands[0][0]), _dtype_code(operands[0][5]),
                                    _ptr(workspace), ws_bytes, _stream(stream)),
           "grinqh_gemv_group")


def grinqh_debug_codes(L: Layout, bits, planes, codes, stream=None) -> None:
    import torch
    _need(bits, "bits", (torch.uint8,), L.d_in)
    _need(planes, "planes", (torch.int32, torch.uint32), grinqh_packed_bytes(L))
    _need(codes, "codes", (torch.uint8,), L.d_in * L.d_out)
    _check(load().grinqh_debug_codes(ctypes.byref(L), _ptr(bits), _ptr(planes), _ptr(codes),
                                     _stream(stream)),
           "grinqh_debug_codes")


def grinqh_debug_force_launch(lane_groups: int, chunk: int, prefill_tile: int) -> None:
    _check(load().grinqh_debug_force_launch(int(lane_groups), int(chunk), int(prefill_tile)),
           "grinqh_debug_force_launch")


_PREFILL_TILE_CODES = {0: 0, (128, 128): 1, (256, 128): 2, (256, 256): 3}


def force_launch_shape(lane_groups: int = 0, chunk: int = 0, prefill_tile=0) -> None:
    """Force the GEMV tile width (lane groups per wave), slice length and the
    prefill tile ((tokens, outputs) or 0) of later calls; 0 = automatic."""
    grinqh_debug_force_launch(lane_groups, chunk, _PREFILL_TILE_CODES[prefill_tile])


def grinqh_calibrate_workspace_bytes() -> int:
    return int(load().grinqh_calibrate_workspace_bytes())


def grinqh_calibrate_thresholds(x, levels, theta, workspace, stream=None) -> None:
    """Thresholds as quantiles of the pooled |x| (x: bf16 or fp32 tensor of any
    shape, contiguous; levels: host sequence of 1..4 levels in [0, 1];
    theta: fp32 tensor [len(levels)])."""
    import torch
    _need(x, "x", (torch.bfloat16, torch.float32), None)
    lv = (ctypes.c_double * len(levels))(*[float(q) for q in levels])
    _need(theta, "theta", (torch.float32,), 4 * len(levels))
    _need(workspace, "workspace", None)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().grinqh_calibrate_thresholds(_ptr(x), _dtype_code(x), x.numel(), lv, len(levels), _ptr(theta),
                                              _ptr(workspace), ws_bytes, _stream(stream)),
           "grinqh_calibrate_thresholds")


def grinqh_quantize_rtn(w, b_max: int, q, s, z, stream=None) -> None:
    """RTN codes (uint8 [d_out][d_in]), scales and zero points (fp16 [d_out])
    of a bf16 weight matrix w [d_out][d_in]."""
    import torch
    if w.dim() != 2:
        raise ValueError("w must be 2-D [d_out][d_in]")
    d_out, d_in = w.shape
    _need(w, "w", (torch.bfloat16,), None)
    _need(q, "q", (torch.uint8,), d_out * d_in)
    _need(s, "s", (torch.float16,), 2 * d_out)
    _need(z, "z", (torch.float16,), 2 * d_out)
    _check(load().grinqh_quantize_rtn(d_in, d_out, int(b_max), _ptr(w), _ptr(q), _ptr(s), _ptr(z), _stream(stream)),
           "grinqh_quantize_rtn")


def grinqh_prefill_workspace_bytes(M: int) -> int:
    return int(load().grinqh_prefill_workspace_bytes(int(M)))


def grinqh_prefill_gemm(L: Layout, x, planes, s, z, y, workspace, stream=None) -> None:
    """Prefill-stage dense b_max GEMM: x bf16 [M][d_in] -> y [M][d_out]."""
    import torch
    if x.dim() != 2 or y.dim() != 2 or x.shape[1] != L.d_in or y.shape[1] != L.d_out or x.shape[0] != y.shape[0]:
        raise ValueError("x must be [M][d_in] and y [M][d_out]")
    M = x.shape[0]
    _need(x, "x", (torch.bfloat16,), M * L.d_in * 2)
    _need(planes, "planes", (torch.int32, torch.uint32), grinqh_packed_bytes(L))
    _need(s, "s", (torch.float16,), 2 * L.d_out)
    _need(z, "z", (torch.float16,), 2 * L.d_out)
    _need(y, "y", (torch.bfloat16, torch.float32), M * L.d_out * y.element_size())
    _need(workspace, "workspace", None)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().grinqh_prefill_gemm(ctypes.byref(L), _ptr(x), _dtype_code(x), M, _ptr(planes), _ptr(s), _ptr(z),
                                      _ptr(y), _dtype_code(y), _ptr(workspace), ws_bytes, _stream(stream)),
           "grinqh_prefill_gemm")


# ------------------------------------------------- allocating conveniences --

def new_workspace(L: Layout, device=None):
    """A zero-filled workspace tensor for grinqh_gemv on `device`."""
    import torch
    n = grinqh_gemv_workspace_bytes(L)
    if n == 0:
        raise GrinqhError(GRINQH_ENODEV, "grinqh_gemv_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def new_group_workspace(layouts, device=None):
    """A zero-filled workspace tensor for grinqh_gemv_group over `layouts`."""
    import torch
    n = grinqh_gemv_group_workspace_bytes(layouts)
    if n == 0:
        raise GrinqhError(GRINQH_EINVAL, "grinqh_gemv_group_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def pack(q, b_max: int, stream=None):
    """q uint8 [d_out][d_in] (cuda) -> (layout, planes int32 [d_in][P][W_row])."""
    import torch
    d_out, d_in = q.shape
    L = grinqh_layout_init(d_in, d_out, b_max)
    planes = torch.empty((d_in, L.n_planes, L.row_words), dtype=torch.int32, device=q.device)
    grinqh_pack(L, q, planes, stream)
    return L, planes


def assign_bits(L: Layout, x, theta, stream=None) -> Tuple:
    import torch
    bits = torch.empty(L.d_in, dtype=torch.uint8, device=x.device)
    idx = torch.empty(L.d_in, dtype=torch.int32, device=x.device)
    n = torch.empty(1, dtype=torch.int32, device=x.device)
    grinqh_assign_bits(L, x, theta, bits, idx, n, stream)
    return bits, idx, n


def gemv(L: Layout, x, theta, planes, s, z, workspace=None, out_dtype=None, stream=None):
    import torch
    if workspace is None:
        workspace = new_workspace(L, x.device)
    y = torch.empty(L.d_out, dtype=out_dtype or torch.float32, device=x.device)
    grinqh_gemv(L, x, theta, planes, s, z, y, workspace, stream)
    return y


def calibrate_thresholds(x, levels, workspace=None, stream=None):
    """fp32 thresholds [len(levels)] on x's device (allocates theta and, if not
    given, the workspace)."""
    import torch
    if workspace is None:
        workspace = torch.empty(grinqh_calibrate_workspace_bytes(), dtype=torch.uint8, device=x.device)
    theta = torch.empty(len(levels), dtype=torch.float32, device=x.device)
    grinqh_calibrate_thresholds(x, levels, theta, workspace, stream)
    return theta


def quantize_rtn(w, b_max: int, stream=None):
    """(q, s, z) of a bf16 weight matrix on its device (allocates them)."""
    import torch
    d_out, d_in = w.shape
    q = torch.empty((d_out, d_in), dtype=torch.uint8, device=w.device)
    s = torch.empty(d_out, dtype=torch.float16, device=w.device)
    z = torch.empty(d_out, dtype=torch.float16, device=w.device)
    grinqh_quantize_rtn(w, b_max, q, s, z, stream)
    return q, s, z


def prefill_gemm(L: Layout, x, planes, s, z, out_dtype=None, workspace=None, stream=None):
    """y [M][d_out] of a bf16 token block x [M][d_in] (allocates y and, if not
    given, the workspace)."""
    import torch
    M = x.shape[0]
    if workspace is None:
        workspace = torch.empty(max(grinqh_prefill_workspace_bytes(M), 256), dtype=torch.uint8, device=x.device)
    y = torch.empty((M, L.d_out), dtype=out_dtype or torch.float32, device=x.device)
    grinqh_prefill_gemm(L, x, planes, s, z, y, workspace, stream)
    return y


def debug_codes(L: Layout, bits, planes, stream=None):
    import torch
    codes = torch.empty((L.d_in, L.d_out), dtype=torch.uint8, device=bits.device)
    grinqh_debug_codes(L, bits, planes, codes, stream)
    return codes
