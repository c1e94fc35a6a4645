"""ctypes binding of librbq (include/rbq.h), with torch tensors as buffers.

Argument marshalling only: every computation runs in the HIP kernels of
librbq.so.  torch provides device memory and the current stream.  If
librbq.so has not been built, every entry point raises RbqLibraryMissing --
there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librbq.so")

RBQ_OK = 0
RBQ_ERR_INVALID_ARG = 1
RBQ_ERR_ALIGNMENT = 2
RBQ_ERR_UNSUPPORTED = 3
RBQ_ERR_NO_DEVICE = 4
RBQ_ERR_HIP = 5
RBQ_ERR_SCRATCH_LIMIT = 6
RBQ_NOALLOC_SCRATCH_BYTES = 8 << 20

RBQ_STATUS_NONFINITE_W = 1
RBQ_STATUS_SCALE_OVERFLOW = 2
RBQ_STATUS_REFIT_KEPT = 4
RBQ_STATUS_PLANES_KEPT = 8
RBQ_STATUS_PROGRAM_TIMEOUT = 16
RBQ_STATUS_PROGRAM_MISMATCH = 32
RBQ_PROGRAM_MAX_OPS = 512
RBQ_EPILOGUE_NONE = 0
RBQ_EPILOGUE_SILU_MUL = 1
RBQ_ENCODE_FORCE_SERIAL = 1
RBQ_LAYOUT_ROWS = 0
RBQ_LAYOUT_TILES = 1

PATH_AUTO, PATH_VALU, PATH_DECODE, PATH_PREFILL, PATH_STREAM, PATH_FLAT, PATH_GROUP, PATH_SPLIT = (
    0, 1, 2, 3, 4, 5, 6, 7)


class RbqLibraryMissing(RuntimeError):
    pass


class RbqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}"
                         + (f" (hipError {last_hip_error()})" if status == RBQ_ERR_HIP else ""))


class Shape(ctypes.Structure):
    _fields_ = [("out_features", ctypes.c_int32), ("in_features", ctypes.c_int32),
                ("num_planes", ctypes.c_int32), ("group_size", ctypes.c_int32)]

    def __repr__(self):
        return (f"Shape(out={self.out_features}, in={self.in_features}, "
                f"K={self.num_planes}, group={self.group_size})")


class ProgramOp(ctypes.Structure):
    """rbq_program_op."""
    _fields_ = [("planes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("out_features", ctypes.c_int32), ("in_features", ctypes.c_int32),
                ("epilogue", ctypes.c_uint32), ("wait_for", ctypes.c_int32), ("planes_layout", ctypes.c_uint32),
                ("group_size", ctypes.c_int32), ("tokens", ctypes.c_int32)]


_lib = None

# name -> (restype, argtypes)
_SIGNATURES = {
    "rbq_check_shape": (ctypes.c_int, [Shape]),
    "rbq_planes_bytes": (ctypes.c_size_t, [Shape]),
    "rbq_scales_bytes": (ctypes.c_size_t, [Shape]),
    "rbq_encode": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_encode_ex": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "rbq_refit": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_rebinarize": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, Shape, ctypes.c_void_p,
                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_size_t, ctypes.c_void_p]),
    "rbq_gemm_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, Shape, ctypes.c_void_p,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]),
    "rbq_gemm_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, Shape, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_gemm_workspace_bytes": (ctypes.c_size_t, [Shape, ctypes.c_int32]),
    "rbq_gemv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, Shape, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_dual_g_bytes": (ctypes.c_size_t, [Shape]),
    "rbq_dual_h_bytes": (ctypes.c_size_t, [Shape]),
    "rbq_encode_dual_workspace_bytes": (ctypes.c_size_t, [Shape]),
    "rbq_encode_dual": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_gemv_dual": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, Shape,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_gemm_dual": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, Shape, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_program_bytes": (ctypes.c_size_t, [ctypes.c_int32]),
    "rbq_program_counters_bytes": (ctypes.c_size_t, [ctypes.c_int32]),
    "rbq_program_build": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t]),
    "rbq_program_run": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]),
    "rbq_qat_encode": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]),
    "rbq_qat_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_qat_backward_workspace_bytes": (ctypes.c_size_t, [Shape, ctypes.c_int32]),
    "rbq_qat_backward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_probe_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_tiles_bytes": (ctypes.c_size_t, [Shape]),
    "rbq_pack_tiles": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_scale_tiles_bytes": (ctypes.c_size_t, [Shape]),
    "rbq_pack_scale_tiles": (ctypes.c_int, [ctypes.c_void_p, Shape, ctypes.c_void_p, ctypes.c_void_p]),
    "rbq_set_path": (ctypes.c_int, [ctypes.c_int]),
    "rbq_select_path": (ctypes.c_int, [Shape, ctypes.c_int32]),
    "rbq_set_stream_split": (ctypes.c_int32, [ctypes.c_int32]),
    "rbq_last_hip_error": (ctypes.c_int32, []),
    "rbq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rbq_version": (ctypes.c_char_p, []),
}


def lib():
    """The loaded librbq.so (raises RbqLibraryMissing if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RbqLibraryMissing(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                f"g.build()'` (hipcc, gfx950). There is no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().rbq_status_string(int(st)).decode()


def last_hip_error() -> int:
    return int(lib().rbq_last_hip_error())


def version() -> str:
    return lib().rbq_version().decode()


def shape(out_features: int, in_features: int, num_planes: int, group_size: int = 0) -> Shape:
    return Shape(int(out_features), int(in_features), int(num_planes), int(group_size))


def groups_per_row(in_features: int, group_size: int) -> int:
    if in_features == 0:
        return 0
    return in_features // group_size if group_size else 1


def planes_bytes(s: Shape) -> int:
    return int(lib().rbq_planes_bytes(s))


def scales_bytes(s: Shape) -> int:
    return int(lib().rbq_scales_bytes(s))


def check(st: int, what: str) -> None:
    if st != RBQ_OK:
        raise RbqError(st, what)


def set_path(path: int) -> int:
    """Force a kernel family for rbq_gemm (PATH_*); returns the old setting."""
    return int(lib().rbq_set_path(int(path)))


def set_stream_split(waves_per_tile: int) -> int:
    """Waves per 16-row tile in the streaming kernel (0 = automatic)."""
    old = int(lib().rbq_set_stream_split(int(waves_per_tile)))
    if old < 0:
        raise ValueError("waves_per_tile must be 0, 1, 2 or 4")
    return old


def select_path(s: Shape, M: int) -> int:
    return int(lib().rbq_select_path(s, int(M)))


def _stream(t: torch.Tensor, stream=None) -> int:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return int(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def encode(W: torch.Tensor, num_planes: int, group_size: int = 0, *,
           status: torch.Tensor | None = None, force_serial: bool = False,
           planes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
           stream=None):
    """rbq_encode: fp32 W [out][in] -> (planes int32 [K][out][in/32],
    scales float16 [K][out][G]).  `status` (int32, 1 element) receives
    RBQ_STATUS_* bits if given."""
    _dev(W, torch.float32, "W")
    out_f, in_f = W.shape
    s = shape(out_f, in_f, num_planes, group_size)
    G = groups_per_row(in_f, group_size)
    if planes is None:
        planes = torch.empty((num_planes, out_f, in_f // 32), dtype=torch.int32, device=W.device)
    if scales is None:
        scales = torch.empty((num_planes, out_f, G), dtype=torch.float16, device=W.device)
    _dev(planes, torch.int32, "planes")
    _dev(scales, torch.float16, "scales")
    if planes.numel() * 4 < planes_bytes(s) or scales.numel() * 2 < scales_bytes(s):
        raise ValueError("planes/scales buffers are too small for the shape")
    sp = None
    if status is not None:
        _dev(status, torch.int32, "status")
        sp = status.data_ptr()
    flags = RBQ_ENCODE_FORCE_SERIAL if force_serial else 0
    check(lib().rbq_encode_ex(W.data_ptr(), s, planes.data_ptr(), scales.data_ptr(), sp,
                              flags, _stream(W, stream)), "rbq_encode")
    return planes, scales


def refit(W: torch.Tensor, planes: torch.Tensor, scales: torch.Tensor, group_size: int = 0, *,
          status: torch.Tensor | None = None, stream=None):
    """rbq_refit: joint least-squares refit of the K scales of every (row,
    group) of W for the fixed planes, in place on `scales` (which also hold
    the scales kept where no refit is made).  Returns `scales`."""
    _dev(W, torch.float32, "W")
    _dev(planes, torch.int32, "planes")
    _dev(scales, torch.float16, "scales")
    out_f, in_f = W.shape
    K = planes.shape[0]
    s = shape(out_f, in_f, K, group_size)
    if planes.numel() * 4 < planes_bytes(s) or scales.numel() * 2 < scales_bytes(s):
        raise ValueError("planes/scales buffers are too small for the shape")
    sp = None
    if status is not None:
        _dev(status, torch.int32, "status")
        sp = status.data_ptr()
    check(lib().rbq_refit(W.data_ptr(), s, planes.data_ptr(), scales.data_ptr(), sp, _stream(W, stream)),
          "rbq_refit")
    return scales


def rebinarize(W: torch.Tensor, planes: torch.Tensor, scales: torch.Tensor, group_size: int = 0, *,
               status: torch.Tensor | None = None, stream=None):
    """rbq_rebinarize: the planes of W for the fixed scales (each weight
    takes the nearest of the 2^K values sum_k +-a_k), in place on `planes`
    (which keep their words where a group's scales are not finite).
    Returns `planes`."""
    _dev(W, torch.float32, "W")
    _dev(planes, torch.int32, "planes")
    _dev(scales, torch.float16, "scales")
    out_f, in_f = W.shape
    K = planes.shape[0]
    s = shape(out_f, in_f, K, group_size)
    if planes.numel() * 4 < planes_bytes(s) or scales.numel() * 2 < scales_bytes(s):
        raise ValueError("planes/scales buffers are too small for the shape")
    sp = None
    if status is not None:
        _dev(status, torch.int32, "status")
        sp = status.data_ptr()
    check(lib().rbq_rebinarize(W.data_ptr(), s, planes.data_ptr(), scales.data_ptr(), sp,
                               _stream(W, stream)), "rbq_rebinarize")
    return planes


def gemm(planes: torch.Tensor, scales: torch.Tensor, X: torch.Tensor, group_size: int = 0, *,
         Y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         epilogue: int = 0, stream=None):
    """rbq_gemm_ex: Y[M][out] = sum_k a_k (.) (B_k X[m]), fp16 in and out;
    with epilogue=RBQ_EPILOGUE_SILU_MUL the rows are (gate, up) pairs and
    Y[M][out/2] holds silu(gate) * up."""
    _dev(planes, torch.int32, "planes")
    _dev(scales, torch.float16, "scales")
    _dev(X, torch.float16, "X")
    K, out_f, words = planes.shape
    in_f = words * 32
    if X.dim() != 2 or X.shape[1] != in_f:
        raise ValueError(f"X must be [M][{in_f}], got {tuple(X.shape)}")
    M = X.shape[0]
    s = shape(out_f, in_f, K, group_size)
    if scales.numel() * 2 < scales_bytes(s):
        raise ValueError("scales buffer too small for the shape")
    ycols = out_f // 2 if epilogue == RBQ_EPILOGUE_SILU_MUL else out_f
    if Y is None:
        Y = torch.empty((M, ycols), dtype=torch.float16, device=X.device)
    _dev(Y, torch.float16, "Y")
    if Y.numel() < M * ycols:
        raise ValueError("Y too small")
    ws_need = int(lib().rbq_gemm_workspace_bytes(s, M))
    ws_ptr, ws_bytes = None, 0
    if ws_need:
        if workspace is None:
            workspace = torch.empty(ws_need, dtype=torch.uint8, device=X.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().rbq_gemm_ex(planes.data_ptr(), scales.data_ptr(), s, X.data_ptr(), M,
                            Y.data_ptr(), ws_ptr, ws_bytes, int(epilogue), _stream(X, stream)), "rbq_gemm")
    return Y


def gemm_noalloc(planes: torch.Tensor, scales: torch.Tensor, X: torch.Tensor, Y: torch.Tensor,
                 group_size: int = 0, *, stream=None):
    """rbq_gemm_noalloc: rbq_gemm into a caller-given Y [M][out], with the
    split kernels' scratch taken from the library's static device buffer
    (nothing is allocated; calls that overlap on one GPU race)."""
    _dev(planes, torch.int32, "planes")
    _dev(scales, torch.float16, "scales")
    _dev(X, torch.float16, "X")
    _dev(Y, torch.float16, "Y")
    K, out_f, words = planes.shape
    in_f = words * 32
    if X.dim() != 2 or X.shape[1] != in_f:
        raise ValueError(f"X must be [M][{in_f}], got {tuple(X.shape)}")
    M = X.shape[0]
    s = shape(out_f, in_f, K, group_size)
    if scales.numel() * 2 < scales_bytes(s):
        raise ValueError("scales buffer too small for the shape")
    if Y.numel() < M * out_f:
        raise ValueError("Y too small")
    check(lib().rbq_gemm_noalloc(planes.data_ptr(), scales.data_ptr(), s, X.data_ptr(), M, Y.data_ptr(),
                                 _stream(X, stream)), "rbq_gemm_noalloc")
    return Y


def gemv(planes: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, group_size: int = 0, *,
         y: torch.Tensor | None = None, stream=None):
    """rbq_gemv: y[out] = sum_k a_k (.) (B_k x) for one fp16 token x [in]."""
    _dev(planes, torch.int32, "planes")
    _dev(scales, torch.float16, "scales")
    _dev(x, torch.float16, "x")
    K, out_f, words = planes.shape
    in_f = words * 32
    if x.numel() != in_f:
        raise ValueError(f"x must have {in_f} elements")
    s = shape(out_f, in_f, K, group_size)
    if y is None:
        y = torch.empty(out_f, dtype=torch.float16, device=x.device)
    _dev(y, torch.float16, "y")
    check(lib().rbq_gemv(planes.data_ptr(), scales.data_ptr(), s, x.data_ptr(), y.data_ptr(),
                         _stream(x, stream)), "rbq_gemv")
    return y


def qat_encode(W: torch.Tensor, scales: torch.Tensor, group_size: int = 0, *,
               planes: torch.Tensor | None = None, status: torch.Tensor | None = None, stream=None):
    """rbq_qat_encode: binary cores of fp32 W [out][in] for the given fp16
    scales [K][out][G]; returns planes int32 [K][out][in/32]."""
    _dev(W, torch.float32, "W")
    _dev(scales, torch.float16, "scales")
    out_f, in_f = W.shape
    K = scales.shape[0]
    s = shape(out_f, in_f, K, group_size)
    if scales.numel() * 2 != int(lib().rbq_scales_bytes(s)):
        raise ValueError("scales do not match the shape")
    if planes is None:
        planes = torch.empty((K, out_f, in_f // 32), dtype=torch.int32, device=W.device)
    _dev(planes, torch.int32, "planes")
    sp = None
    if status is not None:
        _dev(status, torch.int32, "status")
        sp = status.data_ptr()
    check(lib().rbq_qat_encode(W.data_ptr(), s, scales.data_ptr(), planes.data_ptr(), sp, _stream(W, stream)),
          "rbq_qat_encode")
    return planes


def qat_forward(W: torch.Tensor, scales: torch.Tensor, X: torch.Tensor, group_size: int = 0, *,
                planes: torch.Tensor | None = None, Y: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, status: torch.Tensor | None = None, stream=None):
    """rbq_qat_forward: (planes, Y) with planes derived from W for the given
    scales and Y [M][out] = X What^T (fp16)."""
    _dev(W, torch.float32, "W")
    _dev(scales, torch.float16, "scales")
    _dev(X, torch.float16, "X")
    out_f, in_f = W.shape
    K = scales.shape[0]
    s = shape(out_f, in_f, K, group_size)
    if X.dim() != 2 or X.shape[1] != in_f:
        raise ValueError(f"X must be [M][{in_f}]")
    if scales.numel() * 2 != int(lib().rbq_scales_bytes(s)):
        raise ValueError("scales do not match the shape")
    M = X.shape[0]
    if planes is None:
        planes = torch.empty((K, out_f, in_f // 32), dtype=torch.int32, device=W.device)
    if Y is None:
        Y = torch.empty((M, out_f), dtype=torch.float16, device=W.device)
    _dev(planes, torch.int32, "planes")
    _dev(Y, torch.float16, "Y")
    need = int(lib().rbq_gemm_workspace_bytes(s, M))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=W.device)
    wp, wn = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    sp = None
    if status is not None:
        _dev(status, torch.int32, "status")
        sp = status.data_ptr()
    check(lib().rbq_qat_forward(W.data_ptr(), scales.data_ptr(), s, X.data_ptr(), M, planes.data_ptr(),
                                Y.data_ptr(), wp, wn, sp, _stream(W, stream)), "rbq_qat_forward")
    return planes, Y


def qat_backward(planes: torch.Tensor, scales: torch.Tensor, X: torch.Tensor, dY: torch.Tensor,
                 group_size: int = 0, *, need_dx: bool = True, need_dw: bool = True, need_dscales: bool = True,
                 workspace: torch.Tensor | None = None, status: torch.Tensor | None = None, stream=None):
    """rbq_qat_backward: straight-through (dX [M][in], dW [out][in],
    dscales [K][out][G]), fp32; an output not asked for is None."""
    _dev(planes, torch.int32, "planes")
    _dev(scales, torch.float16, "scales")
    _dev(X, torch.float16, "X")
    _dev(dY, torch.float16, "dY")
    K, out_f, words = planes.shape
    in_f = words * 32
    s = shape(out_f, in_f, K, group_size)
    M = X.shape[0]
    if X.shape != (M, in_f) or dY.shape != (M, out_f):
        raise ValueError("X must be [M][in] and dY [M][out]")
    dev = planes.device
    G = in_f // group_size if group_size else 1
    dX = torch.empty((M, in_f), dtype=torch.float32, device=dev) if need_dx else None
    dW = torch.empty((out_f, in_f), dtype=torch.float32, device=dev) if (need_dw or need_dscales) else None
    ds = torch.empty((K, out_f, G), dtype=torch.float32, device=dev) if need_dscales else None
    sp = None
    if status is not None:
        _dev(status, torch.int32, "status")
        sp = status.data_ptr()
    ptr = (lambda t: None if t is None else t.data_ptr())
    need = int(lib().rbq_qat_backward_workspace_bytes(s, M))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wn = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib().rbq_qat_backward(planes.data_ptr(), scales.data_ptr(), s, X.data_ptr(), dY.data_ptr(), M,
                                 ptr(dX), ptr(dW), ptr(ds), ptr(workspace), wn, sp, _stream(planes, stream)),
          "rbq_qat_backward")
    return dX, (dW if need_dw else None), ds


def probe_read(buf: torch.Tensor, sink: torch.Tensor, nbytes: int | None = None, *, stream=None) -> None:
    """rbq_probe_read: one launch reading the first `nbytes` bytes of the
    device tensor `buf` (all of it by default); sink is a device int32."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous device tensor")
    _dev(sink, torch.int32, "sink")
    total = buf.numel() * buf.element_size()
    n = total if nbytes is None else int(nbytes)
    if n < 0 or n > total:
        raise ValueError(f"nbytes must be in [0, {total}]")
    check(lib().rbq_probe_read(buf.data_ptr(), n, sink.data_ptr(), _stream(buf, stream)), "rbq_probe_read")


def tiles_bytes(s: Shape) -> int:
    """rbq_tiles_bytes: bytes of the tile layout of shape s."""
    return int(lib().rbq_tiles_bytes(s))


def pack_tiles(planes: torch.Tensor, *, tiles: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """rbq_pack_tiles: the RBQ_LAYOUT_TILES copy of row-layout planes
    (int32 [K][out][in/32]) as an int32 tensor [K][ceil(out/16)][ceil(in/512)][256]."""
    _dev(planes, torch.int32, "planes")
    K, out_f, words = planes.shape
    s = shape(out_f, words * 32, K)
    dims = (K, (out_f + 15) // 16, (words * 32 + 511) // 512, 256)
    if tiles is None:
        tiles = torch.empty(dims, dtype=torch.int32, device=planes.device)
    else:
        _dev(tiles, torch.int32, "tiles")
        if tuple(tiles.shape) != dims:
            raise ValueError(f"tiles must have shape {dims}")
    check(lib().rbq_pack_tiles(planes.data_ptr(), s, tiles.data_ptr(), _stream(planes, stream)), "rbq_pack_tiles")
    return tiles


def scale_tiles_bytes(s: Shape) -> int:
    """rbq_scale_tiles_bytes: bytes of the scale tiles of a g128 shape (0 if none)."""
    return int(lib().rbq_scale_tiles_bytes(s))


def pack_scale_tiles(scales: torch.Tensor, in_features: int, *, tiles: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """rbq_pack_scale_tiles: the scale tiles of g128 scales (fp16 [K][out][in/128])
    as an fp16 tensor [ceil(out/16)][ceil(in/512)][K*64]."""
    _dev(scales, torch.float16, "scales")
    if scales.dim() != 3 or scales.shape[2] * 128 != in_features:
        raise ValueError("scales must be [K][out][in/128]")
    K, out_f, _ = scales.shape
    s = shape(out_f, in_features, K, 128)
    dims = ((out_f + 15) // 16, (in_features + 511) // 512, K * 64)
    if tiles is None:
        tiles = torch.empty(dims, dtype=torch.float16, device=scales.device)
    else:
        _dev(tiles, torch.float16, "tiles")
        if tuple(tiles.shape) != dims:
            raise ValueError(f"tiles must have shape {dims}")
    check(lib().rbq_pack_scale_tiles(scales.data_ptr(), s, tiles.data_ptr(), _stream(scales, stream)),
          "rbq_pack_scale_tiles")
    return tiles


def encode_dual_workspace_bytes(s: Shape) -> int:
    return int(lib().rbq_encode_dual_workspace_bytes(s))


def encode_dual(W: torch.Tensor, num_planes: int, *, workspace: torch.Tensor | None = None,
                status: torch.Tensor | None = None, planes: torch.Tensor | None = None,
                g: torch.Tensor | None = None, h: torch.Tensor | None = None, stream=None):
    """rbq_encode_dual: fp32 W [out][in] -> (planes int32 [K][out][in/32],
    g float16 [K][out], h float16 [K][in]), scales from a residual SVID."""
    _dev(W, torch.float32, "W")
    out_f, in_f = W.shape
    s = shape(out_f, in_f, num_planes, 0)
    if planes is None:
        planes = torch.empty((num_planes, out_f, in_f // 32), dtype=torch.int32, device=W.device)
    if g is None:
        g = torch.empty((num_planes, out_f), dtype=torch.float16, device=W.device)
    if h is None:
        h = torch.empty((num_planes, in_f), dtype=torch.float16, device=W.device)
    _dev(planes, torch.int32, "planes")
    _dev(g, torch.float16, "g")
    _dev(h, torch.float16, "h")
    if (planes.numel() * 4 < planes_bytes(s) or g.numel() * 2 < int(lib().rbq_dual_g_bytes(s))
            or h.numel() * 2 < int(lib().rbq_dual_h_bytes(s))):
        raise ValueError("planes/g/h buffers are too small for the shape")
    need = encode_dual_workspace_bytes(s)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=W.device)
    sp = None
    if status is not None:
        _dev(status, torch.int32, "status")
        sp = status.data_ptr()
    check(lib().rbq_encode_dual(W.data_ptr(), s, planes.data_ptr(), g.data_ptr(), h.data_ptr(),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(), sp,
                                _stream(W, stream)), "rbq_encode_dual")
    return planes, g, h


def gemv_dual(planes: torch.Tensor, g: torch.Tensor, h: torch.Tensor, x: torch.Tensor, *,
              y: torch.Tensor | None = None, stream=None):
    """rbq_gemv_dual: y[out] = sum_k g_k (.) (B_k (h_k (.) x)), fp16 in and out."""
    _dev(planes, torch.int32, "planes")
    _dev(g, torch.float16, "g")
    _dev(h, torch.float16, "h")
    _dev(x, torch.float16, "x")
    K, out_f, words = planes.shape
    in_f = words * 32
    if x.numel() != in_f:
        raise ValueError(f"x must have {in_f} elements")
    s = shape(out_f, in_f, K, 0)
    if g.numel() * 2 < int(lib().rbq_dual_g_bytes(s)) or h.numel() * 2 < int(lib().rbq_dual_h_bytes(s)):
        raise ValueError("g/h buffers are too small for the shape")
    if y is None:
        y = torch.empty(out_f, dtype=torch.float16, device=x.device)
    _dev(y, torch.float16, "y")
    check(lib().rbq_gemv_dual(planes.data_ptr(), g.data_ptr(), h.data_ptr(), s, x.data_ptr(),
                              y.data_ptr(), _stream(x, stream)), "rbq_gemv_dual")
    return y


def gemm_dual(planes: torch.Tensor, g: torch.Tensor, h: torch.Tensor, X: torch.Tensor, *,
              Y: torch.Tensor | None = None, stream=None):
    """rbq_gemm_dual: Y[M][out] = X Ŵᵀ with Ŵ = sum_k diag(g_k) B_k diag(h_k), fp16 in and out."""
    _dev(planes, torch.int32, "planes")
    _dev(g, torch.float16, "g")
    _dev(h, torch.float16, "h")
    _dev(X, torch.float16, "X")
    K, out_f, words = planes.shape
    in_f = words * 32
    if X.dim() != 2 or X.shape[1] != in_f:
        raise ValueError(f"X must be [M][{in_f}]")
    M = X.shape[0]
    s = shape(out_f, in_f, K, 0)
    if g.numel() * 2 < int(lib().rbq_dual_g_bytes(s)) or h.numel() * 2 < int(lib().rbq_dual_h_bytes(s)):
        raise ValueError("g/h buffers are too small for the shape")
    if Y is None:
        Y = torch.empty((M, out_f), dtype=torch.float16, device=X.device)
    _dev(Y, torch.float16, "Y")
    if Y.numel() < M * out_f:
        raise ValueError("Y too small")
    check(lib().rbq_gemm_dual(planes.data_ptr(), g.data_ptr(), h.data_ptr(), s, X.data_ptr(), M, Y.data_ptr(),
                              _stream(X, stream)), "rbq_gemm_dual")
    return Y


class Program:
    """A list of one-token GEMVs run by one persistent launch (rbq_program_*).

    ops: sequence of dicts with keys planes (int32 [K][out][in/32], or the
    tile layout [K][ceil(out/16)][ceil(in/512)][256] that pack_tiles
    writes), scales (fp16 [K][out]), x (fp16 [in]), y (fp16 [out], or [out/2]
    with epilogue=RBQ_EPILOGUE_SILU_MUL), and optionally epilogue,
    wait_for (index of an earlier op whose y this op reads; -1 = none) and
    tokens (2: x is [2][in] and y [2][out], each token quantised on its own;
    every op of the program then has two tokens).
    g128 ops (group_size=128, every op of the program) take tiled planes,
    the scale tiles of pack_scale_tiles as scales, and out_features.  The tensors
    are kept referenced; the image is built on the host, copied to the
    device once, and run() enqueues the launch on the current stream."""

    def __init__(self, ops, num_planes: int = 2):
        if not ops:
            raise ValueError("a program needs at least one op")
        self._keep = []
        arr = (ProgramOp * len(ops))()
        dev = None
        for i, o in enumerate(ops):
            p, s, x, y = o["planes"], o["scales"], o["x"], o["y"]
            tok = int(o.get("tokens", 1))
            nt = max(tok, 1)
            _dev(p, torch.int32, "planes")
            _dev(s, torch.float16, "scales")
            _dev(x, torch.float16, "x")
            _dev(y, torch.float16, "y")
            gs = int(o.get("group_size", 0))
            if gs:
                if p.dim() != 4 or "out_features" not in o:
                    raise ValueError(f"op {i}: g128 ops take tiled planes and out_features")
                layout = RBQ_LAYOUT_TILES
                K, out_f, words = p.shape[0], int(o["out_features"]), x.numel() // (32 * nt)
                if tuple(p.shape) != (K, (out_f + 15) // 16, (words * 32 + 511) // 512, 256) or \
                        tuple(s.shape) != (p.shape[1], p.shape[2], K * 64):
                    raise ValueError(f"op {i}: tiled planes or scale tiles do not match out_features and x")
            elif p.dim() == 4:   # tile layout: the shape comes from scales and x
                layout = RBQ_LAYOUT_TILES
                K = p.shape[0]
                if s.dim() not in (2, 3) or s.shape[0] != K or s.numel() != K * s.shape[1]:
                    raise ValueError(f"op {i}: scales must be [K][out] (or [K][out][1]) with tiled planes")
                out_f, words = s.shape[1], x.numel() // (32 * nt)
                if tuple(p.shape) != (K, (out_f + 15) // 16, (words * 32 + 511) // 512, 256):
                    raise ValueError(f"op {i}: tiled planes do not match scales and x")
            else:
                layout = RBQ_LAYOUT_ROWS
                K, out_f, words = p.shape
            if K != num_planes:
                raise ValueError(f"op {i}: {K} planes, the program has {num_planes}")
            ep = int(o.get("epilogue", RBQ_EPILOGUE_NONE))
            if x.numel() != nt * words * 32 or (not gs and s.numel() < K * out_f):
                raise ValueError(f"op {i}: x or scales do not match the planes")
            if y.numel() < nt * (out_f // 2 if ep == RBQ_EPILOGUE_SILU_MUL else out_f):
                raise ValueError(f"op {i}: y too small")
            arr[i] = ProgramOp(p.data_ptr(), s.data_ptr(), x.data_ptr(), y.data_ptr(), out_f, words * 32, ep,
                               int(o.get("wait_for", -1)), layout, gs, tok)
            self._keep += [p, s, x, y]
            dev = x.device
        n = len(ops)
        nbytes = int(lib().rbq_program_bytes(n))
        if nbytes == 0:
            raise RbqError(RBQ_ERR_UNSUPPORTED, "rbq_program_bytes")
        host = (ctypes.c_ubyte * nbytes)()
        check(lib().rbq_program_build(ctypes.cast(arr, ctypes.c_void_p), n, int(num_planes),
                                      ctypes.cast(host, ctypes.c_void_p), nbytes), "rbq_program_build")
        self._host = host
        self.n_ops = n
        self.image_dev = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8).to(dev)
        self.counters = torch.zeros(int(lib().rbq_program_counters_bytes(n)) // 4, dtype=torch.int32, device=dev)

    def run(self, status: torch.Tensor | None = None, stream=None) -> None:
        sp = None
        if status is not None:
            _dev(status, torch.int32, "status")
            sp = status.data_ptr()
        check(lib().rbq_program_run(ctypes.cast(self._host, ctypes.c_void_p), self.image_dev.data_ptr(),
                                    self.counters.data_ptr(), sp, _stream(self.image_dev, stream)),
              "rbq_program_run")
