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

RBQ_STATUS_NONFINITE_W = 1
RBQ_STATUS_SCALE_OVERFLOW = 2
RBQ_STATUS_REFIT_KEPT = 4
RBQ_STATUS_PLANES_KEPT = 8
RBQ_EPILOGUE_NONE = 0
RBQ_EPILOGUE_SILU_MUL = 1
RBQ_ENCODE_FORCE_SERIAL = 1

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
