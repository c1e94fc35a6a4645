"""CPU oracle for the residual-binarized linear layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code
with the HIP library in ``gemm_rbq_encode_amd``, and the product path never
imports it.

The arithmetic lives in ``rbq_oracle.c`` (plain C, fp64, serial per row);
this file only builds it with gcc, loads it, and marshals numpy arrays.
Every function here cites the same passages as the C file: the RaBiT
summary (paperlayer.ai) sections 4.1, 4.2, A, B, G and D, and the QBB
summary (atlas.scime.ai) "Approach" (also for ``refit``).

Parity status: every function is pinned (see tests/test_oracle_pins.py):
``f64_to_f16`` against numpy's own float64->float16 conversion, ``encode``
against brute force over all sign patterns, closed forms, planted planes and
a hand-worked example, ``dequant``/``gemm`` against numpy unpacking and
matmul and against closed forms for x = 1 and x = e_j, ``refit`` against
numpy's least-squares solver, planted consistent systems, the cascade's own
scale for one plane, and optimality against the cascade's scales.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rbq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile rbq_oracle.c into liboracle.so with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Load liboracle.so, building it first only if it does not exist."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f64_to_f16_array.argtypes = [vp, i64, vp]
        L.oracle_f64_to_f16_array.restype = None
        L.oracle_encode.argtypes = [vp, i64, i64, i32, i64, vp, vp]
        L.oracle_encode.restype = i32
        L.oracle_dequant.argtypes = [vp, vp, i64, i64, i32, i64, vp]
        L.oracle_dequant.restype = i32
        L.oracle_gemm.argtypes = [vp, vp, i64, i64, i32, i64, vp, i64, vp]
        L.oracle_gemm.restype = i32
        L.oracle_refit.argtypes = [vp, i64, i64, i32, i64, vp, vp]
        L.oracle_refit.restype = i32
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def f64_to_f16(v: float) -> int:
    """fp64 -> binary16 bits, one rounding to nearest, ties to even."""
    return int(lib().oracle_f64_to_f16(float(v)))


def f64_to_f16_array(v: np.ndarray) -> np.ndarray:
    """Element-wise f64_to_f16 over a float64 array (uint16 result)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_f64_to_f16_array(_ptr(v), v.size, _ptr(out))
    return out


def f16_to_f64(h: int) -> float:
    return float(lib().oracle_f16_to_f64(int(h) & 0xFFFF))


def groups_per_row(in_features: int, group_size: int) -> int:
    return in_features // group_size if group_size else 1


def encode(W: np.ndarray, num_planes: int, group_size: int = 0):
    """Sequential residual binarization of fp32 W [out][in].

    Returns (planes uint32 [K][out][in/32], scales uint16 [K][out][G], flags)
    where flags bit 0 = non-finite W, bit 1 = a scale overflowed to inf.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    out, inf = W.shape
    G = groups_per_row(inf, group_size)
    planes = np.zeros((num_planes, out, inf // 32), dtype=np.uint32)
    scales = np.zeros((num_planes, out, G), dtype=np.uint16)
    flags = lib().oracle_encode(_ptr(W), out, inf, num_planes, group_size,
                                _ptr(planes), _ptr(scales))
    if flags < 0:
        raise ValueError("oracle_encode: bad arguments")
    return planes, scales, flags


def refit(W: np.ndarray, planes: np.ndarray, scales: np.ndarray, group_size: int = 0):
    """Joint least-squares refit of the K scales of every (row, group) for
    the fixed planes (QBB summary, "Approach").  ``scales`` are kept where
    no refit is made.  Returns (scales uint16 [K][out][G], flags) with
    flags bit 0 = non-finite W, bit 2 = some (row, group) kept its scales."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    out_scales = np.array(scales, dtype=np.uint16, copy=True, order="C")
    K, out, words = planes.shape
    inf = words * 32
    assert W.shape == (out, inf)
    flags = lib().oracle_refit(_ptr(W), out, inf, K, group_size, _ptr(planes), _ptr(out_scales))
    if flags < 0:
        raise ValueError("oracle_refit: bad arguments")
    return out_scales, flags


def silu_mul(Y: np.ndarray) -> np.ndarray:
    """Gated-MLP epilogue on layer outputs whose columns come in (gate, up)
    pairs 2i, 2i+1: H[m][i] = silu(Y[m][2i]) * Y[m][2i+1] with
    silu(v) = v / (1 + e^-v), in fp64 (the pages measure whole decoder
    layers: RaBiT section 5, QBB "Key results")."""
    Y = np.asarray(Y, dtype=np.float64)
    g, u = Y[:, 0::2], Y[:, 1::2]
    return g / (1.0 + np.exp(-g)) * u


def dequant(planes: np.ndarray, scales: np.ndarray, group_size: int = 0) -> np.ndarray:
    """Materialise What = sum_k a_k (.) B_k in fp64, [out][in]."""
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    K, out, words = planes.shape
    inf = words * 32
    What = np.empty((out, inf), dtype=np.float64)
    if lib().oracle_dequant(_ptr(planes), _ptr(scales), out, inf, K, group_size, _ptr(What)) != 0:
        raise ValueError("oracle_dequant: bad arguments")
    return What


def gemm(planes: np.ndarray, scales: np.ndarray, X: np.ndarray, group_size: int = 0) -> np.ndarray:
    """Y = X @ What^T in fp64.  X: fp16 bits (uint16) [M][in].  Y: [M][out]."""
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    X = np.ascontiguousarray(X)
    if X.dtype == np.float16:
        X = X.view(np.uint16)
    if X.ndim == 1:
        X = X[None, :]
    K, out, words = planes.shape
    inf = words * 32
    M = X.shape[0]
    assert X.shape[1] == inf
    Y = np.empty((M, out), dtype=np.float64)
    if lib().oracle_gemm(_ptr(planes), _ptr(scales), out, inf, K, group_size,
                         _ptr(X), M, _ptr(Y)) != 0:
        raise ValueError("oracle_gemm: bad arguments")
    return Y
