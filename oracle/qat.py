"""CPU oracle for the coupled (QAT-style) forward and its straight-through
backward (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library in ``gemm_rbq_encode_amd``, and the product path never
imports it.

What it computes (RaBiT summary, paperlayer.ai):
  * section 4.2 "Coupled Training": one shared full-precision weight; every
    forward pass derives B_1 from it, computes the first path's residual and
    derives B_2 from that residual; the scales are learnable and kept apart
    from the binary cores, which are recomputed;
  * "RaBiT training" (section G): each path is derived in turn from the
    shared weight, the effective weights are accumulated and the residual is
    updated after every path, then the layer output is formed;
  * the shared weight is updated with the full gradient (the optimisation
    trade-off paragraph).
Readings where the pages are silent:
  * with the scales given (learnable), the cascade is B_k = sign(R_{k-1})
    (R >= 0 gives +1, also -0.0), R_k = R_{k-1} - a_k B_k in fp32 against the
    given binary16 a_k, one rounding per step;
  * the layer output is Y = X What^T, What = sum_k a_k B_k;
  * the backward is the straight-through estimator: sign() passes the
    gradient unchanged, so dW = dWhat = dY^T X; the cores are held fixed for
    the scales, da_k[r][t] = sum_{j in group t} B_k[r][j] dW[r][j]; and
    dX = dY What.

Parity status: pinned in tests/test_qat_pins.py (sign(W) for one plane, the
nearest-value assignment of oracle.rebin for scales that dominate their
successors, planted planes, the C oracle's planes when its own scales are
given, finite differences of the linear surrogate for every gradient, and
closed forms for unit vectors).
"""
from __future__ import annotations

import numpy as np

from .dual import pack_signs, unpack_signs


def _scale_columns(scales_k: np.ndarray, inf: int, group_size: int) -> np.ndarray:
    """Scales of one plane [out][G] (binary16 bits) spread over the columns,
    float32 [out][in]."""
    a = np.asarray(scales_k, dtype=np.uint16).view(np.float16).astype(np.float32)
    if group_size:
        return np.repeat(a, group_size, axis=1)
    return np.repeat(a[:, :1], inf, axis=1)


def cascade(W: np.ndarray, scales: np.ndarray, group_size: int = 0) -> np.ndarray:
    """Binary cores of W for given scales: planes uint32 [K][out][in/32]."""
    R = np.array(W, dtype=np.float32, copy=True)
    K = scales.shape[0]
    out, inf = R.shape
    planes = np.zeros((K, out, inf // 32), dtype=np.uint32)
    for k in range(K):
        B = R >= np.float32(0.0)
        planes[k] = pack_signs(B)
        a = _scale_columns(scales[k], inf, group_size)
        R = np.where(B, R - a, R + a).astype(np.float32)
    return planes


def dequant(planes: np.ndarray, scales: np.ndarray, group_size: int = 0) -> np.ndarray:
    """What = sum_k a_k B_k in fp64, [out][in]."""
    K, out, words = planes.shape
    inf = words * 32
    What = np.zeros((out, inf), dtype=np.float64)
    for k in range(K):
        a = _scale_columns(scales[k], inf, group_size).astype(np.float64)
        What += a * unpack_signs(planes[k], inf)
    return What


def _f16(X) -> np.ndarray:
    X = np.asarray(X)
    if X.dtype == np.uint16:
        X = X.view(np.float16)
    return np.atleast_2d(X).astype(np.float64)


def forward(W: np.ndarray, scales: np.ndarray, X, group_size: int = 0):
    """Returns (planes, Y fp64 [M][out]) with Y = X What^T."""
    planes = cascade(W, scales, group_size)
    return planes, _f16(X) @ dequant(planes, scales, group_size).T


def backward(planes: np.ndarray, scales: np.ndarray, X, dY, group_size: int = 0):
    """Straight-through gradients in fp64: (dX [M][in], dW [out][in],
    dscales [K][out][G])."""
    Xf, dYf = _f16(X), _f16(dY)
    K, out, words = planes.shape
    inf = words * 32
    What = dequant(planes, scales, group_size)
    dX = dYf @ What
    dW = dYf.T @ Xf
    G = inf // group_size if group_size else 1
    n = group_size if group_size else inf
    dscales = np.zeros((K, out, G), dtype=np.float64)
    for k in range(K):
        S = unpack_signs(planes[k], inf) * dW
        dscales[k] = S.reshape(out, G, n).sum(axis=2)
    return dX, dW, dscales
