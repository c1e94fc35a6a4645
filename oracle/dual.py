"""CPU oracle for the dual-scale residual-binarized layer (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library in ``gemm_rbq_encode_amd``, and the product path never
imports it.

What it computes (RaBiT summary, paperlayer.ai):
  * section 4.1: a binary path is a binary core with per-channel scaling
    vectors on both sides, so path k contributes diag(g_k) B_k diag(h_k) and
        y = sum_k g_k (.) (B_k (h_k (.) x));
  * section 4.3 and "RaBiT initialization": the paths' scales come from an
    iterative residual SVID -- B_k = sign(R_{k-1}) and |R_{k-1}| approximated
    by a rank-1 product g_k h_k^T -- with Tmax = 20 SVID iterations
    ("Training configuration").  The calibration-statistics preconditioning
    of that initialization needs data and is left out (the data-free
    reading).
Readings where the pages are silent:
  * the rank-1 product is fitted by alternating least squares starting from
    h = 1: u = |R| v / (v.v), then v = |R|^T u / (u.u), repeated 20 times
    (a power iteration on |R|^T |R|); an all-zero |R| gives zero scales;
  * the pair is balanced so that ||g|| = ||h|| (g = u / c, h = v c with
    c = sqrt(||u|| / ||v||)) and each entry is rounded once to binary16;
  * sign(0) = +1 (also for -0.0), and the residual is updated in fp32 with
    one rounding against the stored scales: R - (bit ? 1 : -1) g_r h_j,
    where the product of two binary16 values is exact in fp32.

Parity status: pinned in tests/test_oracle_pins.py (exact rank-1 magnitudes,
numpy's SVD, row-constant magnitudes, the alternating-least-squares descent
against per-row scales, residual norms, the C oracle's first plane, and a
pure-Python loop for the layer output).
"""
from __future__ import annotations

import numpy as np

from . import f64_to_f16_array

SVID_ITERS = 20


def pack_signs(B: np.ndarray) -> np.ndarray:
    """bool [out][in] -> uint32 words [out][in/32]: bit b of word w is
    column 32w + b, bit 1 = +1."""
    B = np.ascontiguousarray(B, dtype=bool)
    out, inf = B.shape
    by = np.packbits(B.reshape(out, inf // 8, 8), axis=2, bitorder="little").reshape(out, inf // 8)
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32)


def unpack_signs(words: np.ndarray, inf: int) -> np.ndarray:
    """uint32 words [out][in/32] -> float64 [out][in] of +1 / -1."""
    words = np.ascontiguousarray(words, dtype="<u4")
    bits = np.unpackbits(words.view(np.uint8), axis=1, bitorder="little")[:, :inf]
    return np.where(bits.astype(bool), 1.0, -1.0)


def f16(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def svid_rank1(A: np.ndarray, iters: int = SVID_ITERS):
    """Rank-1 fit u v^T of a non-negative fp64 matrix A by `iters`
    alternating least-squares steps from v = 1.  Returns (u, v), zeros when
    A has no non-zero entry."""
    A = np.asarray(A, dtype=np.float64)
    out, inf = A.shape
    v = np.ones(inf)
    vv = float(inf)
    u = np.zeros(out)
    for _ in range(iters):
        u = (A @ v) / vv
        uu = float(u @ u)
        if uu == 0.0:
            return np.zeros(out), np.zeros(inf)
        v = (A.T @ u) / uu
        vv = float(v @ v)
        if vv == 0.0:
            return np.zeros(out), np.zeros(inf)
    return u, v


def svid_balanced(A: np.ndarray, iters: int = SVID_ITERS):
    """The rank-1 fit balanced so that ||g|| = ||h||, before rounding:
    (u / c, v c) in fp64 with c = sqrt(||u|| / ||v||); zeros for a zero fit."""
    u, v = svid_rank1(A, iters)
    nu, nv = np.sqrt(u @ u), np.sqrt(v @ v)
    if nu == 0.0 or nv == 0.0:
        return np.zeros(A.shape[0]), np.zeros(A.shape[1])
    c = np.sqrt(nu / nv)
    return u / c, v * c


def svid_scales(A: np.ndarray, iters: int = SVID_ITERS):
    """Balanced fp16 scales (g bits [out], h bits [in]) of the rank-1 fit."""
    gb, hb = svid_balanced(A, iters)
    return f64_to_f16_array(gb), f64_to_f16_array(hb)


def encode_dual(W: np.ndarray, num_planes: int, iters: int = SVID_ITERS, fits: list | None = None):
    """Residual SVID binarization of fp32 W [out][in] (finite values).

    Returns (planes uint32 [K][out][in/32], g uint16 [K][out], h uint16 [K][in]).
    If `fits` is a list, the unrounded balanced pair (fp64 g, fp64 h) of each
    plane is appended to it (tests use it to see how close a scale lies to a
    binary16 rounding boundary)."""
    R = np.array(W, dtype=np.float32, copy=True)
    out, inf = R.shape
    planes = np.zeros((num_planes, out, inf // 32), dtype=np.uint32)
    g = np.zeros((num_planes, out), dtype=np.uint16)
    h = np.zeros((num_planes, inf), dtype=np.uint16)
    for k in range(num_planes):
        B = R >= np.float32(0.0)
        gb, hb = svid_balanced(np.abs(R).astype(np.float64), iters)
        if fits is not None:
            fits.append((gb, hb))
        g[k], h[k] = f64_to_f16_array(gb), f64_to_f16_array(hb)
        planes[k] = pack_signs(B)
        a = f16(g[k]).astype(np.float32)[:, None] * f16(h[k]).astype(np.float32)[None, :]
        R = np.where(B, R - a, R + a).astype(np.float32)
    return planes, g, h


def dequant_dual(planes: np.ndarray, g: np.ndarray, h: np.ndarray) -> np.ndarray:
    """What = sum_k diag(g_k) B_k diag(h_k) in fp64, [out][in]."""
    K, out, words = planes.shape
    inf = words * 32
    What = np.zeros((out, inf), dtype=np.float64)
    for k in range(K):
        What += f16(g[k])[:, None] * unpack_signs(planes[k], inf) * f16(h[k])[None, :]
    return What


def gemm_dual(planes: np.ndarray, g: np.ndarray, h: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Y = X What^T in fp64.  X: fp16 (or its uint16 bits) [M][in]."""
    X = np.asarray(X)
    if X.dtype == np.uint16:
        X = X.view(np.float16)
    X = np.atleast_2d(X).astype(np.float64)
    return X @ dequant_dual(planes, g, h).T
