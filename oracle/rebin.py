"""CPU oracle for re-binarization with fixed scales (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library in ``gemm_rbq_encode_amd``, and the product path never
imports it.

QBB summary (atlas.scime.ai), "Approach": the binary bases are refined after
the analytical cascade.  The part of that refinement that needs no data
alternates two exact minimisations of ||W - sum_k a_k (.) B_k||^2: the
scales for fixed planes (the least-squares refit, ``oracle.refit``) and the
planes for fixed scales, done here.  For fixed scales the objective is a sum
over single weights, so each W_j independently takes the sign pattern
s in {-1, +1}^K whose value c = sum_k s_k a_k is nearest to it.

Readings where the pages are silent:
  * pattern p = 0 .. 2^K - 1 has s_k = +1 where bit k of p is 1 (plane bit
    1 = +1); c_p is summed in fp64, exactly (K binary16 values);
  * nearest in exact arithmetic; a weight exactly halfway between two
    values takes the larger value, and among patterns of equal value the
    largest p wins.  This keeps the encoder's sign(0) = +1: for K = 1 the
    planes are sign(W), and for K = 2 with a_1 > a_2 they are the cascade's;
  * a NaN weight is taken as -Inf (the smallest value's pattern), +-Inf as
    any other number;
  * a (row, group) whose scales are not all finite keeps its planes.

Exactness: |W - c_p| < |W - c_q|  <=>  (c_q - c_p) (2W - (c_p + c_q)) < 0,
the difference of the squared distances.  Both factors' signs are exact in
fp64: c_q - c_p is an exact sum of 2K binary16 values, and an fp64 sum or
difference is zero only when its exact value is, and never changes sign.

Parity status: pinned in tests/test_oracle_pins.py (exact rational brute
force over every pattern, with crafted ties and special values; the
objective's minimum over all plane choices; the cascade's planes for K = 1
and for K = 2 with a_1 > a_2 from the C oracle; the alternation with the
refit never raising the objective).
"""
from __future__ import annotations

import numpy as np

from .dual import pack_signs, unpack_signs

MAX_PLANES = 4


def patterns(K: int) -> np.ndarray:
    """[2^K][K] signs: row p has +1 where bit k of p is 1."""
    p = np.arange(1 << K)[:, None]
    return np.where((p >> np.arange(K)[None, :]) & 1, 1.0, -1.0)


def scale_values(scales: np.ndarray, group_size: int, inf: int) -> np.ndarray:
    """fp16 scales [K][out][G] -> fp64 per column [K][out][in]."""
    a = np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.repeat(a, group_size if group_size else inf, axis=2)


def rebinarize(W: np.ndarray, planes: np.ndarray, scales: np.ndarray, group_size: int = 0):
    """Planes for the fixed scales (module docstring).

    W fp32 [out][in]; planes uint32 [K][out][in/32] (kept where the scales
    are not finite); scales uint16 [K][out][G].  Returns (planes, flags)
    with flags bit 0 = some W non-finite, bit 3 = some (row, group) kept."""
    W = np.asarray(W, dtype=np.float32)
    out, inf = W.shape
    K = scales.shape[0]
    a = scale_values(scales, group_size, inf)                       # [K][out][in]
    S = patterns(K)
    c = np.einsum("pk,krj->prj", S, a)                              # [P][out][in], exact
    w = W.astype(np.float64)
    w = np.where(np.isnan(w), -np.inf, w)
    best = np.zeros((out, inf), dtype=np.int64)
    cb = c[0].copy()
    with np.errstate(invalid="ignore"):
        for p in range(1, S.shape[0]):
            prod = np.sign(cb - c[p]) * np.sign(2.0 * w - (c[p] + cb))   # < 0: p strictly nearer
            take = (prod < 0) | ((prod == 0) & (c[p] >= cb))
            best = np.where(take, p, best)
            cb = np.where(take, c[p], cb)
    new = np.stack([pack_signs(((best >> k) & 1).astype(bool)) for k in range(K)])
    finite_scale = np.isfinite(a).all(axis=0)                       # [out][in]
    keep = ~finite_scale.reshape(out, inf // 32, 32).all(axis=2)    # words of kept groups
    result = np.where(keep[None], np.asarray(planes, dtype=np.uint32), new)
    flags = (1 if not np.isfinite(W).all() else 0) | (8 if keep.any() else 0)
    return result.astype(np.uint32), flags


def objective(W: np.ndarray, planes: np.ndarray, scales: np.ndarray, group_size: int = 0) -> float:
    """||W - sum_k a_k (.) B_k||^2 in fp64."""
    W = np.asarray(W, dtype=np.float64)
    out, inf = W.shape
    a = scale_values(scales, group_size, inf)
    What = sum(a[k] * unpack_signs(planes[k], inf) for k in range(planes.shape[0]))
    return float(((W - What) ** 2).sum())
