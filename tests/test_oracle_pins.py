"""Pins for the CPU oracle: each test checks the oracle against something
other than itself (numpy's own rounding, brute force, closed forms, planted
structure, a hand-worked example), so that a dropped term, a wrong sign, a
wrong bit order or a wrong reading of the scale fails at least one test.

Method: RaBiT summary (paperlayer.ai) sections 4.1, 4.2, B and G; QBB
summary (atlas.scime.ai) "Approach"; XNOR-Net binarization (QBB "Builds on").
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

pytestmark = [pytest.mark.cpu,
              pytest.mark.filterwarnings("ignore:overflow encountered in cast")]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers written independently of the oracle (numpy / fractions only)
# ---------------------------------------------------------------------------

def unpack_signs(planes):
    """uint32 [K][out][in/32] -> int8 +-1 [K][out][in], LSB = lowest column."""
    K, out, words = planes.shape
    bits = np.unpackbits(planes.view(np.uint8).reshape(K, out, words * 4), axis=-1,
                         bitorder="little")
    return bits.astype(np.int8) * 2 - 1


def pack_signs(signs):
    """+-1 [..., in] -> uint32 words, LSB = lowest column (numpy packbits)."""
    bits = (np.asarray(signs) > 0).astype(np.uint8)
    packed = np.packbits(bits, axis=-1, bitorder="little")
    return packed.view(np.uint32)


def fp16_values(scales):
    return np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)


def rne16_exact(q: Fraction) -> int:
    """Round an exact non-negative rational to binary16 (ties to even), by
    exact comparison: the candidates are consecutive fp16 values."""
    assert q >= 0
    finite = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    # binary search on exact values
    lo, hi = 0, len(finite) - 1
    if q >= Fraction(65520):
        return 0x7C00
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if Fraction(finite[mid]) <= q:
            lo = mid
        else:
            hi = mid
    a, b = Fraction(finite[lo]), Fraction(finite[hi])
    if q == a:
        return lo
    if q >= b:
        return hi
    da, db = q - a, b - q
    if da < db:
        return lo
    if db < da:
        return hi
    return lo if lo % 2 == 0 else hi


# ---------------------------------------------------------------------------
# fp64 -> fp16 rounding: pinned to numpy's direct float64 -> float16 cast
# ---------------------------------------------------------------------------

def test_f16_roundtrip_all_finite():
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = h.view(np.float16)
    fin = np.isfinite(vals)
    back = oracle.f64_to_f16_array(vals[fin].astype(np.float64))
    assert np.array_equal(back, h[fin])
    for b in (0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF):
        assert oracle.f16_to_f64(b) == float(np.uint16(b).view(np.float16))


def test_f16_midpoints_against_numpy():
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2          # exact: fp16 values have <= 11 bits
    cases = [mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)]
    top = np.array([65504.0, 65519.0, 65519.99999999999, 65520.0, 65536.0, 1e10, np.inf,
                    2.0 ** -25, np.nextafter(2.0 ** -25, 1), np.nextafter(2.0 ** -25, 0),
                    2.0 ** -26, 0.0])
    allv = np.concatenate(cases + [top])
    allv = np.concatenate([allv, -allv])
    ref = allv.astype(np.float16).view(np.uint16)
    got = oracle.f64_to_f16_array(allv)
    assert np.array_equal(got, ref)


def test_f16_random_doubles_against_numpy():
    rng = np.random.default_rng(123)
    v = np.exp2(rng.uniform(-30, 17, size=400_000)) * rng.choice([-1.0, 1.0], size=400_000)
    v[::7] = rng.standard_normal(v[::7].size)
    assert np.array_equal(oracle.f64_to_f16_array(v), v.astype(np.float16).view(np.uint16))


def test_f16_rounds_once_not_via_fp32():
    # 1 + 2^-11 is the midpoint between 1 and 1.0009765625; one fp64 ulp above
    # it must round up.  Going through fp32 first would land on the midpoint
    # and round to even (1.0).
    v = np.nextafter(1.0 + 2.0 ** -11, 2.0)
    assert oracle.f64_to_f16(v) == 0x3C01
    assert np.float16(np.float32(v)).view(np.uint16) == 0x3C00


def test_f16_nan_and_overflow():
    assert oracle.f64_to_f16(float("nan")) & 0x7C00 == 0x7C00
    assert oracle.f64_to_f16(float("nan")) & 0x03FF != 0
    assert oracle.f64_to_f16(65520.0) == 0x7C00
    assert oracle.f64_to_f16(-70000.0) == 0xFC00


# ---------------------------------------------------------------------------
# encoder
# ---------------------------------------------------------------------------

def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_k3.json")))
    W = np.array([[float(v) for v in row] for row in g["W"]], dtype=np.float32)
    assert np.signbit(W[2, 16:]).all() and (W[2] == 0).all()
    K = g["num_planes"]
    planes, scales, flags = oracle.encode(W, K, g["group_size"])
    assert flags == 0
    exp_planes = pack_signs(np.array(g["signs"], dtype=np.int8)).reshape(K, g["out"], 1)
    assert np.array_equal(planes, exp_planes)
    exp_scales = np.array([[Fraction(s) for s in row] for row in g["scales"]])
    for k in range(K):
        for r in range(g["out"]):
            a = Fraction(float(np.uint16(scales[k, r, 0]).view(np.float16)))
            assert a == exp_scales[k][r], (k, r)


def _patterns(n):
    return np.array(list(itertools.product([-1.0, 1.0], repeat=n)))


@pytest.mark.parametrize("group", [8, 4])
def test_brute_force_small_groups(group):
    """Each step of the encoder, on each (row, group) of 4x32 matrices, must
    pick a sign pattern that maximises <R, b> over all 2^n patterns (that is
    the least-squares optimum for the best scale a >= 0), and its scale must
    be the fp16 value nearest the exact least-squares scale."""
    P = _patterns(group)
    rng = np.random.default_rng(7 + group)
    n_mats, K = 250, 3
    checked = 0
    for i in range(n_mats):
        W = (rng.standard_normal((4, 32)) * rng.uniform(0.01, 3)).astype(np.float32)
        if i % 10 == 0:
            W[rng.random(W.shape) < 0.2] = 0.0
        if i % 10 == 1:
            W[:, :] = np.float32(rng.uniform(0.1, 1)) * rng.choice([-1, 1], size=W.shape)
        if i % 10 == 2:
            W[rng.random(W.shape) < 0.3] = np.float32(-0.0)
        planes, scales, flags = oracle.encode(W, K, group)
        assert flags == 0
        S = unpack_signs(planes)                 # [K][4][32]
        A = fp16_values(scales)                  # [K][4][32/group]
        R = W.copy()
        for k in range(K):
            Rg = R.reshape(-1, group).astype(np.float64)
            b = S[k].reshape(-1, group).astype(np.float64)
            a = A[k].reshape(-1)
            best = (Rg @ P.T).max(axis=1)
            got = (Rg * b).sum(axis=1)
            assert np.array_equal(got, best), (i, k)
            for gi in range(Rg.shape[0]):
                exact = sum(Fraction(float(abs(v))) for v in Rg[gi]) / group
                assert rne16_exact(exact) == scales[k].reshape(-1)[gi], (i, k, gi)
                checked += 1
            # zeros (either sign) must be coded +1
            zero = (R.reshape(-1, group) == 0)
            assert (b[zero] == 1).all()
            # residual against the stored scale, fp32, one rounding
            R = (R - (A[k].repeat(group, axis=1).astype(np.float32) * S[k].astype(np.float32))
                 ).astype(np.float32)
    assert checked == n_mats * K * 4 * (32 // group)


def test_scale_is_best_fp16_for_its_signs():
    """For each plane the stored scale is the fp16 value minimising
    ||R - a B||^2 over fp16 values of a (checked against both neighbours),
    on per-row (n = 512) and grouped (n = 128) encodings."""
    W = workloads.gaussian_weight(64, 512, seed=11, outliers=True)
    for group in (0, 128):
        K = 4
        planes, scales, _ = oracle.encode(W, K, group)
        S = unpack_signs(planes).astype(np.float64)
        n = group or 512
        R = W.astype(np.float64)
        for k in range(K):
            a = fp16_values(scales[k])
            a_cols = np.repeat(a, n, axis=1)
            for delta in (0, -1, 1):
                h = (scales[k].astype(np.int32) + delta).astype(np.uint16)
                ad = np.repeat(fp16_values(h), n, axis=1)
                err = ((R - ad * S[k]) ** 2).reshape(64, -1, n).sum(axis=2)
                if delta == 0:
                    base = err
                else:
                    assert (base <= err * (1 + 1e-12)).all()
            # fp32 residual chain as the encoder defines it
            R = (R.astype(np.float32) - (a_cols.astype(np.float32) * S[k].astype(np.float32))
                 ).astype(np.float64)


def test_residual_norm_non_increasing():
    W = workloads.gaussian_weight(128, 1024, seed=5, outliers=True)
    for group in (0, 128):
        K = 6
        planes, scales, _ = oracle.encode(W, K, group)
        S = unpack_signs(planes).astype(np.float64)
        n = group or 1024
        approx = np.zeros_like(W, dtype=np.float64)
        prev = np.linalg.norm(W.astype(np.float64), axis=1)
        for k in range(K):
            approx += np.repeat(fp16_values(scales[k]), n, axis=1) * S[k]
            cur = np.linalg.norm(W.astype(np.float64) - approx, axis=1)
            assert (cur <= prev * (1 + 1e-6)).all(), k
            assert (cur < prev).mean() > 0.99, k   # strictly smaller almost everywhere
            prev = cur


def test_k1_is_xnor_binarization():
    """K = 1 is XNOR-Net / BWN binarization: B = sign(W), alpha = ||W_r||_1 / n."""
    W = workloads.gaussian_weight(300, 4096, seed=3, outliers=True)
    planes, scales, _ = oracle.encode(W, 1, 0)
    alpha = np.abs(W.astype(np.float64)).mean(axis=1)       # numpy pairwise sum
    assert np.array_equal(scales[0, :, 0], alpha.astype(np.float16).view(np.uint16))
    assert np.array_equal(unpack_signs(planes)[0], np.where(W >= 0, 1, -1))


def test_planted_planes_recovered():
    rng = np.random.default_rng(99)
    out, n = 40, 256
    B1 = rng.choice([-1, 1], size=(out, n))
    B2 = B1.copy()
    for r in range(out):                   # exactly n/2 disagreements per row
        flip = rng.choice(n, n // 2, replace=False)
        B2[r, flip] *= -1
    c1 = np.float16(rng.uniform(0.1, 1.0, size=(out, 1))).astype(np.float64)
    c2 = (c1 * rng.uniform(0.1, 0.9, size=(out, 1))).astype(np.float16).astype(np.float64)
    W = (c1 * B1 + c2 * B2).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), c1 * B1 + c2 * B2)   # exact
    K = 3
    planes, scales, _ = oracle.encode(W, K, 0)
    S = unpack_signs(planes)
    assert np.array_equal(S[0], B1) and np.array_equal(S[1], B2)
    assert np.array_equal(fp16_values(scales[0]), c1)
    assert np.array_equal(fp16_values(scales[1]), c2)
    assert (S[2] == 1).all() and (scales[2] == 0).all()
    # constant rows: W = +-c gives B_2 = all +1 (sign(0) = +1) and a_2 = 0
    Wc = np.where(rng.random((8, 64)) < 0.5, 0.25, -0.25).astype(np.float32)
    p, s, _ = oracle.encode(Wc, 2, 0)
    assert (unpack_signs(p)[1] == 1).all() and (s[1] == 0).all()
    assert (fp16_values(s[0]) == 0.25).all()


def test_ragged_and_degenerate_shapes():
    W = workloads.gaussian_weight(3, 96, seed=1)
    p, s, f = oracle.encode(W, 2, 0)
    assert p.shape == (2, 3, 3) and s.shape == (2, 3, 1) and f == 0
    p, s, f = oracle.encode(np.zeros((0, 64), np.float32), 2, 0)
    assert p.shape == (2, 0, 2)
    with pytest.raises(ValueError):
        oracle.encode(np.zeros((2, 48), np.float32), 2, 0)        # in % 32 != 0
    with pytest.raises(ValueError):
        oracle.encode(np.zeros((2, 64), np.float32), 9, 0)        # K > 8
    Wn = W.copy()
    Wn[1, 5] = np.nan
    assert oracle.encode(Wn, 2, 0)[2] & 1
    Wbig = np.full((1, 32), 70000.0, np.float32)
    assert oracle.encode(Wbig, 1, 0)[2] & 2


def test_encode_threads_do_not_change_results():
    W = workloads.gaussian_weight(200, 1024, seed=8, outliers=True)
    n0 = oracle.num_threads()
    ref = oracle.encode(W, 3, 128)
    oracle.set_num_threads(1)
    try:
        one = oracle.encode(W, 3, 128)
    finally:
        oracle.set_num_threads(n0)
    assert np.array_equal(ref[0], one[0]) and np.array_equal(ref[1], one[1])


# ---------------------------------------------------------------------------
# dequantize / multiply
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K,group", [(1, 0), (2, 0), (4, 128), (8, 128), (3, 64)])
def test_dequant_against_numpy_unpack(K, group):
    out, inf = 48, 512
    planes = workloads.random_planes(K, out, inf, seed=K)
    G = inf // group if group else 1
    scales = workloads.random_scales(K, out, G, seed=10 + K)
    What = oracle.dequant(planes, scales, group)
    n = group or inf
    ref = (np.repeat(fp16_values(scales), n, axis=2) * unpack_signs(planes)).sum(axis=0)
    assert np.array_equal(What, ref)


@pytest.mark.parametrize("K,group,M", [(2, 0, 1), (2, 0, 5), (4, 128, 3), (1, 0, 2)])
def test_gemm_against_numpy_matmul(K, group, M):
    out, inf = 96, 1024
    planes = workloads.random_planes(K, out, inf, seed=20 + K)
    G = inf // group if group else 1
    scales = workloads.random_scales(K, out, G, seed=30 + K)
    X = workloads.gaussian_activations(M, inf, seed=40 + M)
    Y = oracle.gemm(planes, scales, X, group)
    n = group or inf
    What = (np.repeat(fp16_values(scales), n, axis=2) * unpack_signs(planes)).sum(axis=0)
    ref = X.view(np.float16).astype(np.float64) @ What.T
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_gemm_closed_forms():
    K, out, inf, group = 3, 64, 768, 128
    planes = workloads.random_planes(K, out, inf, seed=1)
    scales = workloads.random_scales(K, out, inf // group, seed=2)
    A = fp16_values(scales)
    # x = 1: y_r = sum_k sum_t a_kt (2 popcount_kt - n)
    ones = np.full((1, inf), 0x3C00, np.uint16)
    y = oracle.gemm(planes, scales, ones, group)[0]
    pc = np.unpackbits(planes.view(np.uint8), bitorder="little").reshape(K, out, inf // group, group).sum(-1).astype(np.int64)
    ref = (A * (2 * pc - group)).sum(axis=(0, 2))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)
    # x = e_j: column j of What
    S = unpack_signs(planes)
    for j in (0, 1, 31, 32, 127, 128, 500, inf - 1):
        e = np.zeros((1, inf), np.uint16)
        e[0, j] = 0x3C00
        col = oracle.gemm(planes, scales, e, group)[0]
        assert np.array_equal(col, (A[:, :, j // group] * S[:, :, j]).sum(axis=0))


def test_gemm_empty_and_ragged():
    planes = workloads.random_planes(2, 5, 96, seed=3)
    scales = workloads.random_scales(2, 5, 1, seed=4)
    assert oracle.gemm(planes, scales, np.zeros((0, 96), np.uint16)).shape == (0, 5)
    X = workloads.gaussian_activations(2, 96, seed=5)
    Y = oracle.gemm(planes, scales, X)
    What = oracle.dequant(planes, scales)
    np.testing.assert_allclose(Y, X.view(np.float16).astype(np.float64) @ What.T, rtol=1e-13)


def test_scale_rounds_once_in_encoder():
    """A row whose exact mean is 1 + 2^-11 + 2^-30: one fp64 -> fp16 rounding
    gives 1 + 2^-10 (0x3C01); rounding through fp32 first would land on the
    fp16 midpoint 1 + 2^-11 and go to even (0x3C00)."""
    row = np.full(32, 1 + 2.0 ** -11, dtype=np.float64)
    row[30] = 2 + 2.0 ** -10
    row[31] = 2.0 ** -25
    W = row.astype(np.float32)[None, :]
    assert np.array_equal(W[0].astype(np.float64), row)
    assert sum(Fraction(v) for v in row) / 32 == 1 + Fraction(1, 2 ** 11) + Fraction(1, 2 ** 30)
    _, scales, _ = oracle.encode(W, 1, 0)
    assert scales[0, 0, 0] == 0x3C01


def test_row_stacking_commutes_with_encoding():
    """Per-row scales make rows independent: encoding [W1; W2] gives the
    planes and scales of W1 and W2 stacked (the fused q/k/v and gate/up
    layouts rely on this)."""
    W1 = workloads.gaussian_weight(40, 512, seed=1, outliers=True)
    W2 = workloads.gaussian_weight(24, 512, seed=2, outliers=True)
    p, s, _ = oracle.encode(np.concatenate([W1, W2]), 2, 0)
    p1, s1, _ = oracle.encode(W1, 2, 0)
    p2, s2, _ = oracle.encode(W2, 2, 0)
    assert np.array_equal(p, np.concatenate([p1, p2], axis=1))
    assert np.array_equal(s, np.concatenate([s1, s2], axis=1))


# ---------------------------------------------------------------------------
# refit: joint least-squares scales for fixed planes (QBB "Approach")
# ---------------------------------------------------------------------------

def _exact_ls(B, w):
    """Exact least-squares coefficients for the +-1 rows of B (K x n ints)
    and fp32 values w (Fractions), by Gaussian elimination on rationals."""
    K = B.shape[0]
    G = [[Fraction(int(np.dot(B[k], B[l]))) for l in range(K)] for k in range(K)]
    b = [sum((wj if s > 0 else -wj) for s, wj in zip(B[k], w)) for k in range(K)]
    A = [G[i] + [b[i]] for i in range(K)]
    for c in range(K):
        piv = next(i for i in range(c, K) if A[i][c] != 0)
        A[c], A[piv] = A[piv], A[c]
        for i in range(K):
            if i != c and A[i][c] != 0:
                f = A[i][c] / A[c][c]
                A[i] = [x - f * y for x, y in zip(A[i], A[c])]
    return [A[i][K] / A[i][i] for i in range(K)]


def _rne16_signed(q):
    h = rne16_exact(abs(q))
    return h | (0x8000 if q < 0 else 0)


def _near_midpoint(q, rel=2.0 ** -40):
    """True if the exact q lies within rel of a binary16 rounding midpoint."""
    lo = np.uint16(rne16_exact(abs(q)))
    v = Fraction(float(lo.view(np.float16)))
    nb = [v]
    for d in (-1, 1):
        u = int(lo) + d
        if 0 <= u < 0x7C00:
            nb.append(Fraction(float(np.uint16(u).view(np.float16))))
    mids = [(x + y) / 2 for x in nb for y in nb if x < y]
    return any(abs(abs(q) - m) <= rel * abs(q) for m in mids)


@pytest.mark.parametrize("K,group", [(1, 0), (2, 0), (3, 128), (4, 128), (8, 0)])
def test_refit_is_exact_least_squares(K, group):
    """Random planes, Gaussian W: each refit scale is the exact least-squares
    coefficient (rational arithmetic on the fp32 values) rounded once to
    binary16, except where that exact value lies within 2^-40 of a rounding
    midpoint (the oracle's fp64 solve may then land on either side)."""
    rng = np.random.default_rng(50 + K)
    out, inf = 5, 256
    signs = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, out, inf))
    W = workloads.gaussian_weight(out, inf, seed=60 + K)
    G = inf // group if group else 1
    keep = np.zeros((K, out, G), dtype=np.uint16)
    refit, flags = oracle.refit(W, pack_signs(signs), keep, group)
    assert flags == 0
    n = group or inf
    checked = 0
    for r in range(out):
        for t in range(G):
            cols = slice(t * n, (t + 1) * n)
            a = _exact_ls(signs[:, r, cols].astype(np.int64), [Fraction(float(x)) for x in W[r, cols]])
            for k in range(K):
                want = _rne16_signed(a[k])
                if refit[k, r, t] != want:
                    assert _near_midpoint(a[k]), (k, r, t, float(a[k]))
                else:
                    checked += 1
    assert checked >= K * out * G - 1


@pytest.mark.parametrize("K,group", [(2, 0), (4, 128)])
def test_refit_matches_numpy_lstsq(K, group):
    """Against numpy's least-squares solver on the +-1 design matrix of each
    (row, group): equal binary16, or one unit apart at most."""
    W = workloads.gaussian_weight(12, 512, seed=70, outliers=True)
    planes, scales, _ = oracle.encode(W, K, group)
    refit, flags = oracle.refit(W, planes, scales, group)
    assert flags == 0
    signs = unpack_signs(planes).astype(np.float64)
    n = group or 512
    G = 512 // n
    for r in range(12):
        for t in range(G):
            cols = slice(t * n, (t + 1) * n)
            a = np.linalg.lstsq(signs[:, r, cols].T, W[r, cols].astype(np.float64), rcond=None)[0]
            got = refit[:, r, t].astype(np.int64)
            want = a.astype(np.float16).view(np.uint16).astype(np.int64)
            assert np.all(np.abs(got - want) <= 1), (r, t, got, want)


def test_refit_one_plane_is_cascade_scale():
    """With one plane the least-squares scale is sum_j |W_j| / n: the
    cascade's own scale, bit for bit (same serial sum, same rounding)."""
    for group in (0, 128):
        W = workloads.gaussian_weight(16, 1024, seed=80 + group, outliers=True)
        planes, scales, _ = oracle.encode(W, 1, group)
        refit, flags = oracle.refit(W, planes, np.zeros_like(scales), group)
        assert flags == 0 and np.array_equal(refit, scales)


def test_refit_recovers_planted_scales():
    """W = sum_k a_k B_k exactly (fp16 scales, +-1 planes, exact in fp32):
    the refit returns a_k exactly for every row, whichever planes."""
    rng = np.random.default_rng(90)
    K, out, inf = 3, 8, 256
    signs = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, out, inf))
    a = rng.choice(np.array([0.5, -0.25, 0.375, 0.0625, -1.5, 2.0, 0.75], dtype=np.float16),
                   size=(K, out))
    W64 = np.einsum("kr,krj->rj", a.astype(np.float64), signs.astype(np.float64))
    W = W64.astype(np.float32)
    assert np.array_equal(W.astype(np.float64), W64)
    refit, flags = oracle.refit(W, pack_signs(signs), np.zeros((K, out, 1), np.uint16), 0)
    assert flags == 0
    assert np.array_equal(refit[:, :, 0], a.view(np.uint16))


def test_refit_never_worse_than_cascade():
    """For the cascade's planes, the refit scales reconstruct W at least as
    well as the cascade's own scales, row by row (both rounded to binary16),
    and clearly better in total."""
    for K, group in ((2, 0), (4, 128)):
        W = workloads.gaussian_weight(32, 1024, seed=100 + K, outliers=True)
        planes, scales, _ = oracle.encode(W, K, group)
        refit, flags = oracle.refit(W, planes, scales, group)
        assert flags == 0
        W64 = W.astype(np.float64)
        e0 = ((W64 - oracle.dequant(planes, scales, group)) ** 2).sum(axis=1)
        e1 = ((W64 - oracle.dequant(planes, refit, group)) ** 2).sum(axis=1)
        assert np.all(e1 <= e0 * (1 + 1e-4))
        assert e1.sum() < 0.99 * e0.sum()


def test_refit_keeps_scales_of_singular_or_nonfinite_groups():
    """All-zero rows give identical planes (all +1), so G is singular: the
    given scales stay and flag bit 2 is set.  A non-finite W sets bit 0 and
    keeps that row's scales; other rows are refit."""
    W = workloads.gaussian_weight(4, 256, seed=5)
    W[1] = 0.0
    W[2, 7] = np.inf
    planes, scales, _ = oracle.encode(W, 2, 0)
    marker = np.full_like(scales, 0x1234)
    refit, flags = oracle.refit(W, planes, marker, 0)
    assert flags == 1 | 4
    assert np.all(refit[:, 1] == 0x1234) and np.all(refit[:, 2] == 0x1234)
    assert np.all(refit[:, 0] != 0x1234) and np.all(refit[:, 3] != 0x1234)


def test_silu_mul_against_scipy_expit():
    """silu(v) * u = v * sigmoid(v) * u, with scipy's logistic function, and
    the closed values silu(0) = 0, silu(v) -> v for large v, -> 0 for very
    negative v; columns pair as (2i, 2i+1)."""
    from scipy.special import expit
    rng = np.random.default_rng(7)
    Y = rng.standard_normal((3, 10)) * 4
    H = oracle.silu_mul(Y)
    assert H.shape == (3, 5)
    np.testing.assert_allclose(H, Y[:, 0::2] * expit(Y[:, 0::2]) * Y[:, 1::2], rtol=1e-14)
    Z = np.array([[0.0, 5.0, 40.0, 2.0, -40.0, 3.0]])
    np.testing.assert_allclose(oracle.silu_mul(Z), [[0.0, 80.0, -40.0 * np.exp(-40.0) * 3.0]], rtol=1e-12)


# ---------------------------------------------------------------------------
# dual-scale paths (RaBiT section 4.1: per-channel scales on both sides of
# each binary core; section 4.3 / "RaBiT initialization": residual SVID)
# ---------------------------------------------------------------------------

from oracle import dual  # noqa: E402


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def test_dual_rank1_exact_for_rank1_magnitudes():
    """|W| = a b^T exactly: the fit reproduces it and B_1 = sign(W)."""
    rng = np.random.default_rng(41)
    # binary16 factors: their products are exact in fp32, so |W| is exactly rank 1
    a = rng.uniform(0.5, 2.0, 24).astype(np.float16).astype(np.float64)
    b = rng.uniform(0.1, 1.0, 64).astype(np.float16).astype(np.float64)
    S = np.where(rng.random((24, 64)) < 0.5, -1.0, 1.0)
    W = (S * np.outer(a, b)).astype(np.float32)
    assert np.array_equal(np.abs(W).astype(np.float64), np.outer(a, b))
    u, v = dual.svid_rank1(np.abs(W).astype(np.float64))
    A = np.abs(W).astype(np.float64)
    assert np.abs(np.outer(u, v) - A).max() <= 1e-12 * A.max()
    planes, g, h = dual.encode_dual(W, 1)
    assert np.array_equal(unpack_signs(planes)[0], S.astype(np.int8))


def test_dual_rank1_matches_numpy_svd():
    """On non-square |R| the fit equals the top singular triple s1 u1 v1^T
    (a transposed operand or a dropped normalisation would not)."""
    rng = np.random.default_rng(42)
    A = np.abs(rng.standard_normal((48, 80)))
    u, v = dual.svid_rank1(A)
    U, s, Vt = np.linalg.svd(A)
    ref = s[0] * np.outer(U[:, 0], Vt[0])
    assert np.linalg.norm(np.outer(u, v) - ref) <= 1e-9 * np.linalg.norm(ref)


def test_dual_row_constant_magnitudes_give_row_scales():
    """|W_rj| = c_r: the rank-1 fit is c 1^T, the per-row scale of the
    single-scale method (mean |W_r| = c_r)."""
    rng = np.random.default_rng(43)
    c = rng.uniform(0.01, 0.05, 16)
    W = (np.where(rng.random((16, 96)) < 0.5, -1.0, 1.0) * c[:, None]).astype(np.float32)
    u, v = dual.svid_rank1(np.abs(W).astype(np.float64))
    assert np.allclose(np.outer(u, v), np.abs(W).astype(np.float64), rtol=1e-12, atol=0)
    assert np.allclose(v, v[0], rtol=1e-12)


def test_dual_fit_never_worse_than_row_means():
    """The first least-squares step from v = 1 is the row-mean fit; later
    steps only lower the error, so the final fit is no worse."""
    rng = np.random.default_rng(44)
    for _ in range(5):
        A = np.abs(rng.standard_normal((32, 64)) * rng.uniform(0.2, 3.0, 64)[None, :])
        u, v = dual.svid_rank1(A)
        e_fit = np.linalg.norm(A - np.outer(u, v))
        e_row = np.linalg.norm(A - A.mean(axis=1, keepdims=True))
        assert e_fit <= e_row * (1 + 1e-12)
        assert e_fit < e_row   # column scales that differ are worth something


def test_dual_residual_norms_do_not_grow():
    rng = np.random.default_rng(45)
    W = workloads.gaussian_weight(32, 256, seed=46, outliers=True)
    planes, g, h = dual.encode_dual(W, 4)
    prev = np.linalg.norm(W.astype(np.float64))
    for k in range(1, 5):
        What = dual.dequant_dual(planes[:k], g[:k], h[:k])
        err = np.linalg.norm(W.astype(np.float64) - What)
        assert err <= prev * (1 + 1e-3)
        prev = err
    # and the dual scales fit at least as well as one scale per row
    p1, s1, _ = oracle.encode(W, 4)
    err_row = np.linalg.norm(W.astype(np.float64) - oracle.dequant(p1, s1))
    assert prev <= err_row * 1.01


def test_dual_first_plane_matches_c_oracle_and_layout():
    """B_1 = sign(W) packed in the canonical layout: the same words as the C
    oracle's first plane (independent code); -0.0 counts as +1."""
    W = workloads.gaussian_weight(8, 160, seed=47)
    W[1, 5] = -0.0
    W[2, 33] = 0.0
    planes, _, _ = dual.encode_dual(W, 1)
    p_c, _, _ = oracle.encode(W, 1)
    assert np.array_equal(planes, p_c)


def test_dual_scales_are_balanced_fp16_roundings():
    rng = np.random.default_rng(48)
    A = np.abs(rng.standard_normal((20, 64))) * 0.02
    u, v = dual.svid_rank1(A)
    c = math.sqrt(math.sqrt(u @ u) / math.sqrt(v @ v))
    g, h = dual.svid_scales(A)
    assert np.array_equal(g, np.asarray(u / c, dtype=np.float64).astype(np.float16).view(np.uint16))
    assert np.array_equal(h, np.asarray(v * c, dtype=np.float64).astype(np.float16).view(np.uint16))
    assert abs(np.linalg.norm(u / c) - np.linalg.norm(v * c)) <= 1e-12 * np.linalg.norm(v * c)


def test_dual_layer_output_against_loops():
    """y_r = sum_k g_k[r] sum_j (bit ? +1 : -1) h_k[j] x_j by plain loops."""
    rng = np.random.default_rng(49)
    out, inf, K = 4, 64, 2
    words = rng.integers(0, 2 ** 32, (K, out, inf // 32), dtype=np.uint64).astype(np.uint32)
    g = rng.uniform(0.01, 0.1, (K, out)).astype(np.float16).view(np.uint16)
    h = rng.uniform(0.2, 2.0, (K, inf)).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((1, inf)).astype(np.float16)
    y = dual.gemm_dual(words, g, h, x)[0]
    for r in range(out):
        ref = 0.0
        for k in range(K):
            acc = 0.0
            for j in range(inf):
                bit = (int(words[k, r, j // 32]) >> (j % 32)) & 1
                acc += (1.0 if bit else -1.0) * float(_f16(h[k, j])) * float(x[0, j])
            ref += float(_f16(g[k, r])) * acc
        assert abs(y[r] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_dual_zero_matrix_gives_zero_scales():
    W = np.zeros((4, 64), np.float32)
    planes, g, h = dual.encode_dual(W, 2)
    assert not g.any() and not h.any()
    assert (planes == 0xFFFFFFFF).all()


# ---------------------------------------------------------------------------
# re-binarization for fixed scales (oracle/rebin.py; QBB "Approach")
# ---------------------------------------------------------------------------

from oracle import rebin  # noqa: E402


def rebin_brute_force(W, scales, group_size=0):
    """Pattern per weight by exact rational arithmetic over every sign
    pattern: smallest |W - c|, then the larger value c, then the larger p
    (p's bit k = sign of plane k); NaN counts as -Inf.  Returns int [out][in]."""
    K, out, G = scales.shape
    inf = W.shape[1]
    n = group_size if group_size else inf
    a = scales.view(np.float16).astype(np.float64)
    best = np.zeros((out, inf), dtype=np.int64)
    for r in range(out):
        for t in range(G):
            vals = [sum(Fraction(float(a[k, r, t])) * (1 if (p >> k) & 1 else -1) for k in range(K))
                    for p in range(1 << K)]
            for j in range(t * n, (t + 1) * n):
                w = float(W[r, j])
                if math.isnan(w) or math.isinf(w):
                    # -Inf (and NaN): the smallest value; +Inf: the largest
                    key = (lambda p: (vals[p], -p)) if (math.isnan(w) or w < 0) else (lambda p: (-vals[p], -p))
                else:
                    fw = Fraction(w)
                    key = lambda p: (abs(fw - vals[p]), -vals[p], -p)
                best[r, j] = min(range(1 << K), key=key)
    return best


def patterns_of(planes):
    """uint32 planes [K][out][in/32] -> pattern index p [out][in]."""
    s = unpack_signs(planes)
    return sum(((s[k] > 0).astype(np.int64) << k) for k in range(s.shape[0]))


def special_rebin_case(K, rng, group_size=0):
    """Scales with equal, zero and negative entries, and weights placed on
    the midpoints, on the values, at +-0, tiny, subnormal, +-Inf and NaN."""
    out, inf = 6, 256
    G = inf // group_size if group_size else 1
    a = np.abs(rng.standard_normal((K, out, G))) * 0.05 + 0.01
    a[:, 1] = a[0, 1]                                # all scales equal in row 1
    a[-1, 2] = 0.0                                   # a zero scale
    a[0, 3] = -a[0, 3]                               # a negative scale
    a[:, 5] = 0.0                                    # an all-zero row
    scales = a.astype(np.float16).view(np.uint16)
    af = scales.view(np.float16).astype(np.float64)
    W = (rng.standard_normal((out, inf)) * 0.05).astype(np.float32)
    n = group_size if group_size else inf
    P = rebin.patterns(K)
    for r in range(out):
        for j in range(0, inf, 3):
            vals = P @ af[:, r, j // n]
            u, v = rng.choice(vals, 2)
            W[r, j] = np.float32((u + v) / 2)        # exact: a few fp16 terms
        for j in range(1, inf, 7):
            W[r, j] = np.float32(rng.choice(P @ af[:, r, j // n]))
    W[0, 2], W[0, 4], W[0, 5] = 0.0, -0.0, 1e-30
    W[0, 7], W[0, 8] = -1e-40, 1e-40                 # fp32 subnormals
    W[4, 10], W[4, 11], W[4, 13] = np.inf, -np.inf, np.nan
    return W, scales


@pytest.mark.parametrize("K,group", [(1, 0), (2, 0), (3, 0), (4, 0), (2, 128), (4, 128)])
def test_rebin_matches_exact_brute_force(K, group):
    rng = np.random.default_rng(100 + K + group)
    W, scales = special_rebin_case(K, rng, group)
    planes0 = np.zeros((K, W.shape[0], W.shape[1] // 32), np.uint32)
    got, flags = rebin.rebinarize(W, planes0, scales, group)
    assert np.array_equal(patterns_of(got), rebin_brute_force(W, scales, group))
    assert flags == 1                                # the Inf/NaN weights


@pytest.mark.parametrize("K", [1, 2, 3])
def test_rebin_reaches_the_minimum_over_all_planes(K):
    """The objective equals the minimum over every choice of K planes (all
    2^(K*in) of them for a 1 x 32 row, checked weight by weight)."""
    rng = np.random.default_rng(7 + K)
    W = (rng.standard_normal((3, 32)) * 0.05).astype(np.float32)
    scales = (np.abs(rng.standard_normal((K, 3, 1))) * 0.05).astype(np.float16).view(np.uint16)
    got, _ = rebin.rebinarize(W, np.zeros((K, 3, 1), np.uint32), scales)
    a = scales.view(np.float16).astype(np.float64)
    best = 0.0
    for r in range(3):
        for j in range(32):
            best += min((float(W[r, j]) - sum(s[k] * a[k, r, 0] for k in range(K))) ** 2
                        for s in itertools.product((-1, 1), repeat=K))
    assert rebin.objective(W, got, scales) == pytest.approx(best, rel=1e-12)


def test_rebin_one_plane_is_sign():
    W = workloads.gaussian_weight(16, 256, seed=31)
    W[3, :5] = [0.0, -0.0, 1e-40, -1e-40, 0.0]
    p, s, _ = oracle.encode(W, 1)
    got, flags = rebin.rebinarize(W, np.zeros_like(p), s)
    assert flags == 0 and np.array_equal(got, p)
    assert np.array_equal(unpack_signs(got)[0], np.where(W >= 0, 1, -1))


@pytest.mark.parametrize("group", [0, 128])
def test_rebin_two_planes_keep_the_cascade_when_a1_exceeds_a2(group):
    """With a_1 > a_2 the cascade's two signs are the nearest of the four
    values (midpoints -a_1, 0, a_1, ties up), so re-binarizing the C
    oracle's encoding changes nothing."""
    W = workloads.gaussian_weight(64, 512, seed=32, outliers=True)
    p, s, _ = oracle.encode(W, 2, group)
    a = s.view(np.float16).astype(np.float64)
    assert (a[0] > a[1]).all()
    got, _ = rebin.rebinarize(W, np.zeros_like(p), s, group)
    assert np.array_equal(got, p)


@pytest.mark.parametrize("K,group", [(3, 0), (4, 128), (4, 0)])
def test_rebin_alternation_with_refit_never_raises_the_objective(K, group):
    """Planes re-chosen for fixed scales are never worse than the cascade's
    planes, and alternating with the C oracle's refit keeps descending
    (each scale rounding can cost at most a binary16 unit's share)."""
    W = workloads.gaussian_weight(48, 512, seed=33 + K, outliers=True)
    p, s, _ = oracle.encode(W, K, group)
    prev = rebin.objective(W, p, s, group)
    for _ in range(3):
        p2, _ = rebin.rebinarize(W, p, s, group)
        e = rebin.objective(W, p2, s, group)
        assert e <= prev * (1 + 1e-12)
        s, _ = oracle.refit(W, p2, s, group)
        prev, p = rebin.objective(W, p2, s, group), p2
        assert prev <= e * (1 + 1e-3)
    first = rebin.objective(W, *oracle.encode(W, K, group)[:2], group)
    assert prev < first


def test_rebin_keeps_planes_of_nonfinite_scales():
    W = workloads.gaussian_weight(4, 256, seed=34)
    p, s, _ = oracle.encode(W, 2, 128)
    s = s.copy()
    s[1, 2, 1] = np.float16(np.inf).view(np.uint16)
    s[0, 3, 0] = np.float16(np.nan).view(np.uint16)
    junk = np.full_like(p, 0x5A5A5A5A)
    got, flags = rebin.rebinarize(W, junk, s, 128)
    assert flags == 8
    kept = np.zeros((4, 8), bool)
    kept[2, 4:8] = kept[3, 0:4] = True
    assert np.array_equal(got[:, kept], junk[:, kept])
    assert np.array_equal(got[:, ~kept], p[:, ~kept])


# ---------------------------------------------------------------------------
# dual-scale residual step: hand-worked example (tests/golden/dual_rank1_k3.json)
# ---------------------------------------------------------------------------

def _rne16_pos_sqrt(x2: Fraction) -> Fraction:
    """binary16 value nearest sqrt(x2) for a positive rational x2 whose square
    root is irrational (no ties), decided exactly by comparing squares."""
    assert x2 > 0
    e = 0
    while Fraction(2) ** (2 * (e + 1)) <= x2:
        e += 1
    while Fraction(2) ** (2 * e) > x2:
        e -= 1
    q = Fraction(2) ** (max(e, -14) - 10)          # quantum of the binade (subnormals: 2^-24)
    k = 0
    lo, hi = 0, 1 << 40                             # largest k with (k q)^2 <= x2
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if (mid * q) ** 2 <= x2:
            lo = mid
        else:
            hi = mid - 1
    k = lo
    m = (k + Fraction(1, 2)) * q
    assert m * m != x2
    return (k + 1) * q if x2 > m * m else k * q


def _decimal_rne16(x, margin):
    """binary16 value nearest the positive Decimal x, with x required to lie
    more than `margin` (relative) away from the midpoint it is compared with."""
    from decimal import Decimal
    e = 0
    while Decimal(2) ** (e + 1) <= x:
        e += 1
    while Decimal(2) ** e > x:
        e -= 1
    q = Decimal(2) ** (max(e, -14) - 10)
    k = int(x / q)
    m = (Decimal(k) + Decimal("0.5")) * q
    assert abs(x - m) > Decimal(margin) * x, f"{x} lies within {margin} of a binary16 midpoint"
    return Fraction((k + 1) if x > m else k) * Fraction(q)


def _decimal_svid(A, iters=20):
    """The rank-1 fit of the dual-scale reading (alternating least squares
    from v = 1) in 80-digit decimal arithmetic, balanced: (g, h) as Decimals."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 80
        Ad = [[Decimal(x.numerator) / Decimal(x.denominator) for x in row] for row in A]
        out, inf = len(Ad), len(Ad[0])
        v = [Decimal(1)] * inf
        for _ in range(iters):
            vv = sum(x * x for x in v)
            u = [sum(Ad[r][j] * v[j] for j in range(inf)) / vv for r in range(out)]
            uu = sum(x * x for x in u)
            v = [sum(Ad[r][j] * u[r] for r in range(out)) / uu for j in range(inf)]
        c = (sum(x * x for x in u).sqrt() / sum(x * x for x in v).sqrt()).sqrt()
        return [x / c for x in u], [x * c for x in v]


def test_dual_residual_subtracts_the_stored_binary16_scales():
    """RaBiT section 4.1 / 4.3: the residual after path k subtracts the path
    as stored, g_k h_k^T in binary16.  On |W| = a b^T exactly (rank 1,
    ||b|| = 2 ||a||) the first plane's scales are a sqrt(2) and b / sqrt(2),
    rounded once to binary16; the residual is then S (a b - g h) exactly, so
    B_2 = S where a b > g h and -S where a b < g h.  Plane 2's scales come
    from an 80-digit evaluation of the same 20 least-squares steps, and B_3
    from the exact sign of R_1 - B_2 g_2 h_2.  Subtracting the unrounded fit
    u v^T (or rounding only one of g, h) breaks B_2."""
    doc = json.load(open(os.path.join(GOLDEN, "dual_rank1_k3.json")))
    a = [Fraction(s) for s in doc["a"]]
    b = [Fraction(s) for s in doc["b"]]
    S = doc["S"]
    out, inf = doc["out"], doc["in"]
    assert sum(x * x for x in b) == 4 * sum(x * x for x in a)
    W = np.array([[float(S[r][j] * a[r] * b[j]) for j in range(inf)] for r in range(out)], dtype=np.float32)
    assert all(Fraction(float(W[r, j])) == S[r][j] * a[r] * b[j] for r in range(out) for j in range(inf))
    planes, g, h = dual.encode_dual(W, 3)
    got = unpack_signs(planes)                       # [K][out][in] of +-1

    # plane 1: exact roundings of a sqrt(2) and b / sqrt(2)
    g1 = [_rne16_pos_sqrt(2 * x * x) for x in a]
    h1 = [_rne16_pos_sqrt(x * x / 2) for x in b]
    assert [Fraction(float(v)) for v in _f16(g[0])] == g1
    assert [Fraction(float(v)) for v in _f16(h[0])] == h1
    assert any(g1[r] * g1[r] > 2 * a[r] * a[r] for r in range(out))      # some round up ...
    assert any(g1[r] * g1[r] < 2 * a[r] * a[r] for r in range(out))      # ... some down
    assert np.array_equal(got[0], np.array(S, dtype=np.int8))

    # plane 2: the signs of S (a b - g h), exact
    R1 = [[S[r][j] * (a[r] * b[j] - g1[r] * h1[j]) for j in range(inf)] for r in range(out)]
    B2 = [[1 if R1[r][j] >= 0 else -1 for j in range(inf)] for r in range(out)]
    flips = sum(B2[r][j] != S[r][j] for r in range(out) for j in range(inf))
    assert 0 < flips < out * inf
    assert np.array_equal(got[1], np.array(B2, dtype=np.int8))
    gd, hd = _decimal_svid([[abs(x) for x in row] for row in R1])
    g2 = [_decimal_rne16(x, 1e-9) for x in gd]
    h2 = [_decimal_rne16(x, 1e-9) for x in hd]
    assert [Fraction(float(v)) for v in _f16(g[1])] == g2
    assert [Fraction(float(v)) for v in _f16(h[1])] == h2

    # plane 3: the exact signs of R_2 = R_1 - B_2 g_2 h_2
    B3 = [[1 if R1[r][j] - B2[r][j] * g2[r] * h2[j] >= 0 else -1 for j in range(inf)] for r in range(out)]
    assert np.array_equal(got[2], np.array(B3, dtype=np.int8))
