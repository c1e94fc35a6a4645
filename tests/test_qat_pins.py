"""Pins of oracle/qat.py: the coupled forward (binary cores re-derived from
the shared weight for given scales) and its straight-through backward
(RaBiT summary section 4.2 "Coupled Training", "RaBiT training").

Independent checks only: numpy sign/packbits and the C oracle for one plane,
the exact nearest-value oracle (oracle.rebin, itself pinned by rational brute
force) for scales that dominate their successors, planted planes, the C
oracle's planes when its own scales are given, finite differences of the
linear surrogate for every gradient, and unit-vector closed forms."""
import numpy as np
import pytest

import oracle
from oracle import qat, rebin


def unpack(planes, inf):
    K, out, words = planes.shape
    bits = np.unpackbits(planes.view(np.uint8).reshape(K, out, words * 4), axis=-1, bitorder="little")
    return bits[:, :, :inf].astype(np.int8) * 2 - 1


def exact_weights(out, inf, rng, bound=0.45):
    """fp32 weights on a 2^-24 grid with |W| < bound: with scales on the
    binary16 grid above 2^-14 every residual step below 1 is exact in fp32."""
    W = np.clip(rng.standard_normal((out, inf)) * 0.12, -bound, bound)
    return (np.round(W * 2.0 ** 24) / 2.0 ** 24).astype(np.float32)


def dominant_scales(K, out, G, rng):
    """a_k > sum_{l>k} a_l, binary16: 0.2, 0.09, 0.04, 0.015 times factors in [0.9, 1.1]."""
    base = np.array([0.2, 0.09, 0.04, 0.015])[:K]
    f = rng.uniform(0.9, 1.1, (K, out, G))
    a = (base[:, None, None] * f).astype(np.float16)
    af = a.astype(np.float64)
    for k in range(K - 1):
        assert (af[k] > af[k + 1:].sum(axis=0)).all()
    return a.view(np.uint16)


def test_one_plane_is_sign():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((9, 96)) * 0.02).astype(np.float32)
    W[2, 5] = -0.0
    W[3, 7] = 0.0
    s = np.full((1, 9, 1), np.float16(0.01)).view(np.uint16)
    p = qat.cascade(W, s)
    assert np.array_equal(unpack(p, 96)[0], np.where(W >= 0, 1, -1))
    p_c, _, _ = oracle.encode(W, 1)
    assert np.array_equal(p, p_c)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("group", [0, 128])
def test_dominant_scales_give_the_nearest_values(K, group):
    """With a_k > sum of the later scales the cascade picks, weight by weight,
    the nearest of the 2^K values sum_k +-a_k (ties to the larger), which the
    exact re-binarization oracle decides by rational comparisons."""
    rng = np.random.default_rng(10 + K + group)
    out, inf = 12, 256
    W = exact_weights(out, inf, rng)
    W[0, :8] = 0.0                                  # ties at 0 -> +1
    G = inf // group if group else 1
    s = dominant_scales(K, out, G, rng)
    p = qat.cascade(W, s, group)
    start = rng.integers(0, 2 ** 32, p.shape, dtype=np.uint64).astype(np.uint32)
    ref, flags = rebin.rebinarize(W, start, s, group)
    assert flags == 0
    assert np.array_equal(p, ref)


@pytest.mark.parametrize("K", [1, 2, 4])
def test_planted_planes_are_recovered(K):
    rng = np.random.default_rng(20 + K)
    out, inf = 10, 128
    s = dominant_scales(K, out, 1, rng)
    B = rng.choice([-1.0, 1.0], size=(K, out, inf))
    a = s.view(np.float16).astype(np.float64)
    W = (a * B).sum(axis=0).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), (a * B).sum(axis=0))      # exact
    p = qat.cascade(W, s)
    assert np.array_equal(unpack(p, inf), B.astype(np.int8))


@pytest.mark.parametrize("group", [0, 128])
def test_encoder_scales_reproduce_the_encoder_planes(group):
    """The residual-binarization encoder (C oracle) derives its scales on
    the way; given those scales, the cascade takes the same steps."""
    rng = np.random.default_rng(30 + group)
    W = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    for K in (1, 2, 3):
        p_c, s_c, _ = oracle.encode(W, K, group)
        assert np.array_equal(qat.cascade(W, s_c, group), p_c)


# ---------------------------------------------------------------------------
# straight-through backward
# ---------------------------------------------------------------------------

def _case(out, inf, K, M, group, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((out, inf)) * 0.05).astype(np.float32)
    G = inf // group if group else 1
    s = (rng.uniform(0.005, 0.05, (K, out, G)) * rng.choice([-1, 1], (K, out, G))).astype(np.float16).view(np.uint16)
    X = rng.standard_normal((M, inf)).astype(np.float16)
    dY = rng.standard_normal((M, out)).astype(np.float16)
    return W, s, X, dY


@pytest.mark.parametrize("group", [0, 128])
def test_gradients_match_finite_differences(group):
    """Central differences of the linear surrogate: L(X) = <dY, X What^T>,
    L(a) = <dY, X (sum_k a_k B_k)^T> with the cores fixed, and, through the
    straight-through estimator, L(W) = <dY, X W^T>.  Each is linear, so the
    difference quotient is the gradient up to fp64 rounding; a transposed
    operand, a dropped sign or a wrong group would not match."""
    out, inf, K, M = 6, 256, 2, 3
    W, s, X, dY = _case(out, inf, K, M, group, 40 + group)
    planes, _ = qat.forward(W, s, X, group)
    dX, dW, ds = qat.backward(planes, s, X, dY, group)
    Xf = X.astype(np.float64)
    dYf = dY.astype(np.float64)
    B = unpack(planes, inf).astype(np.float64)
    G = inf // group if group else 1
    n = group if group else inf
    a = s.view(np.float16).astype(np.float64)

    def what_of(av):
        return sum(np.repeat(av[k], n, axis=1) * B[k] for k in range(K))

    def loss(Xv, av, Wsur=None):
        Wm = what_of(av) if Wsur is None else Wsur
        return float((dYf * (Xv @ Wm.T)).sum())

    h = 0.5
    rng = np.random.default_rng(7)
    for _ in range(12):
        m, j = rng.integers(M), rng.integers(inf)
        E = np.zeros_like(Xf)
        E[m, j] = h
        fd = (loss(Xf + E, a) - loss(Xf - E, a)) / (2 * h)
        assert abs(fd - dX[m, j]) <= 1e-9 * max(1.0, abs(fd))
    for _ in range(12):
        k, r, t = rng.integers(K), rng.integers(out), rng.integers(G)
        E = np.zeros_like(a)
        E[k, r, t] = h
        fd = (loss(Xf, a + E) - loss(Xf, a - E)) / (2 * h)
        assert abs(fd - ds[k, r, t]) <= 1e-9 * max(1.0, abs(fd))
    Wf = W.astype(np.float64)
    for _ in range(12):
        r, j = rng.integers(out), rng.integers(inf)
        E = np.zeros_like(Wf)
        E[r, j] = h
        fd = (loss(Xf, a, Wf + E) - loss(Xf, a, Wf - E)) / (2 * h)
        assert abs(fd - dW[r, j]) <= 1e-9 * max(1.0, abs(fd))


def test_gradients_closed_forms():
    """One token, dY = e_r and x = e_j: dW has a single 1 at (r, j), dX is
    row r of What, and the scale gradient of plane k is B_k[r][j] at row r
    and 0 elsewhere."""
    out, inf, K = 5, 64, 2
    W, s, _, _ = _case(out, inf, K, 1, 0, 50)
    planes = qat.cascade(W, s)
    What = qat.dequant(planes, s)
    B = unpack(planes, inf)
    for r, j in [(0, 0), (3, 17), (4, 63)]:
        x = np.zeros((1, inf), np.float16)
        x[0, j] = 1
        dy = np.zeros((1, out), np.float16)
        dy[0, r] = 1
        dX, dW, ds = qat.backward(planes, s, x, dy)
        E = np.zeros((out, inf))
        E[r, j] = 1
        assert np.array_equal(dW, E)
        assert np.array_equal(dX[0], What[r])
        exp = np.zeros((K, out, 1))
        exp[:, r, 0] = B[:, r, j]
        assert np.array_equal(ds, exp)


def test_forward_is_the_layer_of_the_derived_planes():
    W, s, X, _ = _case(7, 128, 2, 4, 0, 60)
    planes, Y = qat.forward(W, s, X)
    assert np.allclose(Y, oracle.gemm(planes, s, X.view(np.uint16)), rtol=1e-12, atol=1e-12)
