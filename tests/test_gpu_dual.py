"""GPU parity of the dual-scale paths, y = sum_k g_k (.) (B_k (h_k (.) x))
(RaBiT summary section 4.1; scales from a residual SVID, section 4.3),
through the C ABI against the fp64 oracle in oracle/dual.py.

Encoder: planes, g and h equal to the oracle's, every plane and every
scale.  Both sum in fp64 but in different orders (agreeing to ~1e-13
relative), so the inputs are checked on the oracle side to keep every scale
more than 1e-11 (relative) away from a binary16 rounding midpoint.  Layer output: relative L2 error <= 1e-3 and max abs error
<= 1e-2 * rms(y_ref).
"""
import numpy as np
import pytest
import torch

import gemm_rbq_encode_amd as rbq
import workloads
from oracle import dual

pytestmark = pytest.mark.gpu
REL_L2 = 1e-3
MAX_ABS_RMS = 1e-2


def dev():
    return torch.device("cuda:0")


def gpu_encode_dual(W, K):
    Wt = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    p, g, h = rbq.encode_dual(Wt, K, status=status)
    torch.cuda.synchronize()
    return (p.cpu().numpy().view(np.uint32), g.cpu().numpy().view(np.uint16),
            h.cpu().numpy().view(np.uint16), int(status.item()))


def min_midpoint_distance(x):
    """Smallest relative distance of the positive entries of fp64 x to a
    binary16 rounding midpoint (inf when there is none)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    x = x[(x > 0) & (x < 65504.0)]
    if x.size == 0:
        return np.inf
    e = np.maximum(np.floor(np.log2(x)), -14.0)
    q = np.exp2(e - 10.0)
    m = (np.floor(x / q) + 0.5) * q
    return float(np.min(np.abs(x - m) / x))


# The GPU sums its fp64 fits in another order than the oracle; the two agree
# to about 1e-13 relative, so a scale can only round differently when its
# value lies that close to a binary16 midpoint.  The inputs used here are
# checked, on the oracle side, to keep every scale at least AMBIGUOUS away
# from one; then every plane and every scale must be equal.
AMBIGUOUS = 1e-11


def assert_dual_encode_matches(W, K, what=""):
    fits = []
    po, go, ho = dual.encode_dual(W, K, fits=fits)
    d = min(min(min_midpoint_distance(gb), min_midpoint_distance(hb)) for gb, hb in fits)
    assert d > AMBIGUOUS, f"{what}: an oracle scale lies {d:.1e} from a binary16 midpoint; pick other data"
    p, g, h, st = gpu_encode_dual(W, K)
    assert st == 0, f"{what}: status {st}"
    for k in range(K):
        assert np.array_equal(p[k], po[k]), f"{what}: plane {k} differs at {np.argwhere(p[k] != po[k])[:5]}"
        assert np.array_equal(g[k], go[k]), f"{what}: g of plane {k} differs at {np.argwhere(g[k] != go[k])[:5]}"
        assert np.array_equal(h[k], ho[k]), f"{what}: h of plane {k} differs at {np.argwhere(h[k] != ho[k])[:5]}"


def assert_close(y, yref, what=""):
    assert np.isfinite(y).all(), what
    rms = np.sqrt(np.mean(yref ** 2))
    rel = np.linalg.norm(y - yref) / max(np.linalg.norm(yref), 1e-300)
    mx = np.abs(y - yref).max() if y.size else 0.0
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e}"
    assert mx <= MAX_ABS_RMS * rms, f"{what}: max-abs {mx:.3e} vs rms {rms:.3e}"


def gpu_gemv_dual(p, g, h, x):
    pt = torch.from_numpy(np.ascontiguousarray(p).view(np.int32)).to(dev())
    gt = torch.from_numpy(np.ascontiguousarray(g).view(np.float16)).to(dev())
    ht = torch.from_numpy(np.ascontiguousarray(h).view(np.float16)).to(dev())
    xt = torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.float16)).to(dev())
    y = rbq.gemv_dual(pt, gt, ht, xt)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------------------
# encoder
# ---------------------------------------------------------------------------

def test_encode_dual_small_workload():
    wl = workloads.WORKLOADS["small"]
    assert_dual_encode_matches(workloads.workload_weight(wl, 0), 2, "small")


@pytest.mark.parametrize("i", [0, 4, 6])
def test_encode_dual_llama2_7b(i):
    wl = workloads.WORKLOADS["llama2_7b"]
    assert_dual_encode_matches(workloads.workload_weight(wl, i), 2, wl.linears[i].name)


@pytest.mark.parametrize("out,inf,K", [(1, 128, 1), (17, 128, 2), (33, 384, 3), (5, 1280, 4),
                                       (300, 640, 8), (40, 16384, 2), (1031, 4224, 2)])
def test_encode_dual_ragged_shapes(out, inf, K):
    W = workloads.gaussian_weight(out, inf, seed=out * 7 + inf + K, outliers=True)
    assert_dual_encode_matches(W, K, f"{out}x{inf} K={K}")


def test_encode_dual_special_values():
    rng = np.random.default_rng(21)
    W = (rng.standard_normal((24, 256)) * 0.02).astype(np.float32)
    W[3] = 0.0                       # a zero row
    W[5, ::3] = -0.0                 # negative zeros count as +1
    W[7] *= 1e-30                    # a tiny row
    assert_dual_encode_matches(W, 3, "special")
    assert_dual_encode_matches(np.zeros((16, 128), np.float32), 2, "zero matrix")


def test_encode_dual_rank1_magnitudes():
    rng = np.random.default_rng(22)
    a = rng.uniform(0.5, 2.0, 48).astype(np.float16).astype(np.float32)
    b = rng.uniform(0.01, 0.1, 512).astype(np.float16).astype(np.float32)
    W = (np.where(rng.random((48, 512)) < 0.5, -1.0, 1.0) * np.outer(a, b)).astype(np.float32)
    assert_dual_encode_matches(W, 2, "rank-1 magnitudes")


def test_encode_dual_flags_nonfinite_w():
    W = workloads.gaussian_weight(8, 256, seed=3)
    W[2, 9] = np.nan
    _, _, _, st = gpu_encode_dual(W, 1)
    assert st & rbq.RBQ_STATUS_NONFINITE_W


def test_encode_dual_flags_scale_overflow():
    """|W| ~ 1e30: the balanced scales (~ sqrt of the fitted products) pass
    65504 and round to infinity in binary16."""
    W = np.where(np.arange(8 * 128).reshape(8, 128) % 3 == 0, -1e30, 1e30).astype(np.float32)
    _, g, h, st = gpu_encode_dual(W, 1)
    assert st & rbq.RBQ_STATUS_SCALE_OVERFLOW and not st & rbq.RBQ_STATUS_NONFINITE_W
    po, go, ho = dual.encode_dual(W, 1)
    assert np.array_equal(g, go) and np.array_equal(h, ho)


def test_encode_dual_deterministic():
    W = workloads.gaussian_weight(512, 1024, seed=5, outliers=True)
    a = gpu_encode_dual(W, 2)
    b = gpu_encode_dual(W, 2)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# ---------------------------------------------------------------------------
# layer output
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("i", [0, 4, 6])
def test_gemv_dual_llama2_7b(i):
    wl = workloads.WORKLOADS["llama2_7b"]
    W = workloads.workload_weight(wl, i)
    p, g, h = dual.encode_dual(W, 2)
    x = workloads.workload_activations(wl, W.shape[1], 1)
    assert_close(gpu_gemv_dual(p, g, h, x), dual.gemm_dual(p, g, h, x)[0], wl.linears[i].name)


@pytest.mark.parametrize("out,inf,K", [(1, 128, 1), (15, 256, 2), (17, 640, 3), (257, 4224, 4),
                                       (1000, 128, 2), (64, 16384, 2), (33, 32768, 1)])
def test_gemv_dual_random_scales(out, inf, K):
    """Random planes, signed g, h of mixed magnitude and sign."""
    rng = np.random.default_rng(out + inf + K)
    p = rng.integers(0, 2 ** 32, (K, out, inf // 32), dtype=np.uint64).astype(np.uint32)
    g = (rng.standard_normal((K, out)) * 0.05).astype(np.float16).view(np.uint16)
    h = (rng.standard_normal((K, inf)) * np.exp(rng.uniform(-3, 3, (K, inf)))).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((1, inf)).astype(np.float16)
    assert_close(gpu_gemv_dual(p, g, h, x), dual.gemm_dual(p, g, h, x)[0], f"{out}x{inf} K={K}")


DUAL_PATHS = {"auto": rbq.PATH_AUTO, "decode": rbq.PATH_DECODE, "flat": rbq.PATH_FLAT}


@pytest.mark.parametrize("path", list(DUAL_PATHS))
@pytest.mark.parametrize("out,inf,K", [(8200, 6144, 2), (8200, 6144, 1), (22016, 4096, 2),
                                       (4100, 11008, 2), (6000, 16384, 2)])
def test_gemv_dual_kernel_families(path, out, inf, K):
    """The flat kernel (tall layers, K <= 2) and the decode kernel, forced
    and chosen, on ragged row counts and the widths each takes."""
    rng = np.random.default_rng(out + 3 * inf + K)
    p = rng.integers(0, 2 ** 32, (K, out, inf // 32), dtype=np.uint64).astype(np.uint32)
    g = (rng.standard_normal((K, out)) * 0.05).astype(np.float16).view(np.uint16)
    h = (rng.standard_normal((K, inf)) * np.exp(rng.uniform(-2, 2, (K, inf)))).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((1, inf)).astype(np.float16)
    old = rbq.set_path(DUAL_PATHS[path])
    try:
        y = gpu_gemv_dual(p, g, h, x)
    finally:
        rbq.set_path(old)
    assert_close(y, dual.gemm_dual(p, g, h, x)[0], f"{path} {out}x{inf} K={K}")


def test_gemv_dual_forced_unsupported_family():
    p = torch.zeros((2, 64, 8), dtype=torch.int32, device=dev())
    g = torch.zeros((2, 64), dtype=torch.float16, device=dev())
    h = torch.zeros((2, 256), dtype=torch.float16, device=dev())
    x = torch.zeros(256, dtype=torch.float16, device=dev())
    old = rbq.set_path(rbq.PATH_VALU)
    try:
        with pytest.raises(rbq.RbqError):
            rbq.gemv_dual(p, g, h, x)
    finally:
        rbq.set_path(old)


def test_gemv_dual_with_unit_input_scales_is_the_row_scale_layer():
    """h = 1: the dual layer is the per-row-scale layer with a_k = g_k."""
    wl = workloads.WORKLOADS["small"]
    W = workloads.workload_weight(wl, 0)
    p, s, _ = __import__("oracle").encode(W, 2)
    h = np.full((2, W.shape[1]), np.float16(1.0)).view(np.uint16)
    x = workloads.workload_activations(wl, W.shape[1], 1)
    y_dual = gpu_gemv_dual(p, s[:, :, 0], h, x)
    assert_close(y_dual, __import__("oracle").gemm(p, s, x)[0], "h = 1")


def test_gemv_dual_zero_input_columns_and_empty():
    y = torch.full((8,), 7.0, dtype=torch.float16, device=dev())
    L = rbq.lib()
    st = L.rbq_gemv_dual(None, None, None, rbq.shape(8, 0, 2), None, y.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == rbq.RBQ_OK and not y.any()
    assert L.rbq_gemv_dual(None, None, None, rbq.shape(0, 128, 2), None, None, None) == rbq.RBQ_OK


def random_dual_layer(K, out, inf, seed):
    """Random planes; g ~ 1/sqrt(K in) and h ~ 1 (both signs) in binary16."""
    rng = np.random.default_rng(seed)
    p = workloads.random_planes(K, out, inf, seed=seed)
    g = (rng.uniform(0.5, 1.5, (K, out)) / np.sqrt(K * inf) * rng.choice([-1.0, 1.0], (K, out))).astype(np.float16)
    h = (rng.uniform(0.25, 2.0, (K, inf)) * rng.choice([-1.0, 1.0], (K, inf))).astype(np.float16)
    return p, g.view(np.uint16), h.view(np.uint16)


def assert_close_dual(y, yref, what):
    y = np.asarray(y, dtype=np.float64)
    assert np.isfinite(y).all(), what
    rms = np.sqrt(np.mean(yref ** 2))
    rel = np.linalg.norm(y - yref) / max(np.linalg.norm(yref), 1e-300)
    mx = np.abs(y - yref).max()
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e}"
    assert mx <= MAX_ABS_RMS * rms, f"{what}: max-abs {mx:.3e} vs rms {rms:.3e}"


@pytest.mark.parametrize("K,out,inf,M", [(2, 256, 512, 2), (2, 300, 640, 5), (1, 64, 96, 3), (3, 17, 384, 16),
                                         (4, 130, 1152, 4), (2, 4096, 4096, 4), (2, 11008, 4096, 2),
                                         (2, 4096, 11008, 16), (2, 512, 1024, 1), (2, 64, 96, 1)])
def test_gemm_dual_matches_oracle(K, out, inf, M):
    """rbq_gemm_dual for M tokens (one token on the matrix-core kernels where
    they take the shape, else and for several tokens the plain kernel)
    against Y = X What^T in fp64; ragged rows, inputs not a multiple of 128,
    K from 1 to 4, and mixed-magnitude tokens."""
    p, g, h = random_dual_layer(K, out, inf, seed=out * 7 + inf + K + M)
    X = workloads.gaussian_activations(M, inf, seed=M * 13 + inf)
    Xv = X.view(np.float16).copy()
    if M >= 3:
        Xv[1] *= np.float16(1e-3)            # a small token beside ordinary ones
        Xv[2, ::7] = np.float16(300.0)       # a token with large entries
    pt = torch.from_numpy(np.ascontiguousarray(p).view(np.int32)).to(dev())
    gt = torch.from_numpy(g.view(np.float16)).to(dev())
    ht = torch.from_numpy(h.view(np.float16)).to(dev())
    Xt = torch.from_numpy(Xv).to(dev())
    Y = rbq.gemm_dual(pt, gt, ht, Xt)
    torch.cuda.synchronize()
    yref = dual.gemm_dual(p, g, h, Xv.view(np.uint16))
    for m in range(M):
        assert_close_dual(Y[m].cpu().numpy(), yref[m], f"token {m}")
    if M == 1:
        # the plain kernel forced for the same call agrees with the same bar
        old = rbq.set_path(rbq.PATH_VALU)
        try:
            Yv = rbq.gemm_dual(pt, gt, ht, Xt)
        finally:
            rbq.set_path(old)
        torch.cuda.synchronize()
        assert_close_dual(Yv[0].cpu().numpy(), yref[0], "plain kernel, one token")


def test_gemm_dual_on_encoded_layer():
    """The dual-scale encoder's output through rbq_gemm_dual for 8 tokens,
    against the oracle's layer output on the same planes and scales."""
    W = workloads.gaussian_weight(512, 1024, 31)
    p, g, h, st = gpu_encode_dual(W, 2)
    assert st == 0
    X = workloads.gaussian_activations(8, 1024, seed=32)
    Y = rbq.gemm_dual(torch.from_numpy(p.view(np.int32)).to(dev()), torch.from_numpy(g.view(np.float16)).to(dev()),
                      torch.from_numpy(h.view(np.float16)).to(dev()), torch.from_numpy(X.view(np.float16)).to(dev()))
    torch.cuda.synchronize()
    yref = dual.gemm_dual(p, g, h, X)
    for m in range(8):
        assert_close_dual(Y[m].cpu().numpy(), yref[m], f"token {m}")
