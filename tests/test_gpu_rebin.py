"""GPU parity of rbq_rebinarize (the planes for fixed scales; QBB summary,
"Approach": the binary bases refined after the cascade) through the C ABI
against oracle/rebin.py.  Every decision is exact on both sides, so the
planes must be bit-identical."""
import numpy as np
import pytest
import torch

import gemm_rbq_encode_amd as rbq
import oracle
import workloads
from oracle import rebin

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def gpu_rebin(W, planes, scales, group=0):
    Wt = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(dev())
    pt = torch.from_numpy(np.ascontiguousarray(planes, dtype=np.uint32).view(np.int32)).to(dev())
    st = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.uint16).view(np.float16)).to(dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    rbq.rebinarize(Wt, pt, st, group, status=status)
    torch.cuda.synchronize()
    return pt.cpu().numpy().view(np.uint32), int(status.item())


def random_scales(K, out, G, rng):
    return (np.abs(rng.standard_normal((K, out, G))) * 0.03 + 1e-3).astype(np.float16).view(np.uint16)


def assert_rebin_matches(W, planes, scales, group=0, what=""):
    ref, fref = rebin.rebinarize(W, planes, scales, group)
    got, st = gpu_rebin(W, planes, scales, group)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} words differ, first {bad[:4].tolist()}"
    assert st == fref, f"{what}: status {st} vs {fref}"


def test_rebin_small_workload_after_encode():
    wl = workloads.WORKLOADS["small"]
    W = workloads.workload_weight(wl, 0)
    p, s, _ = oracle.encode(W, 2)
    assert_rebin_matches(W, p, s, 0, "small")


@pytest.mark.parametrize("out,inf,K,group", [
    (1, 32, 1, 0), (3, 96, 2, 0), (17, 160, 3, 0), (65, 4224, 4, 0), (40, 16384, 2, 0),
    (5, 128, 4, 128), (300, 640, 2, 128), (1031, 4224, 4, 128), (77, 1152, 3, 128),
    (4100, 256, 2, 0), (9000, 128, 1, 128), (3000, 64, 3, 0), (20000, 128, 2, 0),
    # ragged rows (in % 64 == 32) with more than 4096 segments, so a wave's
    # running word cursor, its 64-word flushes and its loads cross several
    # segments; and the ragged-row kernel with four planes
    (4100, 96, 2, 0), (5000, 160, 4, 0), (33, 4128, 4, 0), (9001, 32, 4, 0), (4500, 224, 3, 0)])
def test_rebin_ragged_shapes_random_scales(out, inf, K, group):
    """Random (not cascade) scales, so every pattern occurs; rows of 32 or
    96 columns end in half chunks; segment counts not a multiple of the
    batch."""
    rng = np.random.default_rng(out * 13 + inf + K + group)
    W = workloads.gaussian_weight(out, inf, seed=out + inf + K, outliers=True)
    G = inf // group if group else 1
    p0 = rng.integers(0, 2 ** 32, (K, out, inf // 32), dtype=np.uint64).astype(np.uint32)
    assert_rebin_matches(W, p0, random_scales(K, out, G, rng), group, f"{out}x{inf} K={K} g{group}")


def special_case(K, group, rng):
    """Weights on midpoints and on values (exact ties), +-0, tiny and
    subnormal weights, +-Inf and NaN; equal, zero and negative scales."""
    out, inf = 8, 512
    G = inf // group if group else 1
    n = group if group else inf
    a = np.abs(rng.standard_normal((K, out, G))) * 0.05 + 0.01
    a[:, 1] = a[0, 1]
    a[-1, 2] = 0.0
    a[0, 3] = -a[0, 3]
    a[:, 5] = 0.0
    scales = a.astype(np.float16).view(np.uint16)
    af = scales.view(np.float16).astype(np.float64)
    P = rebin.patterns(K)
    W = (rng.standard_normal((out, inf)) * 0.05).astype(np.float32)
    for r in range(out):
        for j in range(0, inf, 3):
            u, v = rng.choice(P @ af[:, r, j // n], 2)
            W[r, j] = np.float32((u + v) / 2)
        for j in range(1, inf, 7):
            W[r, j] = np.float32(rng.choice(P @ af[:, r, j // n]))
    W[0, 2], W[0, 4], W[0, 5] = 0.0, -0.0, 1e-30
    W[0, 7], W[0, 8], W[6, 9] = -1e-40, 1e-40, -1e-45
    W[4, 10], W[4, 11], W[4, 13] = np.inf, -np.inf, np.nan
    return W, scales


@pytest.mark.parametrize("K,group", [(1, 0), (2, 0), (3, 0), (4, 0), (2, 128), (4, 128)])
def test_rebin_ties_and_special_values(K, group):
    rng = np.random.default_rng(200 + K + group)
    W, scales = special_case(K, group, rng)
    p0 = np.zeros((K, W.shape[0], W.shape[1] // 32), np.uint32)
    assert_rebin_matches(W, p0, scales, group, f"special K={K} g{group}")


def test_rebin_keeps_planes_of_nonfinite_scales():
    rng = np.random.default_rng(5)
    W = workloads.gaussian_weight(70, 512, seed=35)
    s = random_scales(4, 70, 4, rng)
    s[1, 2, 1] = np.float16(np.inf).view(np.uint16)
    s[0, 69, 3] = np.float16(np.nan).view(np.uint16)
    s[2, 40, 0] = np.float16(-np.inf).view(np.uint16)
    junk = rng.integers(0, 2 ** 32, (4, 70, 16), dtype=np.uint64).astype(np.uint32)
    assert_rebin_matches(W, junk, s, 128, "kept groups")
    got, st = gpu_rebin(W, junk, s, 128)
    assert st == rbq.RBQ_STATUS_PLANES_KEPT
    assert np.array_equal(got[:, 2, 4:8], junk[:, 2, 4:8])


@pytest.mark.parametrize("wl_name,i,K,group", [("llama2_7b", 4, 2, 0), ("llama2_7b", 6, 2, 0),
                                               ("llama2_13b_g128", 4, 4, 128)])
def test_rebin_full_size_sampled_rows(wl_name, i, K, group):
    """Full-size layers (gate 11008 x 4096, down 4096 x 11008, 13B gate
    13824 x 5120 with 128-column groups) in the launch the library makes
    for them; the oracle checks 48 sampled rows (rows are independent)."""
    wl = workloads.WORKLOADS[wl_name]
    W = workloads.workload_weight(wl, i)
    out, inf = W.shape
    G = inf // group if group else 1
    rng = np.random.default_rng(i + K)
    s = random_scales(K, out, G, rng)
    p0 = np.zeros((K, out, inf // 32), np.uint32)
    got, st = gpu_rebin(W, p0, s, group)
    rows = np.unique(np.concatenate([[0, out - 1], rng.integers(0, out, 46)]))
    ref, _ = rebin.rebinarize(W[rows], p0[:, rows], s[:, rows], group)
    assert np.array_equal(got[:, rows], ref)
    assert st == 0


@pytest.mark.parametrize("K,group", [(2, 0), (4, 128), (3, 0)])
def test_rebin_alternation_with_gpu_refit(K, group):
    """encode -> (refit -> rebinarize) x 3 on the GPU: each re-binarization
    equals the oracle's for the GPU's scales, and the objective never rises
    by more than the scales' binary16 rounding allows."""
    W = workloads.gaussian_weight(512, 1024, seed=36 + K, outliers=True)
    Wt = torch.from_numpy(W).to(dev())
    planes, scales = rbq.encode(Wt, K, group)
    torch.cuda.synchronize()
    first = rebin.objective(W, planes.cpu().numpy().view(np.uint32), scales.cpu().numpy().view(np.uint16), group)
    prev = first
    for _ in range(3):
        rbq.refit(Wt, planes, scales, group)
        s_np = scales.cpu().numpy().view(np.uint16)
        p_before = planes.cpu().numpy().view(np.uint32)
        e_refit = rebin.objective(W, p_before, s_np, group)
        assert e_refit <= prev * (1 + 1e-3)
        rbq.rebinarize(Wt, planes, scales, group)
        torch.cuda.synchronize()
        p_np = planes.cpu().numpy().view(np.uint32)
        ref, _ = rebin.rebinarize(W, p_before, s_np, group)
        assert np.array_equal(p_np, ref)
        prev = rebin.objective(W, p_np, s_np, group)
        assert prev <= e_refit * (1 + 1e-12)
    assert prev < first
