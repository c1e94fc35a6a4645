"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Encoder: planes and scales bit-exact.  Layer output: relative L2 error
<= 1e-3 and max abs error <= 1e-2 * rms(y_ref) against the fp64 oracle
(fp32 accumulation, fp16 output), on every workload shape, on edge cases,
and on every kernel family.
"""
import json
import os

import numpy as np
import pytest
import torch

import gemm_rbq_encode_amd as rbq
import oracle
import workloads

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
REL_L2 = 1e-3
MAX_ABS_RMS = 1e-2

# kernel families rbq_gemm can be forced to, with the largest M each takes
PATHS = {"valu": (rbq.PATH_VALU, 1 << 30), "decode": (rbq.PATH_DECODE, 64),
         "stream": (rbq.PATH_STREAM, 2), "flat": (rbq.PATH_FLAT, 16),
         "group": (rbq.PATH_GROUP, 1), "split": (rbq.PATH_SPLIT, 16),
         "prefill": (rbq.PATH_PREFILL, 1 << 30)}


def dev():
    return torch.device("cuda:0")


def gpu_encode(W, K, group, force_serial=False):
    Wt = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    planes, scales = rbq.encode(Wt, K, group, status=status, force_serial=force_serial)
    torch.cuda.synchronize()
    return (planes.cpu().numpy().view(np.uint32), scales.cpu().numpy().view(np.uint16),
            int(status.item()))


def gpu_gemm(planes, scales, X, group, path=rbq.PATH_AUTO):
    p = torch.from_numpy(np.ascontiguousarray(planes).view(np.int32)).to(dev())
    s = torch.from_numpy(np.ascontiguousarray(scales).view(np.float16)).to(dev())
    x = torch.from_numpy(np.ascontiguousarray(X).view(np.float16)).to(dev())
    old = rbq.set_path(path)
    try:
        Y = rbq.gemm(p, s, x, group)
        torch.cuda.synchronize()
    except rbq.RbqError as e:
        if e.status == rbq.RBQ_ERR_UNSUPPORTED and path != rbq.PATH_AUTO:
            pytest.skip("this kernel family does not take the shape")
        raise
    finally:
        rbq.set_path(old)
    return Y.cpu().numpy().astype(np.float64)


def assert_close(Y, Yref, what=""):
    assert Y.shape == Yref.shape
    assert np.isfinite(Y).all(), what
    rms = np.sqrt(np.mean(Yref ** 2))
    rel = np.linalg.norm(Y - Yref) / max(np.linalg.norm(Yref), 1e-300)
    mx = np.abs(Y - Yref).max() if Y.size else 0.0
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e}"
    assert mx <= MAX_ABS_RMS * rms, f"{what}: max-abs {mx:.3e} vs rms {rms:.3e}"
    return rel


def assert_encode_matches(W, K, group, force_serial=False, what=""):
    p, s, f = oracle.encode(W, K, group)
    gp, gs, gf = gpu_encode(W, K, group, force_serial)
    assert gf == f, f"{what}: status {gf} vs {f}"
    assert np.array_equal(gs, s), f"{what}: scales differ at {np.argwhere(gs != s)[:5]}"
    assert np.array_equal(gp, p), f"{what}: planes differ at {np.argwhere(gp != p)[:5]}"
    return p, s


# ---------------------------------------------------------------------------
# encoder
# ---------------------------------------------------------------------------

def test_encode_small_workload():
    wl = workloads.WORKLOADS["small"]
    assert_encode_matches(workloads.workload_weight(wl, 0), wl.num_planes, wl.group_size, what="small")


@pytest.mark.parametrize("i", range(7))
def test_encode_llama2_7b(i):
    wl = workloads.WORKLOADS["llama2_7b"]
    W = workloads.workload_weight(wl, i)
    assert_encode_matches(W, wl.num_planes, wl.group_size, what=wl.linears[i].name)


@pytest.mark.parametrize("i", [0, 4, 6])
def test_encode_llama2_13b_g128(i):
    wl = workloads.WORKLOADS["llama2_13b_g128"]
    W = workloads.workload_weight(wl, i)
    assert_encode_matches(W, wl.num_planes, wl.group_size, what=wl.linears[i].name)


@pytest.mark.parametrize("i", [0, 1])
def test_encode_llama3_8b_prefill_shapes(i):
    wl = workloads.WORKLOADS["llama3_8b_prefill"]
    assert_encode_matches(workloads.workload_weight(wl, i), wl.num_planes, wl.group_size)


def test_encode_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_k3.json")))
    W = np.array([[float(v) for v in row] for row in g["W"]], dtype=np.float32)
    assert_encode_matches(W, g["num_planes"], g["group_size"], what="golden")


@pytest.mark.parametrize("out,inf,K,group", [
    (1, 32, 1, 0), (3, 96, 2, 0), (5, 160, 3, 0), (7, 4128, 2, 0), (2, 4160, 8, 0),
    (9, 16384, 2, 0), (4, 32768, 2, 0), (3, 128, 4, 128), (6, 384, 4, 128),
    (5, 8320, 4, 128), (2, 32768, 3, 128), (17, 1024, 8, 0), (33, 640, 5, 128)])
def test_encode_ragged_shapes(out, inf, K, group):
    W = workloads.gaussian_weight(out, inf, seed=out * 1000 + inf + K, outliers=True)
    assert_encode_matches(W, K, group, what=f"{out}x{inf} K={K} g={group}")


def test_encode_special_values():
    rng = np.random.default_rng(5)
    rows = []
    rows.append(np.zeros(256, np.float32))                               # all +0
    rows.append(np.full(256, -0.0, np.float32))                          # all -0
    z = rng.standard_normal(256).astype(np.float32)
    z[rng.random(256) < 0.3] = -0.0
    rows.append(z)
    rows.append((rng.standard_normal(256) * 1e-40).astype(np.float32))   # fp32 denormals
    rows.append(np.full(256, 1e-7, np.float32))                          # fp16-subnormal scale
    rows.append(np.where(rng.random(256) < 0.5, 0.25, -0.25).astype(np.float32))
    rows.append((rng.standard_normal(256) * 3e3).astype(np.float32))     # large scales
    W = np.stack(rows)
    for K, group in ((4, 0), (4, 128), (8, 0)):
        assert_encode_matches(W, K, group, what=f"special K={K} g={group}")


def test_encode_ties_take_the_serial_path():
    """Rows whose mean is exactly an fp16 midpoint cannot be decided by the
    parallel sum's error bound, so the serial path decides them."""
    rows = []
    for base in (1.0, 0.5, 2.0 ** -14, 3.0):
        v = np.float32(base * (1 + 2.0 ** -11))           # midpoint between two fp16 values
        rows.append(np.full(512, v, np.float32) * np.where(np.arange(512) % 3 == 0, -1, 1))
    row = np.full(512, 1 + 2.0 ** -11, np.float64)        # one ulp-of-fp64 above the midpoint
    row[510] = 2 + 2.0 ** -10
    row[511] = 2.0 ** -25
    row[509] = 1 + 2.0 ** -11 + 2.0 ** -23
    rows.append(row.astype(np.float32))
    W = np.stack(rows).astype(np.float32)
    for group in (0, 128):
        assert_encode_matches(W, 3, group, what=f"ties g={group}")


def _near_midpoint_rows():
    """Rows of 512 columns (four 128-column groups) whose group means sit 0,
    1, 2, 4, 16 and 64 fp32 ulps from an fp16 rounding boundary, at several
    magnitudes (normal and subnormal fp16 scales), with mixed signs."""
    rows = []
    signs = np.where(np.arange(128) % 5 < 2, -1.0, 1.0).astype(np.float32)
    for base in (1.0, 0.375, 2.0 ** -14, 3.0 * 2.0 ** -22, 700.0):
        h = np.float16(base)
        mid = (float(h) + float(np.nextafter(h, np.float16(np.inf)))) / 2     # exact in fp32
        groups = []
        for ulps in (0, 1, -1, 2, -2, 4, -4, 16, -16, 64):
            v = np.float32(mid)
            step = np.float32(np.inf if ulps > 0 else -np.inf)
            for _ in range(abs(ulps)):
                v = np.nextafter(v, step)
            groups.append(np.full(128, v, np.float32) * signs)
        # an exact midpoint mean from unequal values, and one a hair above it
        lo = np.float32(mid * (1 - 2.0 ** -12))
        hi = np.float32(2 * mid - float(lo))
        g = np.where(np.arange(128) % 2 == 0, lo, hi).astype(np.float32)
        groups.append(g * signs)
        g2 = g.copy()
        g2[7] = np.nextafter(g2[7], np.float32(np.inf))
        groups.append(g2 * signs)
        rows.extend(np.concatenate(groups[i:i + 4]) for i in range(0, len(groups), 4))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("group", [0, 128])
def test_encode_means_near_fp16_midpoints(group):
    """Means within a few fp32 ulps of an fp16 midpoint cannot be decided by
    an fp32 sum; the encoder must still return the serial fp64 result."""
    assert_encode_matches(_near_midpoint_rows(), 3, group, what=f"near midpoints g={group}")


@pytest.mark.parametrize("out,inf,K,group", [(64, 512, 3, 0), (32, 4096, 2, 0), (16, 1024, 4, 128),
                                             (8, 11008, 2, 0)])
def test_encode_forced_serial_path(out, inf, K, group):
    W = workloads.gaussian_weight(out, inf, seed=77 + inf, outliers=True)
    assert_encode_matches(W, K, group, force_serial=True, what="serial")


def test_encode_status_flags():
    W = workloads.gaussian_weight(4, 256, seed=1)
    W[2, 17] = np.inf
    _, _, f = gpu_encode(W, 2, 0)
    assert f & rbq.RBQ_STATUS_NONFINITE_W
    Wb = np.full((2, 256), 7.0e4, np.float32)
    _, _, f = gpu_encode(Wb, 1, 128)
    assert f & rbq.RBQ_STATUS_SCALE_OVERFLOW and not f & rbq.RBQ_STATUS_NONFINITE_W


def test_encode_deterministic_and_stream_ordered():
    W = workloads.gaussian_weight(512, 4096, seed=9, outliers=True)
    Wt = torch.from_numpy(W).to(dev())
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        p1, s1 = rbq.encode(Wt, 3, 0)
        p2, s2 = rbq.encode(Wt, 3, 0)
    side.synchronize()
    assert torch.equal(p1, p2) and torch.equal(s1, s2)


# ---------------------------------------------------------------------------
# layer output
# ---------------------------------------------------------------------------

def _encoded(wl_name, i):
    wl = workloads.WORKLOADS[wl_name]
    W = workloads.workload_weight(wl, i)
    p, s, _ = oracle.encode(W, wl.num_planes, wl.group_size)
    return wl, p, s


@pytest.mark.parametrize("path", list(PATHS))
def test_gemv_small_workload(path):
    wl, p, s = _encoded("small", 0)
    X = workloads.workload_activations(wl, 512, 1)
    Y = gpu_gemm(p, s, X, wl.group_size, PATHS[path][0])
    assert_close(Y, oracle.gemm(p, s, X, wl.group_size), "small")


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("i", [0, 4, 6])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm_llama2_7b(path, i, M):
    if M > PATHS[path][1]:
        pytest.skip("path does not take this M")
    wl, p, s = _encoded("llama2_7b", i)
    X = workloads.workload_activations(workloads.WORKLOADS["llama2_7b_skinny"] if M > 1 else wl,
                                       wl.linears[i].in_features, M)
    Y = gpu_gemm(p, s, X, wl.group_size, PATHS[path][0])
    assert_close(Y, oracle.gemm(p, s, X, wl.group_size), f"{wl.linears[i].name} M={M}")


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("i", [0, 4, 6])
def test_gemv_llama2_13b_g128(path, i):
    wl, p, s = _encoded("llama2_13b_g128", i)
    X = workloads.workload_activations(wl, wl.linears[i].in_features, 1)
    Y = gpu_gemm(p, s, X, wl.group_size, PATHS[path][0])
    assert_close(Y, oracle.gemm(p, s, X, wl.group_size), wl.linears[i].name)


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("i", [0, 1])
def test_gemm_prefill_all_tokens(path, i):
    """M = 2048 at full size, every output: the oracle's fp64 What
    (oracle.dequant) times X in fp64 (a library matmul as the product step)."""
    if PATHS[path][1] < 2048:
        pytest.skip("path does not take M = 2048")
    wl, p, s = _encoded("llama3_8b_prefill", i)
    X = workloads.workload_activations(wl, wl.linears[i].in_features, 2048)
    Y = gpu_gemm(p, s, X, wl.group_size, PATHS[path][0])
    Xf = X.view(np.float16).astype(np.float64)
    Yref = Xf @ oracle.dequant(p, s, wl.group_size).T
    assert_close(Y, Yref, f"prefill {i}")
    # and every 128-token tile on its own (a tile mapped to the wrong rows
    # would also show in the whole, but not as clearly)
    for t0 in range(0, 2048, 128):
        assert_close(Y[t0:t0 + 128], Yref[t0:t0 + 128], f"prefill {i} tokens {t0}..{t0 + 127}")


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("out,inf,K,group,M", [
    (1, 32, 1, 0, 1), (3, 96, 2, 0, 2), (17, 4128, 3, 0, 5), (40, 384, 4, 128, 3),
    (65, 1024, 8, 0, 16), (129, 11008, 2, 0, 7), (31, 5120, 4, 128, 17), (70, 2048, 2, 0, 33),
    (1, 512, 1, 128, 1), (40, 1536, 4, 128, 1), (33, 5120, 3, 128, 1), (4100, 2048, 2, 128, 1),
    (17, 16384, 4, 128, 1)])
def test_gemm_ragged_random_signed_scales(path, out, inf, K, group, M):
    if M > PATHS[path][1]:
        pytest.skip("path does not take this M")
    p = workloads.random_planes(K, out, inf, seed=out + inf)
    G = inf // group if group else 1
    s = workloads.random_scales(K, out, G, seed=M + K, signed=True)
    X = workloads.gaussian_activations(M, inf, seed=inf + M)
    Y = gpu_gemm(p, s, X, group, PATHS[path][0])
    assert_close(Y, oracle.gemm(p, s, X, group), f"{out}x{inf} K={K} g={group} M={M}")


@pytest.mark.parametrize("out,inf,K,group,M", [
    (300, 1024, 1, 0, 200), (520, 2048, 2, 128, 300), (257, 640, 2, 0, 129),
    (2304, 1024, 2, 0, 300), (1000, 4096, 1, 128, 257), (64, 8192, 2, 128, 2048)])
def test_gemm_prefill_tiles_ragged(out, inf, K, group, M):
    """Several 128-token and 256-row tiles with ragged last tiles, one and two
    planes, per-row and per-128-column scales (signed)."""
    p = workloads.random_planes(K, out, inf, seed=out + 7 * inf)
    G = inf // group if group else 1
    s = workloads.random_scales(K, out, G, seed=M + 3 * K, signed=True)
    X = workloads.gaussian_activations(M, inf, seed=inf + 5 * M)
    Y = gpu_gemm(p, s, X, group, rbq.PATH_PREFILL)
    assert_close(Y, oracle.gemm(p, s, X, group), f"{out}x{inf} K={K} g={group} M={M}")


@pytest.mark.parametrize("path", list(PATHS))
def test_gemm_closed_forms(path):
    K, out, inf, group = 2, 96, 4096, 0
    p = workloads.random_planes(K, out, inf, seed=3)
    s = workloads.random_scales(K, out, 1, seed=4)
    ones = np.full((1, inf), 0x3C00, np.uint16)
    A = s.view(np.float16).astype(np.float64)[:, :, 0]
    pc = np.unpackbits(p.view(np.uint8), bitorder="little").reshape(K, out, inf).sum(-1).astype(np.int64)
    ref = (A * (2 * pc - inf)).sum(axis=0)
    assert_close(gpu_gemm(p, s, ones, group, PATHS[path][0])[0], ref, "x=1")
    E = np.zeros((3, inf), np.uint16)
    for m, j in enumerate((0, 33, inf - 1)):
        E[m, j] = 0x3C00
    Y = gpu_gemm(p, s, E, group, PATHS[path][0])
    What = oracle.dequant(p, s, group)
    for m, j in enumerate((0, 33, inf - 1)):
        assert np.array_equal(Y[m], What[:, j].astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("path", list(PATHS))
def test_gemv_g128_closed_forms(path):
    """x = 1 gives sum_k sum_t a_k,t (2 popcount - 128); a unit vector e_j
    gives column j of the dequantised matrix, rounded once to fp16."""
    K, out, inf, group = 4, 48, 2048, 128
    p = workloads.random_planes(K, out, inf, seed=13)
    s = workloads.random_scales(K, out, inf // group, seed=14, signed=True)
    ones = np.full((1, inf), 0x3C00, np.uint16)
    A = s.view(np.float16).astype(np.float64)
    bits = np.unpackbits(p.view(np.uint8), bitorder="little").reshape(K, out, inf // group, group)
    ref = (A * (2 * bits.sum(-1).astype(np.int64) - group)).sum(axis=(0, 2))
    assert_close(gpu_gemm(p, s, ones, group, PATHS[path][0])[0], ref, "x=1")
    What = oracle.dequant(p, s, group)
    for j in (0, 127, 128, 1000, inf - 1):
        e = np.zeros((1, inf), np.uint16)
        e[0, j] = 0x3C00
        Y = gpu_gemm(p, s, e, group, PATHS[path][0])
        assert np.array_equal(Y[0], What[:, j].astype(np.float16).astype(np.float64)), j


def test_group_path_needs_aligned_scales():
    """Scales 2 bytes off an 8-byte boundary: the automatic choice falls back
    to another kernel with the same result; the forced group kernel refuses."""
    K, out, inf, group = 2, 64, 1024, 128
    p = workloads.random_planes(K, out, inf, seed=21)
    s = workloads.random_scales(K, out, inf // group, seed=22)
    X = workloads.gaussian_activations(1, inf, seed=23)
    pt = torch.from_numpy(p.view(np.int32)).to(dev())
    buf = torch.zeros(s.size + 1, dtype=torch.float16, device=dev())
    buf[1:] = torch.from_numpy(s.reshape(-1).view(np.float16)).to(dev())
    st = buf[1:].view(s.shape)
    assert st.data_ptr() % 8 != 0
    x = torch.from_numpy(X.view(np.float16)).to(dev())
    Y = rbq.gemm(pt, st, x, group).cpu().numpy().astype(np.float64)
    assert_close(Y, oracle.gemm(p, s, X, group), "misaligned scales")
    old = rbq.set_path(rbq.PATH_GROUP)
    try:
        with pytest.raises(rbq.RbqError) as ei:
            rbq.gemm(pt, st, x, group)
        assert ei.value.status == rbq.RBQ_ERR_ALIGNMENT
    finally:
        rbq.set_path(old)


def test_gemm_empty_inputs():
    p = torch.zeros((2, 8, 0), dtype=torch.int32, device=dev())
    s = torch.zeros((2, 8, 0), dtype=torch.float16, device=dev())
    X = torch.zeros((3, 0), dtype=torch.float16, device=dev())
    Y = torch.full((3, 8), 7.0, dtype=torch.float16, device=dev())
    rbq.gemm(p, s, X, 0, Y=Y)
    torch.cuda.synchronize()
    assert (Y == 0).all()
    p2 = torch.zeros((2, 8, 4), dtype=torch.int32, device=dev())
    s2 = torch.zeros((2, 8, 1), dtype=torch.float16, device=dev())
    X0 = torch.zeros((0, 128), dtype=torch.float16, device=dev())
    assert rbq.gemm(p2, s2, X0, 0).shape == (0, 8)


def test_gemm_deterministic_on_side_stream():
    wl, p, s = _encoded("llama2_7b", 4)
    X = workloads.workload_activations(wl, 4096, 1)
    pt = torch.from_numpy(p.view(np.int32)).to(dev())
    st = torch.from_numpy(s.view(np.float16)).to(dev())
    xt = torch.from_numpy(X.view(np.float16)).to(dev())
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y1 = rbq.gemm(pt, st, xt)
        y2 = rbq.gemm(pt, st, xt)
    side.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("split", [1, 2, 4])
@pytest.mark.parametrize("i,M", [(0, 1), (4, 1), (6, 1), (6, 2)])
def test_stream_splits_agree(split, i, M):
    """Every waves-per-tile setting of the streaming kernel meets the bar."""
    wl, p, s = _encoded("llama2_7b", i)
    X = workloads.workload_activations(workloads.WORKLOADS["llama2_7b_skinny"],
                                       wl.linears[i].in_features, M)
    old = rbq.set_stream_split(split)
    try:
        Y = gpu_gemm(p, s, X, wl.group_size, rbq.PATH_STREAM)
    finally:
        rbq.set_stream_split(old)
    assert_close(Y, oracle.gemm(p, s, X, wl.group_size), f"split {split}")


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("idx", [(0, 1, 2), (4, 5)])
def test_gemv_fused_llama2_7b(path, idx):
    """The stacked q/k/v (12288x4096) and gate/up (22016x4096) matrices."""
    wl = workloads.WORKLOADS["llama2_7b"]
    W = np.concatenate([workloads.workload_weight(wl, i) for i in idx])
    p, s = assert_encode_matches(W, wl.num_planes, wl.group_size, what=f"fused {idx}")
    X = workloads.workload_activations(wl, 4096, 1)
    Y = gpu_gemm(p, s, X, wl.group_size, PATHS[path][0])
    assert_close(Y, oracle.gemm(p, s, X, wl.group_size), f"fused {idx}")


def test_graph_replays_match_eager():
    """The calls bench.py captures -- encodes and GEMMs on every kernel family
    the automatic choice takes -- captured in one HIP graph: each of several
    replays, with eager work and synchronisations between them, reproduces the
    eager results bit for bit (the kernels are deterministic, and no call
    records a memset)."""
    cases = [(12288, 4096, 2, 0, 1), (4096, 4096, 2, 0, 1), (4096, 11008, 2, 0, 4),
             (1024, 5120, 4, 128, 1), (512, 1024, 2, 0, 40)]
    W = [torch.from_numpy(workloads.gaussian_weight(o, i, seed=o + i, outliers=True)).to(dev())
         for o, i, _, _, _ in cases]
    X = [torch.from_numpy(workloads.gaussian_activations(m, i, seed=m + i).view(np.float16)).to(dev())
         for _, i, _, _, m in cases]
    enc = [rbq.encode(w, K, g) for w, (_, _, K, g, _) in zip(W, cases)]
    Y = [rbq.gemm(p, s, x, g) for (p, s), x, (_, _, _, g, _) in zip(enc, X, cases)]
    torch.cuda.synchronize()
    ref_p = [p.clone() for p, _ in enc]
    ref_s = [s.clone() for _, s in enc]
    ref_y = [y.clone() for y in Y]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for w, (p, s), x, y, (_, _, K, g, _) in zip(W, enc, X, Y, cases):
            rbq.encode(w, K, g, planes=p, scales=s)
            rbq.gemm(p, s, x, g, Y=y)
    for rep in range(3):
        for p, s, y in zip(*zip(*enc), Y):
            p.zero_()
            s.zero_()
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j in range(len(cases)):
            assert torch.equal(enc[j][0], ref_p[j]), (rep, j, "planes")
            assert torch.equal(enc[j][1], ref_s[j]), (rep, j, "scales")
            assert torch.equal(Y[j], ref_y[j]), (rep, j, "y")
        _ = rbq.gemm(enc[0][0], enc[0][1], X[0], 0)   # eager work between replays


def test_split_workspace_any_contents():
    """The workspace needs no initialisation: filled with 0x00, 0xFF or
    0xA5, then reused by calls of other shapes (other slice and row-group
    counts), it gives the oracle's result every time."""
    cases = [(2, 700, 4096, 16), (1, 300, 9216, 9), (2, 2000, 1536, 4), (2, 700, 4096, 16)]
    L = rbq.lib()
    need = max(L.rbq_gemm_workspace_bytes(rbq.shape(o, i, K, 0), M) for K, o, i, M in cases)
    assert need > 0
    old = rbq.set_path(rbq.PATH_SPLIT)
    try:
        for fill in (0x00, 0xFF, 0xA5):
            ws = torch.full((need,), fill, dtype=torch.uint8, device=dev())
            for K, out, inf, M in cases:
                p = workloads.random_planes(K, out, inf, seed=out + inf + fill)
                s = workloads.random_scales(K, out, 1, seed=M + fill, signed=True)
                X = workloads.gaussian_activations(M, inf, seed=inf + M + fill)
                pt = torch.from_numpy(p.view(np.int32)).to(dev())
                st = torch.from_numpy(s.view(np.float16)).to(dev())
                xt = torch.from_numpy(X.view(np.float16)).to(dev())
                Y = rbq.gemm(pt, st, xt, 0, workspace=ws)
                torch.cuda.synchronize()
                assert_close(Y.cpu().numpy().astype(np.float64), oracle.gemm(p, s, X, 0),
                             f"fill {fill:#x} {out}x{inf} K={K} M={M}")
    finally:
        rbq.set_path(old)


def test_split_path_workspace_contract():
    """A layer split into several column slices needs a workspace: without
    one the automatic choice takes a family that needs none (same result)
    and the forced split family refuses.  A layer of one slice (in <= 4096)
    needs none, and the forced split family runs without it."""
    K, out, inf, M = 2, 256, 4096, 8
    L = rbq.lib()
    assert L.rbq_gemm_workspace_bytes(rbq.shape(out, inf, K, 0), M) == 0
    p = workloads.random_planes(K, out, inf, seed=34)
    s = workloads.random_scales(K, out, 1, seed=35)
    X = workloads.gaussian_activations(M, inf, seed=36)
    assert_close(gpu_gemm(p, s, X, 0, rbq.PATH_SPLIT), oracle.gemm(p, s, X, 0), "one slice")
    K, out, inf, M = 2, 256, 11008, 8
    p = workloads.random_planes(K, out, inf, seed=31)
    s = workloads.random_scales(K, out, 1, seed=32)
    X = workloads.gaussian_activations(M, inf, seed=33)
    L = rbq.lib()
    shp = rbq.shape(out, inf, K, 0)
    assert L.rbq_gemm_workspace_bytes(shp, M) > 0
    assert L.rbq_gemm_workspace_bytes(shp, 1) == 0
    pt = torch.from_numpy(p.view(np.int32)).to(dev())
    st = torch.from_numpy(s.view(np.float16)).to(dev())
    xt = torch.from_numpy(X.view(np.float16)).to(dev())
    Y = torch.empty((M, out), dtype=torch.float16, device=dev())
    stream = torch.cuda.current_stream().cuda_stream
    rc = L.rbq_gemm(pt.data_ptr(), st.data_ptr(), shp, xt.data_ptr(), M, Y.data_ptr(), None, 0, stream)
    assert rc == rbq.RBQ_OK
    torch.cuda.synchronize()
    assert_close(Y.cpu().numpy().astype(np.float64), oracle.gemm(p, s, X, 0), "no workspace")
    old = rbq.set_path(rbq.PATH_SPLIT)
    try:
        rc = L.rbq_gemm(pt.data_ptr(), st.data_ptr(), shp, xt.data_ptr(), M, Y.data_ptr(), None, 0, stream)
        assert rc == rbq.RBQ_ERR_INVALID_ARG
    finally:
        rbq.set_path(old)


# ---------------------------------------------------------------------------
# refit: joint least-squares scales for fixed planes
# ---------------------------------------------------------------------------

def gpu_refit(W, planes, scales, group):
    Wt = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(dev())
    p = torch.from_numpy(np.ascontiguousarray(planes).view(np.int32)).to(dev())
    s = torch.from_numpy(np.ascontiguousarray(scales).view(np.float16)).to(dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    rbq.refit(Wt, p, s, group, status=status)
    torch.cuda.synchronize()
    return s.cpu().numpy().view(np.uint16), int(status.item())


def assert_refit_close(got, want, what):
    """Equal binary16, or one unit apart (the fp64 sums of b are added in
    another order, which can move a value across a rounding midpoint); such
    differences stay rare."""
    g = got.view(np.float16).astype(np.float64)
    w = want.view(np.float16).astype(np.float64)
    unit = np.spacing(np.maximum(np.abs(g), np.abs(w)).astype(np.float16)).astype(np.float64)
    bad = np.abs(g - w) > unit
    assert not bad.any(), (what, np.argwhere(bad)[:5], g[bad][:5], w[bad][:5])
    assert (got != want).mean() <= 1e-3, (what, (got != want).mean())


@pytest.mark.parametrize("name,i", [("small", 0), ("llama2_7b", 0), ("llama2_7b", 4), ("llama2_7b", 6),
                                    ("llama2_13b_g128", 0), ("llama2_13b_g128", 4)])
def test_refit_matches_oracle_on_workloads(name, i):
    wl = workloads.WORKLOADS[name]
    W = workloads.workload_weight(wl, i)
    planes, scales, _ = oracle.encode(W, wl.num_planes, wl.group_size)
    want, wflags = oracle.refit(W, planes, scales, wl.group_size)
    got, gflags = gpu_refit(W, planes, scales, wl.group_size)
    assert gflags == wflags
    assert_refit_close(got, want, f"{name} {i}")


@pytest.mark.parametrize("out,inf,K,group", [(3, 96, 2, 0), (17, 640, 3, 128), (33, 4128, 8, 0),
                                             (9, 1024, 1, 128), (70, 2048, 4, 0), (5, 32768, 2, 0)])
def test_refit_ragged_shapes(out, inf, K, group):
    W = workloads.gaussian_weight(out, inf, seed=out * 7 + inf, outliers=True)
    planes, scales, _ = oracle.encode(W, K, group)
    want, wflags = oracle.refit(W, planes, scales, group)
    got, gflags = gpu_refit(W, planes, scales, group)
    assert gflags == wflags
    assert_refit_close(got, want, f"{out}x{inf} K={K} g={group}")


def test_refit_keeps_singular_and_nonfinite_groups():
    W = workloads.gaussian_weight(6, 512, seed=11)
    W[1] = 0.0
    W[4, 100] = np.nan
    for group in (0, 128):
        planes, scales, _ = oracle.encode(W, 2, group)
        marker = np.full_like(scales, 0x1234)
        want, wflags = oracle.refit(W, planes, marker, group)
        got, gflags = gpu_refit(W, planes, marker, group)
        assert gflags == wflags == rbq.RBQ_STATUS_NONFINITE_W | rbq.RBQ_STATUS_REFIT_KEPT
        assert np.array_equal(got == 0x1234, want == 0x1234)
        assert_refit_close(got, want, f"kept g={group}")


def test_refit_one_plane_is_the_encoder_scale_and_deterministic():
    """K = 1: the least-squares scale is the encoder's mean |W| (within one
    binary16 unit: the refit's sum is parallel).  Two runs agree bit for bit."""
    W = workloads.gaussian_weight(300, 4096, seed=12, outliers=True)
    gp, gs, _ = gpu_encode(W, 1, 0)
    got1, f1 = gpu_refit(W, gp, np.zeros_like(gs), 0)
    got2, f2 = gpu_refit(W, gp, np.zeros_like(gs), 0)
    assert f1 == f2 == 0 and np.array_equal(got1, got2)
    assert_refit_close(got1, gs, "K=1")


# ---------------------------------------------------------------------------
# gated-MLP epilogue: silu(gate) * up from interleaved (gate, up) rows
# ---------------------------------------------------------------------------

def _interleaved_gate_up():
    wl = workloads.WORKLOADS["llama2_7b"]
    gate, up = workloads.workload_weight(wl, 4), workloads.workload_weight(wl, 5)
    W = np.empty((2 * gate.shape[0], gate.shape[1]), dtype=np.float32)
    W[0::2], W[1::2] = gate, up
    p, s, _ = oracle.encode(W, 2, 0)
    return p, s


_GU = {}


def gpu_gemm_epi(planes, scales, X, path):
    p = torch.from_numpy(np.ascontiguousarray(planes).view(np.int32)).to(dev())
    s = torch.from_numpy(np.ascontiguousarray(scales).view(np.float16)).to(dev())
    x = torch.from_numpy(np.ascontiguousarray(X).view(np.float16)).to(dev())
    old = rbq.set_path(path)
    try:
        Y = rbq.gemm(p, s, x, 0, epilogue=rbq.RBQ_EPILOGUE_SILU_MUL)
        torch.cuda.synchronize()
    finally:
        rbq.set_path(old)
    return Y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("path", ["auto", "flat", "valu"])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm_silu_mul_llama2_7b_gate_up(path, M):
    if "p" not in _GU:
        _GU["p"], _GU["s"] = _interleaved_gate_up()
    p, s = _GU["p"], _GU["s"]
    X = workloads.gaussian_activations(M, 4096, seed=40 + M)
    pid = {"auto": rbq.PATH_AUTO, "flat": rbq.PATH_FLAT, "valu": rbq.PATH_VALU}[path]
    H = gpu_gemm_epi(p, s, X, pid)
    assert H.shape == (M, 11008)
    assert_close(H, oracle.silu_mul(oracle.gemm(p, s, X, 0)), f"silu-mul {path} M={M}")


@pytest.mark.parametrize("path", ["flat", "valu"])
@pytest.mark.parametrize("out,inf,K,M", [(34, 512, 1, 3), (2, 128, 2, 1), (66, 11008, 2, 16), (4098, 2048, 2, 2)])
def test_gemm_silu_mul_ragged(path, out, inf, K, M):
    p = workloads.random_planes(K, out, inf, seed=out + inf)
    s = workloads.random_scales(K, out, 1, seed=M + K, signed=True)
    X = workloads.gaussian_activations(M, inf, seed=inf + M)
    pid = {"flat": rbq.PATH_FLAT, "valu": rbq.PATH_VALU}[path]
    H = gpu_gemm_epi(p, s, X, pid)
    assert_close(H, oracle.silu_mul(oracle.gemm(p, s, X, 0)), f"silu-mul {out}x{inf} K={K} M={M}")


def test_gemm_epilogue_errors():
    L = rbq.lib()
    p = torch.zeros((2, 6, 4), dtype=torch.int32, device=dev())
    s = torch.zeros((2, 6, 1), dtype=torch.float16, device=dev())
    x = torch.zeros((1, 128), dtype=torch.float16, device=dev())
    y = torch.zeros((1, 6), dtype=torch.float16, device=dev())
    st = torch.cuda.current_stream().cuda_stream
    args = (p.data_ptr(), s.data_ptr(), rbq.shape(6, 128, 2, 0), x.data_ptr(), 1, y.data_ptr(), None, 0)
    assert L.rbq_gemm_ex(*args, 7, st) == rbq.RBQ_ERR_INVALID_ARG
    odd = (p.data_ptr(), s.data_ptr(), rbq.shape(5, 128, 2, 0), x.data_ptr(), 1, y.data_ptr(), None, 0)
    assert L.rbq_gemm_ex(*odd, rbq.RBQ_EPILOGUE_SILU_MUL, st) == rbq.RBQ_ERR_INVALID_ARG
    old = rbq.set_path(rbq.PATH_DECODE)
    try:
        assert L.rbq_gemm_ex(*args, rbq.RBQ_EPILOGUE_SILU_MUL, st) == rbq.RBQ_ERR_UNSUPPORTED
    finally:
        rbq.set_path(old)
    assert L.rbq_gemm_ex(*args, rbq.RBQ_EPILOGUE_SILU_MUL, st) == rbq.RBQ_OK
    torch.cuda.synchronize()
    assert (y[0, 3:] == 0).all()   # only out/2 = 3 columns written
