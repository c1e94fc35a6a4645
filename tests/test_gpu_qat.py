"""GPU parity of the coupled forward and its straight-through backward
(rbq_qat_encode / rbq_qat_forward / rbq_qat_backward) against oracle/qat.py.

Cores: bit-exact.  Forward output: the rbq_gemm tolerance (rel-L2 1e-3,
max-abs 1e-2 of the rms) against the oracle, and bit-exact against rbq_gemm
on the oracle's planes.  Gradients: per element, bounds derived from the
kernels' arithmetic --
  dW   exact fp16 products, fp32 accumulation over M tokens:
       |err| <= 2 M 2^-24 sum_m |dY[m][r] X[m][j]|
  da   the fp32 dW errors summed over the group, one fp64 sum, one fp32
       rounding: sum_j tol_dW[r][j] + 2^-23 |da|
  dX   What formed in fp32 (K roundings of 2^-24) and carried by two fp16
       parts (2^-22 relative, 2^-25 absolute where the lower part is
       subnormal), fp32 accumulation over 2 out terms:
       |err| <= sum_r |dY[m][r]| (2^-21 |w| + 2^-25) + 4 out 2^-24 sum_r |dY w|
"""
import ctypes

import numpy as np
import pytest
import torch

import gemm_rbq_encode_amd as rbq
import workloads
from oracle import qat

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS_RMS = 1e-2
U = 2.0 ** -24


def dev():
    return torch.device("cuda:0")


def t_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def t_f16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).to(dev())


def case(out, inf, K, group, M, seed, signed=True):
    W = workloads.gaussian_weight(out, inf, seed, outliers=True)
    G = inf // group if group else 1
    s = workloads.random_scales(K, out, G, seed + 1, signed=signed)
    X = workloads.gaussian_activations(max(M, 1), inf, seed + 2)[:M]
    dY = workloads.gaussian_activations(max(M, 1), out, seed + 3)[:M]
    return W, s, X, dY


def gpu_cores(W, s, group):
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    p = rbq.qat_encode(t_f32(W), t_f16(s), group, status=st)
    torch.cuda.synchronize()
    return p.cpu().numpy().view(np.uint32), int(st.item())


SHAPES = [(256, 512, 2, 0), (384, 1024, 4, 128), (100, 4128, 3, 0), (64, 96, 1, 0), (33, 4128, 4, 0),
          (4096, 4096, 2, 0), (5120, 5120, 4, 128), (11008, 4096, 2, 0)]


@pytest.mark.parametrize("out,inf,K,group", SHAPES)
def test_cores_match_the_oracle(out, inf, K, group):
    for signed in (False, True):
        W, s, _, _ = case(out, inf, K, group, 1, 10 + out + K, signed)
        got, st = gpu_cores(W, s, group)
        assert st == 0
        assert np.array_equal(got, qat.cascade(W, s, group)), f"signed={signed}"


def test_cores_special_values():
    out, inf, K = 16, 256, 3
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((out, inf)) * 0.02).astype(np.float32)
    W[0, :6] = [np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-42]
    W[1, :] = 0.0
    W[2, :] = -0.0
    W[3, :] = np.float32(1e-40)
    s = workloads.random_scales(K, out, 1, 6, signed=True)
    s[0, 4, 0] = 0x0000                                   # zero scale
    s[1, 5, 0] = 0x0001                                   # subnormal scale
    s[2, 6, 0] = 0x7C00                                   # +Inf scale
    s[1, 7, 0] = 0x7E00                                   # NaN scale
    got, st = gpu_cores(W, s, 0)
    assert np.array_equal(got, qat.cascade(W, s, 0))
    assert st & rbq.RBQ_STATUS_NONFINITE_W


def test_cores_given_encoder_scales_are_the_encoder_planes():
    """Given the scales rbq_encode derived, the cascade retraces its planes."""
    W = workloads.gaussian_weight(512, 2048, 77, outliers=True)
    for K, group in ((2, 0), (4, 128)):
        p_enc, s_enc = rbq.encode(t_f32(W), K, group)
        p = rbq.qat_encode(t_f32(W), s_enc, group)
        torch.cuda.synchronize()
        assert torch.equal(p, p_enc)


@pytest.mark.parametrize("out,inf,K,group,M", [(256, 512, 2, 0, 4), (384, 1024, 4, 128, 1),
                                               (4096, 4096, 2, 0, 16), (1024, 4096, 2, 0, 300)])
def test_forward_matches_the_oracle(out, inf, K, group, M):
    W, s, X, _ = case(out, inf, K, group, M, 20 + M, signed=False)
    planes, Y = rbq.qat_forward(t_f32(W), t_f16(s), t_f16(X), group)
    torch.cuda.synchronize()
    p_ref, Y_ref = qat.forward(W, s, X, group)
    assert np.array_equal(planes.cpu().numpy().view(np.uint32), p_ref)
    Yg = Y.cpu().numpy().astype(np.float64)
    assert np.isfinite(Yg).all()
    rms = np.sqrt(np.mean(Y_ref ** 2))
    assert np.linalg.norm(Yg - Y_ref) <= REL_L2 * np.linalg.norm(Y_ref)
    assert np.abs(Yg - Y_ref).max() <= MAX_ABS_RMS * rms
    # the layer half is rbq_gemm itself
    Y2 = rbq.gemm(torch.from_numpy(p_ref.view(np.int32)).to(dev()), t_f16(s), t_f16(X), group)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)


def grad_tolerances(planes, s, X, dY, group):
    Xa = np.abs(X.view(np.float16).astype(np.float64))
    dYa = np.abs(dY.view(np.float16).astype(np.float64))
    M = X.shape[0]
    tol_dw = 2.0 * max(M, 1) * U * (dYa.T @ Xa) + 1e-300
    What = qat.dequant(planes, s, group)
    Wa = np.abs(What)
    out = What.shape[0]
    tol_dx = dYa @ (2.0 ** -21 * Wa + 2.0 ** -25) + 4.0 * out * U * (dYa @ Wa) + 1e-300
    K = planes.shape[0]
    inf = What.shape[1]
    G = inf // group if group else 1
    n = group if group else inf
    tol_ds = np.broadcast_to(tol_dw.reshape(out, G, n).sum(axis=2), (K, out, G))
    return tol_dx, tol_dw, tol_ds


BACKWARD = [(256, 512, 2, 0, 5), (384, 1024, 4, 128, 130), (100, 4128, 3, 0, 33), (64, 96, 1, 0, 1),
            (4096, 4096, 2, 0, 16), (1024, 2048, 4, 128, 257), (200, 1024, 2, 0, 0)]


@pytest.mark.parametrize("out,inf,K,group,M", BACKWARD)
def test_backward_matches_the_oracle(out, inf, K, group, M):
    W, s, X, dY = case(out, inf, K, group, M, 30 + out + M)
    planes = qat.cascade(W, s, group)
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    Xt = t_f16(X.reshape(M, inf))
    dYt = t_f16(dY.reshape(M, out))
    dX, dW, ds = rbq.qat_backward(torch.from_numpy(planes.view(np.int32)).to(dev()), t_f16(s), Xt, dYt, group,
                                  status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rdX, rdW, rds = qat.backward(planes, s, X.reshape(M, inf), dY.reshape(M, out), group)
    tdx, tdw, tds = grad_tolerances(planes, s, X.reshape(M, inf), dY.reshape(M, out), group)
    gdW = dW.cpu().numpy().astype(np.float64)
    gds = ds.cpu().numpy().astype(np.float64)
    gdX = dX.cpu().numpy().astype(np.float64)
    assert (np.abs(gdW - rdW) <= tdw).all(), f"dW max err {np.abs(gdW - rdW).max():.3e}"
    assert (np.abs(gds - rds) <= tds + 2.0 ** -23 * np.abs(rds) + 1e-300).all(), \
        f"dscales max err {np.abs(gds - rds).max():.3e}"
    assert gdX.shape == (M, inf)
    if M:
        assert (np.abs(gdX - rdX) <= tdx).all(), f"dX max err {np.abs(gdX - rdX).max():.3e}"
    if M == 0:
        assert not gdW.any() and not gds.any()


def test_backward_outputs_on_request():
    out, inf, K, group, M = 128, 256, 2, 0, 8
    W, s, X, dY = case(out, inf, K, group, M, 44)
    planes = torch.from_numpy(qat.cascade(W, s, group).view(np.int32)).to(dev())
    full = rbq.qat_backward(planes, t_f16(s), t_f16(X), t_f16(dY), group)
    only_dx = rbq.qat_backward(planes, t_f16(s), t_f16(X), t_f16(dY), group, need_dw=False, need_dscales=False)
    only_dw = rbq.qat_backward(planes, t_f16(s), t_f16(X), t_f16(dY), group, need_dx=False, need_dscales=False)
    torch.cuda.synchronize()
    assert only_dx[1] is None and only_dx[2] is None and torch.equal(only_dx[0], full[0])
    assert only_dw[0] is None and only_dw[2] is None and torch.equal(only_dw[1], full[1])


def test_backward_reports_weights_beyond_fp16():
    out, inf, K, M = 64, 128, 2, 4
    _, _, X, dY = case(out, inf, K, 0, M, 45)
    s = np.full((K, out, 1), np.float16(40000.0)).view(np.uint16)
    # planes with equal bits somewhere give 80000 (the cascade itself would
    # give opposite bits and 0 everywhere for such scales)
    planes = torch.from_numpy(workloads.random_planes(K, out, inf, 46).view(np.int32)).to(dev())
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    rbq.qat_backward(planes, t_f16(s), t_f16(X), t_f16(dY), 0, need_dw=False, need_dscales=False, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & rbq.RBQ_STATUS_SCALE_OVERFLOW


def test_argument_errors():
    L = rbq.lib()
    buf = torch.zeros(1 << 16, dtype=torch.int32, device=dev())
    p = buf.data_ptr()
    assert L.rbq_qat_encode(p, rbq.shape(32, 64, 5, 0), p, p, None, None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_qat_encode(p, rbq.shape(32, 48, 2, 0), p, p, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_qat_encode(None, rbq.shape(32, 64, 2, 0), p, p, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_qat_encode(ctypes.c_void_p(p + 2), rbq.shape(32, 64, 2, 0), p, p, None, None) == \
        rbq.RBQ_ERR_ALIGNMENT
    # the scale gradient needs dW
    assert L.rbq_qat_backward(p, p, rbq.shape(32, 64, 2, 0), p, p, 4, p, None, p, None, 0, None, None) == \
        rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_qat_backward(p, p, rbq.shape(32, 64, 2, 0), p, None, 4, p, p, None, None, 0, None, None) == \
        rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_qat_backward(p, p, rbq.shape(32, 64, 2, 0), p, p, -1, p, p, None, None, 0, None, None) == \
        rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_qat_backward(p, p, rbq.shape(32, 64, 2, 0), p, p, 4, p, p, None, None, 64, None, None) == \
        rbq.RBQ_ERR_INVALID_ARG


@pytest.mark.parametrize("M", [1, 16, 40])
def test_backward_slices_equal_one_slice(M):
    """With few tokens dX is summed over contraction slices in a workspace;
    without the workspace the same dX comes from one slice, within the bound,
    and two runs with the workspace are bit-identical."""
    out, inf, K, group = 4096, 1024, 2, 0
    W, s, X, dY = case(out, inf, K, group, M, 70 + M)
    planes = torch.from_numpy(qat.cascade(W, s, group).view(np.int32)).to(dev())
    need = rbq.lib().rbq_qat_backward_workspace_bytes(rbq.shape(out, inf, K, group), M)
    assert need > 0
    a = rbq.qat_backward(planes, t_f16(s), t_f16(X), t_f16(dY), group, need_dw=False, need_dscales=False)[0]
    b = rbq.qat_backward(planes, t_f16(s), t_f16(X), t_f16(dY), group, need_dw=False, need_dscales=False)[0]
    one = rbq.qat_backward(planes, t_f16(s), t_f16(X), t_f16(dY), group, need_dw=False, need_dscales=False,
                           workspace=torch.empty(0, dtype=torch.uint8, device=dev()))[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    rdX = qat.backward(qat.cascade(W, s, group), s, X, dY, group)[0]
    tdx = grad_tolerances(qat.cascade(W, s, group), s, X, dY, group)[0]
    for got in (a, one):
        assert (np.abs(got.cpu().numpy().astype(np.float64) - rdX) <= tdx).all()
