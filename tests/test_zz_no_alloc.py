"""rbq_gemm_noalloc through the C ABI: the split-column kernels' scratch
from the library's static device buffer instead of a caller workspace.
Its output must equal rbq_gemm's with a workspace, bit for bit (same
kernels, fixed summation order), on two calls in a row, the second with a
smaller input, and calls needing more than the buffer are refused before
anything is enqueued."""
import numpy as np
import pytest
import torch

import gemm_rbq_encode_amd as rbq
import workloads

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def operands(out, inf, K, M, seed):
    p = workloads.random_planes(K, out, inf, seed=seed)
    s = workloads.random_scales(K, out, 1, seed=seed + 1, signed=True)
    X = workloads.gaussian_activations(M, inf, seed=seed + 2)
    return (torch.from_numpy(p.view(np.int32)).to(dev()), torch.from_numpy(s.view(np.float16)).to(dev()),
            torch.from_numpy(X.view(np.float16)).to(dev()))


def call_noalloc(p, s, X, Y):
    L = rbq.lib()
    K, out, words = p.shape
    st = L.rbq_gemm_noalloc(p.data_ptr(), s.data_ptr(), rbq.shape(out, words * 32, K, 0), X.data_ptr(),
                            X.shape[0], Y.data_ptr(), torch.cuda.current_stream(dev()).cuda_stream)
    return st


def call_with_workspace(p, s, X):
    L = rbq.lib()
    K, out, words = p.shape
    sh = rbq.shape(out, words * 32, K, 0)
    need = int(L.rbq_gemm_workspace_bytes(sh, X.shape[0]))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev())
    Y = torch.empty((X.shape[0], out), dtype=torch.float16, device=dev())
    st = L.rbq_gemm(p.data_ptr(), s.data_ptr(), sh, X.data_ptr(), X.shape[0], Y.data_ptr(), ws.data_ptr(), need,
                    torch.cuda.current_stream(dev()).cuda_stream)
    assert st == rbq.RBQ_OK, rbq.status_string(st)
    return Y, need


@pytest.mark.parametrize("path", [rbq.PATH_SPLIT, rbq.PATH_AUTO], ids=["split", "auto"])
def test_noalloc_matches_workspace_twice_then_smaller(path):
    old = rbq.set_path(path)
    try:
        for out, inf, K, M, seed in [(4096, 11008, 2, 16, 3), (1000, 8320, 1, 9, 5)]:
            p, s, X = operands(out, inf, K, M, seed)
            ref, need = call_with_workspace(p, s, X)
            assert need > 0 or path == rbq.PATH_AUTO    # the forced split family uses the scratch
            Y = torch.full((M, out), float("nan"), dtype=torch.float16, device=dev())
            st = call_noalloc(p, s, X, Y)
            assert st == rbq.RBQ_OK, rbq.status_string(st)
            torch.cuda.synchronize()
            assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), f"{out}x{inf} M={M}"
    finally:
        rbq.set_path(old)


def test_noalloc_refuses_more_than_its_buffer():
    old = rbq.set_path(rbq.PATH_SPLIT)
    try:
        # the first layer the split kernels take whose partial sums exceed the
        # buffer (the split plan depends on the device's LDS size)
        K, M = 1, 16
        big = [(o, i) for o, i in [(16000, 16384), (16128, 16384), (12000, 32768), (7000, 65536),
                                   (60000, 8192), (30000, 16384)]
               if rbq.lib().rbq_gemm_workspace_bytes(rbq.shape(o, i, K, 0), M) > rbq.RBQ_NOALLOC_SCRATCH_BYTES]
        assert big, "no candidate layer needs more scratch than the buffer"
        out, inf = big[0]
        p = torch.zeros((K, out, inf // 32), dtype=torch.int32, device=dev())
        s = torch.zeros((K, out), dtype=torch.float16, device=dev())
        X = torch.zeros((M, inf), dtype=torch.float16, device=dev())
        Y = torch.full((M, out), 3.0, dtype=torch.float16, device=dev())
        assert call_noalloc(p, s, X, Y) == rbq.RBQ_ERR_SCRATCH_LIMIT
        torch.cuda.synchronize()
        assert bool((Y == 3.0).all())          # nothing was written
    finally:
        rbq.set_path(old)


def test_noalloc_empty_and_small_calls():
    """Calls that need no scratch (one token, empty shapes) go through too."""
    p, s, X = operands(512, 1024, 2, 1, 9)
    ref, _ = call_with_workspace(p, s, X)
    Y = torch.empty((1, 512), dtype=torch.float16, device=dev())
    assert call_noalloc(p, s, X, Y) == rbq.RBQ_OK
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), ref.view(torch.int16))
    L = rbq.lib()
    assert L.rbq_gemm_noalloc(None, None, rbq.shape(0, 128, 2, 0), None, 4, None, None) == rbq.RBQ_OK
