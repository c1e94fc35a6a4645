"""Host-side checks of the C ABI (include/rbq.h): the library loads, exports
every declared symbol, and validates arguments before touching a device.
No compute call is made here."""
import ctypes
import os
import re

import pytest
import torch

import gemm_rbq_encode_amd as rbq

pytestmark = pytest.mark.cpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "rbq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rbq_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 13, names
    L = ctypes.CDLL(rbq.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_binding_covers_header():
    from gemm_rbq_encode_amd import _binding
    assert set(declared_functions()) == set(_binding._SIGNATURES)


def test_sizes_and_shape_checks():
    s = rbq.shape(4096, 11008, 2, 0)
    assert rbq.planes_bytes(s) == 2 * 4096 * (11008 // 32) * 4
    assert rbq.scales_bytes(s) == 2 * 4096 * 2
    g = rbq.shape(13824, 5120, 4, 128)
    assert rbq.planes_bytes(g) == 4 * 13824 * 160 * 4
    assert rbq.scales_bytes(g) == 4 * 13824 * 40 * 2
    L = rbq.lib()
    assert L.rbq_check_shape(s) == rbq.RBQ_OK
    bad = [rbq.shape(-1, 64, 2), rbq.shape(8, 48, 2), rbq.shape(8, 64, 0), rbq.shape(8, 64, 9),
           rbq.shape(8, 64, 2, 64), rbq.shape(8, 96, 2, 128), rbq.shape(8, -32, 2)]
    for b in bad:
        assert L.rbq_check_shape(b) == rbq.RBQ_ERR_INVALID_ARG, b
        assert rbq.planes_bytes(b) == 0 and rbq.scales_bytes(b) == 0
    assert rbq.planes_bytes(rbq.shape(0, 64, 2)) == 0
    # the split family takes 2..16 tokens; its workspace holds whole
    # slices of fp32 partial outputs
    assert rbq.lib().rbq_gemm_workspace_bytes(s, 17) == 0
    assert rbq.lib().rbq_gemm_workspace_bytes(s, 16) % (16 * 4096 * 4) == 0


def test_status_strings_and_version():
    for st in range(6):
        assert rbq.status_string(st).startswith("RBQ_")
    assert "unknown" in rbq.status_string(99)
    assert "gfx950" in rbq.version()
    assert rbq.last_hip_error() == 0


def test_argument_errors_before_any_launch():
    L = rbq.lib()
    s = rbq.shape(64, 128, 2, 0)
    ok = 0x10000  # aligned stand-in addresses: argument checks never dereference
    # null pointers
    assert L.rbq_encode(None, s, ok, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_encode(ok, s, None, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm(ok, ok, s, None, 1, ok, None, 0, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm(ok, ok, s, ok, 1, None, None, 0, None) == rbq.RBQ_ERR_INVALID_ARG
    # bad shape / M / flags
    assert L.rbq_encode(ok, rbq.shape(64, 100, 2), ok, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm(ok, ok, s, ok, -1, ok, None, 0, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_encode_ex(ok, s, ok, ok, None, 8, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm(ok, ok, s, ok, 1, ok, None, 16, None) == rbq.RBQ_ERR_INVALID_ARG
    # misalignment
    assert L.rbq_encode(ok + 2, s, ok, ok, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_encode(ok, s, ok, ok + 1, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_gemm(ok + 4, ok, s, ok, 1, ok, None, 0, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_gemm(ok, ok, s, ok + 8, 1, ok, None, 0, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_gemm(ok, ok, s, ok, 1, ok + 1, None, 0, None) == rbq.RBQ_ERR_ALIGNMENT
    # too long a row for the encoder
    big = rbq.shape(4, 32768 + 32, 2, 0)
    assert L.rbq_encode(ok, big, ok, ok, None, None) == rbq.RBQ_ERR_UNSUPPORTED
    # refit: null pointers, shape, W alignment (16 bytes), row length
    assert L.rbq_refit(None, s, ok, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_refit(ok, s, ok, None, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_refit(ok, rbq.shape(64, 100, 2), ok, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_refit(ok + 4, s, ok, ok, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_refit(ok, s, ok, ok + 1, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_refit(ok, big, ok, ok, None, None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_refit(None, rbq.shape(0, 64, 2), None, None, None, None) == rbq.RBQ_OK
    # rebinarize: null pointers, shape, alignment, K beyond 4
    assert L.rbq_rebinarize(None, s, ok, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_rebinarize(ok, s, None, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_rebinarize(ok, s, ok, None, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_rebinarize(ok, rbq.shape(64, 100, 2), ok, ok, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_rebinarize(ok + 2, s, ok, ok, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_rebinarize(ok, s, ok + 2, ok, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_rebinarize(ok, s, ok, ok + 1, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_rebinarize(ok, s, ok, ok, ok + 2, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_rebinarize(ok, rbq.shape(64, 128, 5), ok, ok, None, None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_rebinarize(None, rbq.shape(0, 64, 2), None, None, None, None) == rbq.RBQ_OK
    # empty work is fine and enqueues nothing
    assert L.rbq_encode(None, rbq.shape(0, 64, 2), None, None, None, None) == rbq.RBQ_OK
    assert L.rbq_gemm(None, None, s, None, 0, None, None, 0, None) == rbq.RBQ_OK
    assert L.rbq_gemm(None, None, rbq.shape(0, 64, 2), None, 3, None, None, 0, None) == rbq.RBQ_OK


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_valid_call_without_device_reports_no_device():
    L = rbq.lib()
    s = rbq.shape(64, 128, 2, 0)
    ok = 0x10000
    assert L.rbq_encode(ok, s, ok, ok, None, None) == rbq.RBQ_ERR_NO_DEVICE
    assert L.rbq_refit(ok, s, ok, ok, None, None) == rbq.RBQ_ERR_NO_DEVICE
    assert L.rbq_rebinarize(ok + 4, s, ok, ok, None, None) == rbq.RBQ_ERR_NO_DEVICE
    assert L.rbq_gemv(ok, ok, s, ok, ok, None) == rbq.RBQ_ERR_NO_DEVICE
    assert L.rbq_gemm(ok, ok, s, ok, 2, ok, None, 0, None) == rbq.RBQ_ERR_NO_DEVICE


def test_path_override_roundtrip():
    old = rbq.set_path(rbq.PATH_VALU)
    try:
        assert rbq.set_path(rbq.PATH_AUTO) == rbq.PATH_VALU
    finally:
        rbq.set_path(old)
    assert rbq.set_stream_split(2) == 0
    assert rbq.set_stream_split(0) == 2
    with pytest.raises(ValueError):
        rbq.set_stream_split(3)
    L = rbq.lib()
    assert L.rbq_select_path(rbq.shape(4096, 4096, 2), 1) == rbq.PATH_STREAM
    assert L.rbq_select_path(rbq.shape(22016, 4096, 2), 1) == rbq.PATH_FLAT
    assert L.rbq_select_path(rbq.shape(4096, 11008, 2), 1) == rbq.PATH_FLAT
    assert L.rbq_select_path(rbq.shape(22016, 4096, 2), 2) == rbq.PATH_FLAT
    assert L.rbq_select_path(rbq.shape(4096, 4096, 2), 2) == rbq.PATH_STREAM
    assert L.rbq_select_path(rbq.shape(4096, 4096, 2), 4) == rbq.PATH_DECODE
    assert L.rbq_select_path(rbq.shape(4096, 4096, 2), 16) == rbq.PATH_SPLIT
    assert L.rbq_select_path(rbq.shape(11008, 4096, 2), 8) == rbq.PATH_SPLIT
    assert L.rbq_select_path(rbq.shape(4096, 11008, 2), 16) == rbq.PATH_SPLIT
    # the split family needs a workspace only where it can run
    assert L.rbq_gemm_workspace_bytes(rbq.shape(4096, 11008, 2), 1) == 0
    assert L.rbq_gemm_workspace_bytes(rbq.shape(5120, 5120, 4, 128), 16) == 0
    assert L.rbq_select_path(rbq.shape(11008, 4096, 2), 4) == rbq.PATH_FLAT
    assert L.rbq_select_path(rbq.shape(4096, 4096, 8), 1) == rbq.PATH_VALU


def test_binding_refuses_host_tensors():
    with pytest.raises(TypeError):
        rbq.encode(torch.zeros(4, 64), 2)


def test_dual_sizes_and_argument_errors():
    L = rbq.lib()
    s = rbq.shape(64, 256, 2, 0)
    assert L.rbq_dual_g_bytes(s) == 2 * 64 * 2 and L.rbq_dual_h_bytes(s) == 2 * 256 * 2
    assert L.rbq_dual_g_bytes(rbq.shape(64, 256, 2, 128)) == 0
    ws = L.rbq_encode_dual_workspace_bytes(s)
    assert ws >= 64 * 256 * 4 + 64 * 8 + 256 * 8 and ws % 256 == 0
    ok = 0x10000
    g128 = rbq.shape(64, 256, 2, 128)
    assert L.rbq_encode_dual(ok, g128, ok, ok, ok, ok, ws, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemv_dual(ok, ok, ok, g128, ok, ok, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_encode_dual(None, s, ok, ok, ok, ok, ws, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_encode_dual(ok, s, ok, ok, ok, None, ws, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_encode_dual(ok, s, ok, ok, ok, ok, ws - 1, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_encode_dual(ok, s, ok, ok, ok, ok + 16, ws, None, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_encode_dual(ok, rbq.shape(64, 96, 2), ok, ok, ok, ok, ws, None, None) == rbq.RBQ_ERR_UNSUPPORTED
    big = rbq.shape(4, rbq_dual_max_in() + 128, 2)
    assert L.rbq_encode_dual(ok, big, ok, ok, ok, ok, 1 << 40, None, None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_gemv_dual(ok, ok, ok, rbq.shape(64, 256, 5), ok, ok, None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_gemv_dual(ok, ok, ok, rbq.shape(64, 96, 2), ok, ok, None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_gemv_dual(ok, ok, None, s, ok, ok, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemv_dual(ok, ok, ok + 8, s, ok, ok, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_gemv_dual(ok, ok, ok, s, ok + 8, ok, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_gemv_dual(ok + 4, ok, ok, s, ok, ok, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_gemv_dual(ok, ok, ok, s, ok, ok + 1, None) == rbq.RBQ_ERR_ALIGNMENT
    # empty shapes enqueue nothing
    assert L.rbq_encode_dual(None, rbq.shape(0, 256, 2), None, None, None, None, 0, None, None) == rbq.RBQ_OK
    assert L.rbq_gemv_dual(None, None, None, rbq.shape(0, 256, 2), None, None, None) == rbq.RBQ_OK


def rbq_dual_max_in():
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "rbq.h")).read()
    return int(re.search(r"#define RBQ_DUAL_MAX_IN\s+(\d+)", text).group(1))


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_dual_valid_call_without_device_reports_no_device():
    L = rbq.lib()
    s = rbq.shape(64, 256, 2, 0)
    ok = 0x10000
    ws = L.rbq_encode_dual_workspace_bytes(s)
    assert L.rbq_encode_dual(ok, s, ok, ok, ok, ok, ws, None, None) == rbq.RBQ_ERR_NO_DEVICE
    assert L.rbq_gemv_dual(ok, ok, ok, s, ok, ok, None) == rbq.RBQ_ERR_NO_DEVICE


def test_gemm_dual_argument_errors():
    L = rbq.lib()
    s = rbq.shape(64, 128, 2, 0)
    ok = 0x10000
    assert L.rbq_gemm_dual(ok, ok, ok, s, ok, -1, ok, None) == rbq.RBQ_ERR_INVALID_ARG         # M < 0
    assert L.rbq_gemm_dual(ok, ok, ok, rbq.shape(64, 128, 2, 128), ok, 4, ok, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm_dual(ok, ok, ok, rbq.shape(64, 100, 2), ok, 4, ok, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm_dual(None, ok, ok, s, ok, 4, ok, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm_dual(ok, ok, ok, s, ok, 4, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_gemm_dual(ok, ok, ok + 8, s, ok, 4, ok, None) == rbq.RBQ_ERR_ALIGNMENT          # h
    assert L.rbq_gemm_dual(ok, ok, ok, s, ok + 8, 4, ok, None) == rbq.RBQ_ERR_ALIGNMENT          # X
    assert L.rbq_gemm_dual(ok, ok, ok, s, ok, 4, ok + 1, None) == rbq.RBQ_ERR_ALIGNMENT          # Y
    assert L.rbq_gemm_dual(ok, ok, ok, s, ok, 0, ok, None) == rbq.RBQ_OK                         # nothing to do
