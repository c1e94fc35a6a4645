"""The streaming-read probe (rbq_probe_read) runs on every size, touches
nothing but its sink's one word, and refuses bad arguments before launch."""
import ctypes

import pytest
import torch

import gemm_rbq_encode_amd as rbq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 1, 15, 16, 17, 4096 + 5, (1 << 20) + 3, 23 << 20])
def test_probe_reads_and_writes_nothing(nbytes):
    dev = torch.device("cuda:0")
    buf = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    guard = torch.full((4,), 7, dtype=torch.int32, device=dev)
    sink = guard[1:2]
    rbq.probe_read(buf, sink, nbytes)
    torch.cuda.synchronize()
    assert guard.tolist() == [7, 7, 7, 7]
    assert int(buf.sum()) == 0


def test_probe_refuses_bad_arguments():
    dev = torch.device("cuda:0")
    buf = torch.zeros(64, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    L = rbq.lib()
    assert L.rbq_probe_read(None, 16, sink.data_ptr(), None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_probe_read(buf.data_ptr(), 16, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_probe_read(buf.data_ptr() + 8, 16, sink.data_ptr(), None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_probe_read(buf.data_ptr(), 16, ctypes.c_void_p(sink.data_ptr() + 2), None) == \
        rbq.RBQ_ERR_ALIGNMENT
