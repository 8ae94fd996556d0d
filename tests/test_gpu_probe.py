"""The read probe (qmv_read_probe, a measurement aid): it runs over ragged
and large sizes without touching anything but its sink, and rejects bad
arguments."""
import ctypes

import pytest

from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("nbytes", [16, 1008, 1 << 20, (3 << 20) + 48, 48 << 20])
def test_probe_reads_and_leaves_memory(nbytes):
    import torch
    src = torch.arange(nbytes // 4 + 64, dtype=torch.int32, device="cuda")
    before = src.clone()
    sink = torch.zeros(64 + 64, dtype=torch.int32, device="cuda")
    Q.qmv_read_probe(src, nbytes, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, before)
    # only the first 64 words of the sink may change (and practically never do)
    assert torch.count_nonzero(sink[64:]).item() == 0


def test_probe_rejects_bad_arguments():
    import torch
    L = Q.lib()
    src = torch.zeros(1024, dtype=torch.int32, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p, k = src.data_ptr(), sink.data_ptr()
    assert L.qmv_read_probe(None, 16, k, s) == Q.QMV_E_ARG
    assert L.qmv_read_probe(p, 16, None, s) == Q.QMV_E_ARG
    assert L.qmv_read_probe(p, 0, k, s) == Q.QMV_E_ARG
    assert L.qmv_read_probe(p, 24, k, s) == Q.QMV_E_ARG
    assert L.qmv_read_probe(p + 4, 16, k, s) == Q.QMV_E_ARG
    assert L.qmv_read_probe(p, 16, k + 2, s) == Q.QMV_E_ARG
    assert L.qmv_read_probe(p, 4096, k, s) == Q.QMV_OK
    torch.cuda.synchronize()
