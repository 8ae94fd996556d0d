"""The two measurement aids.  The read probe (qmv_read_probe) runs over
ragged and large sizes without touching anything but its sink; the
matrix-core probe (qmv_mfma_probe) reports plausible cycle and tick counts
for every wave and writes only its outputs; both reject bad arguments."""
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


@pytest.mark.parametrize("wps,rnd", [(1, 0), (1, 1), (2, 0), (2, 1)])
def test_mfma_probe_counts_and_writes_only_its_outputs(wps, rnd):
    """Every wave reports a positive cycle and tick count within the range
    the products' count allows; the lanes' sums are finite (zero for the
    constant operands, whose second factor is 0); nothing past the outputs
    changes."""
    import torch
    waves = 1024 * wps
    iters = 64
    clocks = torch.zeros(2 * waves + 16, dtype=torch.int64, device="cuda")
    sink = torch.zeros(64 * waves + 64, dtype=torch.float32, device="cuda")
    Q.qmv_mfma_probe(rnd, wps, iters, clocks, sink)
    torch.cuda.synchronize()
    c = clocks[:2 * waves].view(-1, 2).cpu()
    products = 8 * iters
    assert bool((c[:, 0] >= 4 * products).all()) and bool((c[:, 0] < 4096 * products).all())
    assert bool((c[:, 1] > 0).all())
    s = sink[:64 * waves]
    assert bool(torch.isfinite(s).all())
    if rnd == 0:
        assert torch.count_nonzero(s).item() == 0
    assert torch.count_nonzero(clocks[2 * waves:]).item() == 0
    assert torch.count_nonzero(sink[64 * waves:]).item() == 0


def test_mfma_probe_rejects_bad_arguments():
    import torch
    L = Q.lib()
    clocks = torch.zeros(4096, dtype=torch.int64, device="cuda")
    sink = torch.zeros(64 * 2048, dtype=torch.float32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    c, k = clocks.data_ptr(), sink.data_ptr()
    assert L.qmv_mfma_probe(0, 1, 16, None, k, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(0, 1, 16, c, None, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(2, 1, 16, c, k, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(0, 0, 16, c, k, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(0, 3, 16, c, k, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(0, 1, 0, c, k, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(0, 1, (1 << 20) + 1, c, k, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(0, 1, 16, c + 4, k, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(0, 1, 16, c, k + 2, s) == Q.QMV_E_ARG
    assert L.qmv_mfma_probe(1, 2, 16, c, k, s) == Q.QMV_OK
    torch.cuda.synchronize()
