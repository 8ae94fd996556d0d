"""QMV_E_NOMEM: with the GPU's memory taken (by torch allocations, nothing
launched), calls that must allocate report QMV_E_NOMEM and leave no state
behind; once the memory is released the same calls succeed.

- qmv_upload of a 512 MiB matrix (its device image);
- qmv_gemm of 65536 tokens on a new stream (its 512 MiB workspace of staged
  activations; the workspace is cached per stream, so a fresh stream is
  used)."""
import numpy as np
import pytest

import cases as K
from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def fill_device(torch, floor):
    """Allocates device memory in shrinking chunks until even `floor` bytes
    no longer fit; returns the held tensors."""
    held = []
    chunk = 64 << 30
    while chunk >= floor:
        try:
            held.append(torch.empty(chunk, dtype=torch.uint8, device="cuda"))
        except torch.OutOfMemoryError:
            chunk //= 2
    return held


def test_nomem_then_recovery():
    import torch
    R, C, B = 32, 4096, 65536
    img = K.make_image(995, 0, K.Q4, 1, R, C)
    h = K.upload(img, K.Q4, 1, R, C)
    big = np.zeros(Q.qmv_span(K.Q8, 0, 16384, 32768)["min_span"], dtype=np.uint8)  # 537 MB
    x = torch.zeros((B, C), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((B, R), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    held = []
    try:
        held = fill_device(torch, 64 << 20)
        s = torch.cuda.Stream()
        with pytest.raises(Q.QmvError) as e1:
            Q.qmv_gemm(h, x, y, stream=s)
        assert e1.value.status == Q.QMV_E_NOMEM
        h2 = Q.qmv_create(K.Q8, 0, 16384, 32768)
        with pytest.raises(Q.QmvError) as e2:
            Q.qmv_upload(h2, big)
        assert e2.value.status == Q.QMV_E_NOMEM
    finally:
        del held
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    try:
        # the same calls once memory is free: the handle was left unuploaded
        Q.qmv_upload(h2, big)
        Q.qmv_gemm(h, x[:512], y[:512], stream=s)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y[:512]).item() == 0   # zero activations
    finally:
        Q.qmv_destroy(h2)
        Q.qmv_destroy(h)
