"""GPU parity of the product on Q8_0-quantized activations (qmv_gemm_q8,
int8 matrix cores) against the oracle: exact block sums, float32 combine
within (cols/32 + 2) 2^-23 sum_b |dw dx s|."""
import numpy as np
import pytest

import cases as K
import oracle as O
from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def quantized(config, matrix, batch, cols):
    """Seeded activations quantized on the CPU by the oracle's rule."""
    x = K.make_x(config, matrix, batch, cols)
    xq = np.zeros((batch, cols), dtype=np.int8)
    dx = np.zeros((batch, cols // 32), dtype=np.float32)
    for t in range(batch):
        xq[t], dx[t] = O.quantize_q8(x[t])
    return x, xq, dx


def gpu_q8(h, xq, dx):
    import torch
    y = torch.empty((xq.shape[0], h.rows), dtype=torch.float32, device="cuda")
    Q.qmv_gemm_q8(h, K.dev(xq), K.dev(dx), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("wt,sf", [(1, 0), (1, 1), (2, 0), (2, 1)])
@pytest.mark.parametrize("R,C,B", [(1, 32, 1), (37, 96, 5), (300, 1024, 130), (129, 4128, 7),
                                   (260, 2048, 257)])
def test_q8act_small_full(wt, sf, R, C, B):
    img = K.make_image(95, wt, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        x, xq, dx = quantized(95, B, B, C)
        y = gpu_q8(h, xq, dx)
        ref, bound = O.gemm_q8act(img, wt, sf, R, C, xq, dx, threads=K.THREADS)
        ok, worst = O.q8act_within_tolerance(y, ref, bound, C)
        assert ok, f"worst {worst:.3g} of the tolerance"
        # and within the activation quantization of the float32 product
        ref_x, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
        assert O.within_tolerance(y, ref_x, norm, 2e-2)[0]
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("wt,sf,R,C", [(2, 1, 14336, 4096), (1, 0, 4096, 14336)])
def test_q8act_prefill_shapes(wt, sf, R, C):
    """The two 512-token prefill shapes, every token, sampled rows."""
    img = K.make_image(4, 0 if wt == 2 else 1, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        _, xq, dx = quantized(4, 7, 512, C)
        y = gpu_q8(h, xq, dx)
        sel = K.sample_rows(R, 48, seed=R)
        ref, bound = O.gemm_q8act(img, wt, sf, R, C, xq, dx, sel, threads=K.THREADS)
        ok, worst = O.q8act_within_tolerance(y[:, sel], ref, bound, C)
        assert ok, f"worst {worst:.3g} of the tolerance"
    finally:
        Q.qmv_destroy(h)


def test_q8act_zero_activations_and_argument_errors():
    import torch
    R, C = 64, 128
    img = K.make_image(96, 2, 2, 1, R, C)
    h = K.upload(img, 2, 1, R, C)
    try:
        xq = np.zeros((3, C), dtype=np.int8)
        dx = np.zeros((3, C // 32), dtype=np.float32)
        assert not gpu_q8(h, xq, dx).any()
        L = Q.lib()
        a = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
        p = a.data_ptr()
        assert L.qmv_gemm_q8(h.ptr, p, p, p, 0, None) == Q.QMV_E_ARG
        assert L.qmv_gemm_q8(h.ptr, None, p, p, 1, None) == Q.QMV_E_ARG
        assert L.qmv_gemm_q8(h.ptr, p + 4, p, p, 1, None) == Q.QMV_E_ARG
        assert L.qmv_gemm_q8(None, p, p, p, 1, None) == Q.QMV_E_ARG
        torch.cuda.synchronize()
    finally:
        Q.qmv_destroy(h)
