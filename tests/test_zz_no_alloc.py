"""qmv_gemm_noalloc (the allocation-free prefill product, on the library's
fixed scratch) against qmv_gemm on the same inputs, through the C ABI: two
calls in a row, the second smaller than the first (the scratch keeps the
first call's contents), plus a batch that needs several passes of the
scratch, each checked against the oracle at the parity bar
|y - ref| <= 2e-3 * sum |w||x|."""
import ctypes

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


def run(fn, h, xb):
    """y from fn (the C entry point) called through ctypes on the current stream."""
    import torch
    xd = K.dev(xb.view(np.int16)).view(torch.bfloat16)
    y = torch.full((xb.shape[0], h.rows), np.nan, dtype=torch.float32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = fn(h.ptr, ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(y.data_ptr()), xb.shape[0], s)
    torch.cuda.synchronize()
    assert st == Q.QMV_OK, Q.qmv_status_str(st)
    return y.cpu().numpy()


# (wtype, scale_f16, rows, cols, first batch, second batch): the second
# call smaller; the last shape splits K (few row tiles)
CASES = [(K.Q4, 1, 1000, 4096, 300, 37), (K.Q8, 0, 4096, 14336, 512, 100),
         (K.Q8, 1, 257, 2048, 64, 9)]


@pytest.mark.parametrize("wt,sf,R,C,B1,B2", CASES)
def test_noalloc_matches_gemm_twice(wt, sf, R, C, B1, B2):
    L = Q.lib()
    img = K.make_image(990, 0, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        sel = K.sample_rows(R, 48, seed=R) if R > 600 else None
        for call, B in enumerate((B1, B2)):
            xb = K.make_xb(990, call, B, C)
            y_na = run(L.qmv_gemm_noalloc, h, xb)
            y_ref = run(L.qmv_gemm, h, xb)
            # the same kernels on the same pass: the same bits
            assert np.array_equal(y_na.view(np.uint32), y_ref.view(np.uint32)), f"call {call}"
            ref, norm = O.product(img, wt, sf, R, C, xb, sel=sel, threads=K.THREADS)
            ok, worst = O.within_tolerance(y_na if sel is None else y_na[:, sel], ref, norm)
            assert ok, f"call {call}: worst {worst:.3e}"
    finally:
        Q.qmv_destroy(h)


def test_noalloc_takes_large_batches_in_passes():
    """A batch whose staged activations exceed the scratch (64 MiB) runs in
    passes; each token's outputs still meet the bar (the split of K may
    differ from qmv_gemm's, so the bits may too)."""
    L = Q.lib()
    # 2200 x 16384 tokens: 72 MB staged, more than the scratch: two passes
    # of 1120 tokens
    wt, sf, R, C, B = K.Q4, 1, 160, 16384, 2200
    img = K.make_image(991, 0, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        xb = K.make_xb(991, 0, B, C)
        y = run(L.qmv_gemm_noalloc, h, xb)
        toks = np.array([0, 1, 1119, 1120, 1121, 1500, 2199], dtype=np.int64)
        ref, norm = O.product(img, wt, sf, R, C, xb[toks], threads=K.THREADS)
        ok, worst = O.within_tolerance(y[toks], ref, norm)
        assert ok, worst
        assert np.all(np.isfinite(y))
    finally:
        Q.qmv_destroy(h)


def test_noalloc_argument_errors():
    import torch
    L = Q.lib()
    h = K.upload(K.make_image(992, 0, K.Q4, 1, 64, 256), K.Q4, 1, 64, 256)
    try:
        x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
        y = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        px, py = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr())
        assert L.qmv_gemm_noalloc(None, px, py, 4, s) == Q.QMV_E_ARG
        assert L.qmv_gemm_noalloc(h.ptr, None, py, 4, s) == Q.QMV_E_ARG
        assert L.qmv_gemm_noalloc(h.ptr, px, None, 4, s) == Q.QMV_E_ARG
        assert L.qmv_gemm_noalloc(h.ptr, px, py, 0, s) == Q.QMV_E_ARG
        assert L.qmv_gemm_noalloc(h.ptr, ctypes.c_void_p(x.data_ptr() + 2), py, 4, s) == Q.QMV_E_ARG
        torch.cuda.synchronize()
    finally:
        Q.qmv_destroy(h)
