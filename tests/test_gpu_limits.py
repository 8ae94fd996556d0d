"""GPU parity at the dimension limits (rows or cols = 2^24, the largest the
.mlb page's limits sentence leaves standing): the tallest matrix (2^24 x 32)
and the widest row (1 x 2^24), through the GEMV, the GEMM and the gather,
against the oracle on sampled rows."""
import numpy as np
import pytest

import cases as K
import oracle as O
from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu

LIMIT = 1 << 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_tallest_matrix():
    """2^24 rows x 32 cols, Q4_0 with f16 scales (288 MB)."""
    import torch
    R, C = LIMIT, 32
    img = K.make_image(80, 0, K.Q4, 1, R, C)
    h = K.upload(img, K.Q4, 1, R, C)
    try:
        sel = np.array(sorted({0, 1, 2, R // 2, R - 2, R - 1} |
                              set(np.random.default_rng(80).integers(0, R, 64).tolist())),
                       dtype=np.int64)
        for batch in (1, 5):
            x = K.make_x(80, batch, batch, C)
            y = K.gpu_gemv(h, x)
            ref, norm = O.product(img, K.Q4, 1, R, C, x, sel)
            ok, worst = O.within_tolerance(y[:, sel], ref, norm)
            assert ok, worst
        # the prefill GEMM on 128 tokens (the large-tile kernel), sampled rows
        xb = K.make_xb(80, 9, 128, C)
        xd = K.dev(xb.view(np.int16)).view(torch.bfloat16)
        yd = torch.empty((128, R), dtype=torch.float32, device="cuda")
        Q.qmv_gemm(h, xd, yd)
        torch.cuda.synchronize()
        ys = yd[:, torch.from_numpy(sel).cuda()].cpu().numpy()
        del yd
        ref, norm = O.product(img, K.Q4, 1, R, C, xb, sel)
        ok, worst = O.within_tolerance(ys, ref, norm)
        assert ok, worst
        ids = np.array([0, 1, R - 1], dtype=np.int32)
        out = K.gpu_embed(h, ids)
        rows = O.dequant_rows(img, K.Q4, 1, R, C, ids.astype(np.int64))
        assert np.array_equal(out.view(np.uint32), rows.view(np.uint32))
    finally:
        Q.qmv_destroy(h)


def test_widest_row():
    """1 row x 2^24 cols, Q8_0 with f32 scales (18 MB)."""
    R, C = 1, LIMIT
    img = K.make_image(81, 0, K.Q8, 0, R, C)
    h = K.upload(img, K.Q8, 0, R, C)
    try:
        for batch in (1, 3, 9):
            x = K.make_x(81, batch, batch, C)
            y = K.gpu_gemv(h, x)
            ref, norm = O.product(img, K.Q8, 0, R, C, x)
            ok, worst = O.within_tolerance(y, ref, norm)
            assert ok, worst
        xb = K.make_xb(81, 7, 2, C)
        y = K.gpu_gemm(h, xb)
        ref, norm = O.product(img, K.Q8, 0, R, C, xb)
        ok, worst = O.within_tolerance(y, ref, norm)
        assert ok, worst
        out = K.gpu_embed(h, np.array([0], dtype=np.int32))
        row = O.dequant_rows(img, K.Q8, 0, R, C, np.array([0], dtype=np.int64))
        assert np.array_equal(out.view(np.uint32), row.view(np.uint32))
    finally:
        Q.qmv_destroy(h)


def test_past_the_limit_is_refused():
    for R, C in ((LIMIT + 1, 32), (1, LIMIT + 32)):
        with pytest.raises(Q.QmvError) as e:
            Q.qmv_create(K.Q4, 1, R, C)
        assert e.value.status == Q.QMV_E_SHAPE
