"""GPU parity of the gated feed-forward pair, h = act(W1 x) * (W3 x) in one
launch (qmv_gemv_gated), against the oracle, plus its agreement with the
two plain products and its argument checks."""
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


def gpu_gated(h1, h3, x, act):
    import torch
    xd = K.dev(x.astype(np.float32))
    h = torch.empty((x.shape[0], h1.rows), dtype=torch.float32, device="cuda")
    Q.qmv_gemv_gated(h1, h3, xd, h, act=act)
    torch.cuda.synchronize()
    return h.cpu().numpy()


# (wtype, scale_f16, rows, cols): every row length class of the kernel
# (1, 2, 3 and 4 steps of 64 chunks), ragged row counts, and the decode
# layer's w1 | w3 (11008 x 4096 Q4_0, f16 scales)
SHAPES = [(K.Q4, 1, 37, 96), (K.Q8, 0, 300, 1024), (K.Q8, 1, 513, 2048),
          (K.Q4, 0, 1001, 4096), (K.Q8, 1, 129, 4096), (K.Q4, 1, 77, 8192),
          (K.Q4, 1, 11008, 4096)]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("wt,sf,R,C", SHAPES)
def test_gated_parity(wt, sf, R, C, act):
    h1 = K.upload(K.make_image(60 + wt, 1, wt, sf, R, C), wt, sf, R, C)
    h3 = K.upload(K.make_image(60 + wt, 3, wt, sf, R, C), wt, sf, R, C)
    img1 = K.make_image(60 + wt, 1, wt, sf, R, C)
    img3 = K.make_image(60 + wt, 3, wt, sf, R, C)
    try:
        sel = K.sample_rows(R, 96, seed=R) if R > 600 else None
        for batch in (1, 3, 8):
            x = K.make_x(60, 10 + batch, batch, C)
            h = gpu_gated(h1, h3, x, act)
            assert np.isfinite(h).all()
            href, y1, n1, y3, n3 = O.gated(img1, img3, wt, sf, R, C, x, act, sel,
                                           threads=K.THREADS)
            hs = h if sel is None else h[:, sel]
            ok, worst = O.gated_within_tolerance(hs, href, y1, n1, y3, n3, act)
            assert ok, f"batch {batch}: worst {worst:.3g} of the bound"
            # the gate and up sums are the plain products, bit for bit: the
            # only rounding left is the activation and the product
            # (float32 activation: a few roundings, plus the relative error
            # of e^v for an argument v of size |a| or 2|u|; below 2^-120 of
            # |a * up| the float32 e^v has overflowed and the gate is 0)
            z1, z3 = K.gpu_gemv(h1, x), K.gpu_gemv(h3, x)
            z = z1.astype(np.float64)
            with np.errstate(over="ignore"):
                a = np.vectorize(lambda v: O.ffn_act(v, act))(z)
            expect = a * z3.astype(np.float64)
            arg = np.abs(z) if act == 0 else 2 * np.abs(0.7978845608 * (z + 0.044715 * z ** 3))
            rel = 2.0 ** -20 * (1 + arg)
            floor = 2.0 ** -120 * (1 + np.abs(z * z3))
            assert np.all(np.abs(h - expect) <= rel * np.abs(expect) + floor)
    finally:
        Q.qmv_destroy(h1)
        Q.qmv_destroy(h3)


def test_gated_edge_inputs():
    """Zero activations give exactly zero; rows whose gate sum is large and
    negative give SiLU's -0 times the up sum."""
    import torch
    wt, sf, R, C = K.Q4, 1, 64, 256
    img1 = K.make_image(66, 1, wt, sf, R, C)
    img3 = K.make_image(66, 3, wt, sf, R, C)
    h1, h3 = K.upload(img1, wt, sf, R, C), K.upload(img3, wt, sf, R, C)
    try:
        x = np.zeros((2, C), dtype=np.float32)
        for act in (0, 1):
            assert not gpu_gated(h1, h3, x, act).any()
        x = K.make_x(66, 2, 1, C) * np.float32(3e4)
        h = gpu_gated(h1, h3, x, 0)
        href, y1, n1, y3, n3 = O.gated(img1, img3, wt, sf, R, C, x, 0)
        assert O.gated_within_tolerance(h, href, y1, n1, y3, n3, 0)[0]
        neg = y1 < -200
        assert neg.any()
        assert np.all(h[neg] == 0)
        torch.cuda.synchronize()
    finally:
        Q.qmv_destroy(h1)
        Q.qmv_destroy(h3)


def test_gated_rejects():
    import torch
    a = K.upload(K.make_image(67, 1, K.Q4, 1, 32, 128), K.Q4, 1, 32, 128)
    b8 = K.upload(K.make_image(67, 2, K.Q8, 1, 32, 128), K.Q8, 1, 32, 128)
    bf = K.upload(K.make_image(67, 3, K.Q4, 0, 32, 128), K.Q4, 0, 32, 128)
    br = K.upload(K.make_image(67, 4, K.Q4, 1, 33, 128), K.Q4, 1, 33, 128)
    w8 = K.upload(K.make_image(67, 5, K.Q8, 1, 8, 8192), K.Q8, 1, 8, 8192)
    hs = [a, b8, bf, br, w8]
    try:
        x = torch.zeros((1, 8192), dtype=torch.float32, device="cuda")
        h = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
        cases = [((a, b8, 0), Q.QMV_E_FORMAT), ((a, bf, 0), Q.QMV_E_FORMAT),
                 ((a, br, 0), Q.QMV_E_SHAPE), ((w8, w8, 0), Q.QMV_E_SHAPE),
                 ((a, a, 2), Q.QMV_E_ARG)]
        for (p, q, act), want in cases:
            st = Q.lib().qmv_gemv_gated(p.ptr, q.ptr, act, x.data_ptr(), h.data_ptr(), 1, None)
            assert st == want, (st, want)
        assert Q.lib().qmv_gemv_gated(a.ptr, a.ptr, 0, x.data_ptr(), h.data_ptr(), 0, None) == Q.QMV_E_ARG
        assert Q.lib().qmv_gemv_gated(a.ptr, a.ptr, 0, None, h.data_ptr(), 1, None) == Q.QMV_E_ARG
        torch.cuda.synchronize()
    finally:
        for m in hs:
            Q.qmv_destroy(m)
