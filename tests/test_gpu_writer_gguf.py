"""GPU parity of the GGUF upload (blocks repacked on the device) and of the
weight writer (the .mlb page's quantization rules on the GPU), both bit for
bit against the oracle."""
import numpy as np
import pytest

import cases as K
import oracle as O
from block_quant_weight_amd import qmv as Q
from test_oracle_writer_gguf import pack_gguf

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def gguf_matrix(seed, wt, R, C):
    g = np.random.default_rng(seed)
    if wt == K.Q8:
        q = g.integers(-127, 128, size=(R, C)).astype(np.int8)
    else:
        q = g.integers(0, 256, size=(R, C // 2)).astype(np.uint8)
    d = (g.uniform(1e-3, 1e-2, size=R * C // 32) * g.choice([-1, 1], size=R * C // 32))
    d = d.astype(np.float16)
    d[:3] = [0, -0.0, 6e-8]                     # zero, negative zero, an f16 subnormal
    return pack_gguf(wt, q, d.view(np.uint16))


@pytest.mark.parametrize("wt", [1, 2])
@pytest.mark.parametrize("R,C", [(37, 96), (300, 1024), (4096, 4096)])
def test_gguf_upload_bit_exact(wt, R, C):
    import torch
    blob = gguf_matrix(900 + R, wt, R, C)
    h = Q.qmv_create(wt, 1, R, C)
    hm = None
    try:
        Q.qmv_upload_gguf(h, blob)
        img = O.gguf_to_image(wt, R, C, blob)
        # every weight, bit for bit, through the gather
        ids = np.arange(R, dtype=np.int32)
        out = K.gpu_embed(h, ids)
        ref = O.dequant_rows(img, wt, 1, R, C, ids.astype(np.int64))
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
        # the same products as the two-array upload of the same weights
        hm = K.upload(img, wt, 1, R, C)
        for batch in (1, 3, 64):
            x = K.make_x(900, R + batch, batch, C)
            assert np.array_equal(K.gpu_gemv(h, x).view(np.uint32),
                                  K.gpu_gemv(hm, x).view(np.uint32))
        xb = K.make_xb(900, R, 130, C)
        assert np.array_equal(K.gpu_gemm(h, xb).view(np.uint32), K.gpu_gemm(hm, xb).view(np.uint32))
        torch.cuda.synchronize()
    finally:
        Q.qmv_destroy(h)
        Q.qmv_destroy(hm)


def writer_weights(seed, R, C):
    """Blocks spanning many magnitudes, with the edge cases of the rules."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((R, C)) * np.exp(g.uniform(-25, 9, (R, C // 32))).repeat(32, axis=1)
    w = w.astype(np.float32)
    flat = w.reshape(-1, 32)
    flat[0] = 0                                   # zero block
    flat[1] = 9e-31                               # below 1e-30
    flat[2] = np.float32(1e-40)                   # float32 subnormals
    flat[3, :] = 127 / 16                         # exact scale 1/16, ties
    flat[3, 1::2] = -1 / 32
    flat[4] = np.float32(2.0 ** -30) * np.arange(-16, 16)   # f16 scale underflows
    flat[5, 7] = -3 * np.abs(flat[5]).max()       # negative largest magnitude
    flat[6, :] = 0.5                              # equal magnitudes: first wins
    flat[6, 3] = -0.5
    return w


@pytest.mark.parametrize("wt,sf", [(1, 0), (1, 1), (2, 0), (2, 1)])
@pytest.mark.parametrize("R,C", [(5, 64), (300, 1024), (14336, 4096)])
def test_writer_bit_exact(wt, sf, R, C):
    import torch
    w = writer_weights(1000 + R + 7 * wt + sf, R, C)
    st, ref = O.quantize_weights(wt, sf, R, C, w)
    assert st == "ok"
    n = Q.qmv_span(wt, sf, R, C)["min_span"]
    img = torch.full((n + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    Q.qmv_quantize_weights(wt, sf, torch.from_numpy(w).cuda(), img)
    got = img.cpu().numpy()
    assert np.array_equal(got[:n], ref[:n])
    assert np.all(got[n:] == 0xAB)                # nothing written past min_span


@pytest.mark.parametrize("wt", [1, 2])
def test_writer_refuses_unstorable_f16_scale(wt):
    import torch
    R, C = 3, 64
    w = np.ones((R, C), dtype=np.float32)
    w[1, 40] = 127 * 70000.0 if wt == 1 else 8 * 70000.0
    assert O.quantize_weights(wt, 1, R, C, w)[0] == "format"
    n = Q.qmv_span(wt, 1, R, C)["min_span"]
    img = torch.zeros(n, dtype=torch.uint8, device="cuda")
    with pytest.raises(Q.QmvError) as e:
        Q.qmv_quantize_weights(wt, 1, torch.from_numpy(w).cuda(), img)
    assert e.value.status == Q.QMV_E_FORMAT
    # f32 scales store it
    st, ref = O.quantize_weights(wt, 0, R, C, w)
    n = Q.qmv_span(wt, 0, R, C)["min_span"]
    img = torch.zeros(n, dtype=torch.uint8, device="cuda")
    Q.qmv_quantize_weights(wt, 0, torch.from_numpy(w).cuda(), img)
    assert np.array_equal(img.cpu().numpy(), ref[:n])


def test_writer_image_uploads_and_multiplies():
    # quantize on the GPU, upload the bytes, multiply: the product of the
    # written matrix against the oracle
    import torch
    R, C = 512, 2048
    w = np.random.default_rng(5).standard_normal((R, C)).astype(np.float32)
    for wt, sf in ((1, 1), (2, 1)):
        n = Q.qmv_span(wt, sf, R, C)["min_span"]
        img = torch.zeros(n, dtype=torch.uint8, device="cuda")
        Q.qmv_quantize_weights(wt, sf, torch.from_numpy(w).cuda(), img)
        host = img.cpu().numpy()
        h = K.upload(host, wt, sf, R, C)
        try:
            x = K.make_x(950, wt, 2, C)
            ref, norm = O.product(host, wt, sf, R, C, x)
            ok, worst = O.within_tolerance(K.gpu_gemv(h, x), ref, norm, 2e-3)
            assert ok, worst
        finally:
            Q.qmv_destroy(h)


# ---- the Q4_0 least-squares writer ------------------------------------------

def search_rows_ref(w, sf, rows_sel):
    """Oracle image bytes (q rows, d entries) of the selected rows: rows are
    quantized independently, so a sample of rows checks the whole image."""
    C = w.shape[1]
    st, ref = O.quantize_q4_search(sf, len(rows_sel), C, w[rows_sel])
    assert st == "ok"
    sp = Q.qmv_span(2, sf, len(rows_sel), C)
    q = ref[:sp["q_bytes"]].reshape(len(rows_sel), C // 2)
    d = ref[sp["d_offset"]:sp["d_offset"] + sp["d_bytes"]].reshape(len(rows_sel), -1)
    return q, d


@pytest.mark.parametrize("sf", [0, 1])
@pytest.mark.parametrize("R,C", [(5, 64), (300, 1024), (14336, 4096)])
def test_search_writer_bit_exact(sf, R, C):
    import torch
    w = writer_weights(2000 + R + sf, R, C)
    sp = Q.qmv_span(2, sf, R, C)
    n = sp["min_span"]
    img = torch.full((n + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    Q.qmv_quantize_weights(2, sf, torch.from_numpy(w).cuda(), img, rule=Q.QMV_Q4_SEARCH)
    got = img.cpu().numpy()
    assert np.all(got[n:] == 0xAB)                # nothing written past min_span
    if R * C <= 300 * 1024:
        st, ref = O.quantize_q4_search(sf, R, C, w)
        assert st == "ok"
        assert np.array_equal(got[:n], ref[:n])
        return
    sel = K.sample_rows(R, 400, seed=R)
    q_ref, d_ref = search_rows_ref(w, sf, sel)
    q_got = got[:sp["q_bytes"]].reshape(R, C // 2)[sel]
    d_got = got[sp["d_offset"]:sp["d_offset"] + sp["d_bytes"]].reshape(R, -1)[sel]
    assert np.array_equal(q_got, q_ref)
    assert np.array_equal(d_got, d_ref)
    assert not got[sp["q_bytes"]:sp["d_offset"]].any()   # the zero pad


def test_search_writer_refusals():
    import torch
    R, C = 4, 64
    w = np.random.default_rng(9).standard_normal((R, C)).astype(np.float32)
    big = w.copy()
    big[2, 7] = 9e5                               # fitted |d| ~ 1.1e5: not an f16
    huge = w.copy()
    huge[1, 50] = 1e13                            # float32 cubes overflow
    for x, sf in ((big, 1), (huge, 0), (huge, 1)):
        assert O.quantize_q4_search(sf, R, C, x)[0] == "format"
        img = torch.zeros(Q.qmv_span(2, sf, R, C)["min_span"], dtype=torch.uint8, device="cuda")
        with pytest.raises(Q.QmvError) as e:
            Q.qmv_quantize_weights(2, sf, torch.from_numpy(x).cuda(), img, rule=Q.QMV_Q4_SEARCH)
        assert e.value.status == Q.QMV_E_FORMAT
    st, ref = O.quantize_q4_search(0, R, C, big)
    img = torch.zeros(Q.qmv_span(2, 0, R, C)["min_span"], dtype=torch.uint8, device="cuda")
    Q.qmv_quantize_weights(2, 0, torch.from_numpy(big).cuda(), img, rule=Q.QMV_Q4_SEARCH)
    assert np.array_equal(img.cpu().numpy(), ref[:img.numel()])
