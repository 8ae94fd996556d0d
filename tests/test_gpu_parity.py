"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: dequantized values, integer dots and quantized activations bit for
bit; float32 products within |y - ref| <= 2e-3 * sum |w||x| per output
against the oracle's float64 product of the exact weights."""
import numpy as np
import pytest

import cases as K
import golden_io as G
import oracle as O
from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu
TOL = 2e-3


def close(y, ref, norm, what):
    ok, worst = O.within_tolerance(y, ref, norm, TOL)
    print(f"{what}: worst |y-ref|/norm = {worst:.3e}")
    assert ok, f"{what}: outside 2e-3 * norm (worst ratio {worst:.3e})"
    return worst


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


# ---- hand-derived fixtures --------------------------------------------------

FIXTURES = ["e1_q8_f32.txt", "e2_q4_f16.txt", "e3_q4_nibble_order.txt",
            "e4_f16_scale_edges.txt", "e4b_f32_scale_rounding.txt",
            "e7_q4_addressing.txt", "e8_q8_rows_batch.txt"]


@pytest.mark.parametrize("name", FIXTURES)
def test_fixture_on_gpu(name):
    kv = G.load(name)
    wt, sf, R, C, q, d = G.matrix(kv)
    img = O.layout(wt, sf, R, C, q, d, trailing_pad=False)
    h = K.upload(img, wt, sf, R, C)
    try:
        w = K.gpu_embed(h, list(range(R)))
        ref_w = O.dequant_rows(img, wt, sf, R, C, np.arange(R))
        assert np.array_equal(w.view(np.uint32), ref_w.view(np.uint32))
        if "expect_w_bits" in kv:
            assert np.array_equal(w.reshape(-1).view(np.uint32),
                                  np.array(G.words(kv["expect_w_bits"]), np.uint32))
        elif "expect_w" in kv:
            assert np.array_equal(w.reshape(-1), np.array(G.floats(kv["expect_w"]), np.float32))
        for xk, yk in (("x", "expect_y"), ("x2", "expect_y2")):
            if xk not in kv:
                continue
            x = G.activations(kv[xk], C)
            ref, norm = O.product(img, wt, sf, R, C, x)
            assert np.array_equal(ref, G.batch_floats(kv[yk]))
            close(K.gpu_gemv(h, x), ref, norm, f"{name} gemv {xk}")
            xb = np.ascontiguousarray(x).view(np.uint32)
            xb = (xb >> 16).astype(np.uint16)          # 0, 1, -1: exact in bf16
            close(K.gpu_gemm(h, xb), ref, norm, f"{name} gemm {xk}")
    finally:
        Q.qmv_destroy(h)


# ---- decode GEMV: small shapes, full oracle ---------------------------------

SMALL = [(1, 32), (3, 96), (37, 160), (130, 4096), (257, 1056), (64, 11008)]


@pytest.mark.parametrize("wt,sf", [(1, 0), (1, 1), (2, 0), (2, 1)])
@pytest.mark.parametrize("R,C", SMALL)
def test_gemv_small_full(wt, sf, R, C):
    img = K.make_image(100 + R, C, wt, sf, R, C, lo=-1e-2)   # negative scales too
    h = K.upload(img, wt, sf, R, C)
    try:
        for batch in (1, 2, 3, 8):
            x = K.make_x(100 + R, C + batch, batch, C)
            ref, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
            close(K.gpu_gemv(h, x), ref, norm, f"gemv {wt}/{sf} {R}x{C} b{batch}")
    finally:
        Q.qmv_destroy(h)


# Every one-shot launch shape, full oracle: rows per wave 4 / 2 / 1 for rows
# of one step (64 chunks of 16 bytes), 2 or 1 for two steps, sixteen-wave
# groups of one row for 4096-8192 rows of two to four steps (at both ends
# of that band, ragged), eight-wave groups below it, and rows of more steps.
SHAPES = [(2, 0, 8200, 1024), (1, 1, 5000, 512), (2, 1, 8500, 4096), (2, 1, 4100, 4096),
          (1, 0, 8192, 2048), (1, 1, 5000, 4096), (2, 0, 4097, 6144), (2, 1, 1000, 4096),
          (1, 1, 2000, 4096), (2, 1, 4095, 4096), (1, 0, 8193, 2048)]


@pytest.mark.parametrize("wt,sf,R,C", SHAPES)
def test_gemv_launch_shapes_full(wt, sf, R, C):
    img = K.make_image(150, R + C, wt, sf, R, C, lo=-1e-2)
    h = K.upload(img, wt, sf, R, C)
    try:
        for batch in (1, 3):
            x = K.make_x(150, R + batch, batch, C)
            ref, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
            close(K.gpu_gemv(h, x), ref, norm, f"gemv {wt}/{sf} {R}x{C} b{batch}")
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("wt,sf", [(1, 1), (2, 1), (2, 0)])
@pytest.mark.parametrize("batch", [9, 16, 33, 64, 65])
def test_gemv_large_batch_matrix_core_path(wt, sf, batch):
    R, C = 300, 1056
    img = K.make_image(200, batch, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        x = K.make_x(200, batch, batch, C)
        ref, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
        close(K.gpu_gemv(h, x), ref, norm, f"gemv-mfma {wt}/{sf} b{batch}")
    finally:
        Q.qmv_destroy(h)


# long rows on the batched fallback (f32 activations staged as scaled f16 in
# chunks of 8192 values: several chunks, one re-read, and a K tail)
@pytest.mark.parametrize("wt,sf,C", [(K.Q8, 0, 14336), (K.Q4, 1, 11008), (K.Q4, 0, 16416)])
def test_gemv_large_batch_long_rows(wt, sf, C):
    R, batch = 70, 12
    img = K.make_image(210, C, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        x = K.make_x(210, batch, batch, C)
        ref, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
        close(K.gpu_gemv(h, x), ref, norm, f"gemv-fallback {wt}/{sf} {R}x{C} b{batch}")
    finally:
        Q.qmv_destroy(h)


def test_gemv_unit_vectors_give_columns_exactly():
    # x = e_c: one nonzero product per row, so y is the dequantized column
    # bit for bit (the only rounding is fl32(v * d)).
    for wt, sf in ((1, 0), (2, 1), (2, 0), (1, 1)):
        R, C = 70, 256
        img = K.make_image(300, wt * 2 + sf, wt, sf, R, C, lo=-1e-2)
        h = K.upload(img, wt, sf, R, C)
        try:
            cols = [0, 1, 15, 16, 31, 32, 100, 255]
            x = np.zeros((len(cols), C), np.float32)
            x[np.arange(len(cols)), cols] = 1.0
            w = O.dequant_rows(img, wt, sf, R, C, np.arange(R))
            y = K.gpu_gemv(h, x)
            for i, c in enumerate(cols):
                assert np.array_equal(y[i], w[:, c]), (wt, sf, c)
        finally:
            Q.qmv_destroy(h)


def test_gemv_zero_weight_rows_are_exactly_zero():
    # Row 0: every Q4_0 nibble 8 (w = 0) with nonzero scales; row 1: zero
    # scales.  Their norms are 0, so y must be exactly 0.
    R, C = 3, 4096
    for sf in (0, 1):
        q = np.full(R * C // 2, 0x88, dtype=np.uint8)
        q[2 * C // 2:] = 0x13
        d = np.full(R * C // 32, 0.01, dtype=np.float16 if sf else np.float32)
        d[C // 32:2 * C // 32] = 0
        img = O.layout(2, sf, R, C, q, d)
        h = K.upload(img, 2, sf, R, C)
        try:
            x = K.make_x(301, sf, 4, C)
            ref, norm = O.product(img, 2, sf, R, C, x)
            assert np.all(norm[:, :2] == 0)
            y = K.gpu_gemv(h, x)
            assert np.all(y[:, :2] == 0)
            close(y, ref, norm, "zero rows")
        finally:
            Q.qmv_destroy(h)
    # Q8_0 rows of zero quants
    q = np.zeros(2 * 1024, dtype=np.int8)
    q[1024:] = 5
    img = O.layout(1, 1, 2, 1024, q, np.full(64, 0.5, np.float16))
    h = K.upload(img, 1, 1, 2, 1024)
    try:
        y = K.gpu_gemv(h, K.make_x(302, 0, 3, 1024))
        assert np.all(y[:, 0] == 0)
    finally:
        Q.qmv_destroy(h)


def test_gemv_is_deterministic():
    R, C = 4096, 4096
    img = K.make_image(2, 0, 2, 1, R, C)
    h = K.upload(img, 2, 1, R, C)
    try:
        x = K.make_x(2, 0, 1, C)
        a, b = K.gpu_gemv(h, x), K.gpu_gemv(h, x)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    finally:
        Q.qmv_destroy(h)


# ---- prefill GEMM: small shapes, full oracle --------------------------------

@pytest.mark.parametrize("wt,sf", [(1, 0), (1, 1), (2, 0), (2, 1)])
@pytest.mark.parametrize("R,C,B", [(1, 32, 1), (129, 96, 33), (200, 4160, 130),
                                   (128, 64, 64), (257, 1024, 7), (300, 96, 256),
                                   (130, 1056, 200), (1, 2048, 513)])
def test_gemm_small_full(wt, sf, R, C, B):
    img = K.make_image(400 + B, R, wt, sf, R, C, lo=-1e-2)
    h = K.upload(img, wt, sf, R, C)
    try:
        xb = K.make_xb(400 + B, R + 1, B, C)
        ref, norm = O.product(img, wt, sf, R, C, xb, threads=K.THREADS)
        close(K.gpu_gemm(h, xb), ref, norm, f"gemm {wt}/{sf} {R}x{C} b{B}")
    finally:
        Q.qmv_destroy(h)


# Large-batch GEMM shapes (batch >= 128): ragged rows and tokens, odd step
# counts, and a split K whose slices have different step counts.
@pytest.mark.parametrize("wt,sf", [(1, 0), (1, 1), (2, 0), (2, 1)])
@pytest.mark.parametrize("R,C,B", [(300, 384, 129), (1000, 640, 200), (256, 3200, 130),
                                   (513, 1152, 333)])
def test_gemm_large_batch_shapes(wt, sf, R, C, B):
    img = K.make_image(420 + B, R, wt, sf, R, C, lo=-1e-2)
    h = K.upload(img, wt, sf, R, C)
    try:
        xb = K.make_xb(420 + B, R + 2, B, C)
        ref, norm = O.product(img, wt, sf, R, C, xb, threads=K.THREADS)
        close(K.gpu_gemm(h, xb), ref, norm, f"gemm-large {wt}/{sf} {R}x{C} b{B}")
    finally:
        Q.qmv_destroy(h)


# ---- embedding gather -------------------------------------------------------

@pytest.mark.parametrize("wt,sf", [(1, 0), (1, 1), (2, 0), (2, 1)])
def test_embed_rows_bit_exact_small(wt, sf):
    R, C = 50, 4128
    img = K.make_image(500, wt * 2 + sf, wt, sf, R, C, lo=-1e-2)
    h = K.upload(img, wt, sf, R, C)
    try:
        ids = [0, 49, 7, 7, 13, -1, 50, 2**31 - 1, 25]
        out = K.gpu_embed(h, ids)
        good = [i for i in ids if 0 <= i < R]
        ref = O.dequant_rows(img, wt, sf, R, C, np.array(good))
        j = 0
        for k, i in enumerate(ids):
            if 0 <= i < R:
                assert np.array_equal(out[k].view(np.uint32), ref[j].view(np.uint32))
                j += 1
            else:
                assert np.all(out[k] == 0)            # out of range: zero row
    finally:
        Q.qmv_destroy(h)


# ---- activation quantizer and integer block dots ----------------------------

def test_quantize_q8_bit_exact():
    import torch
    kv = G.load("e5_quantizer.txt")
    blocks = [np.array(G.floats(kv[f"block_{b}_x"]), np.float32) for b in "abcde"]
    g = np.random.default_rng(11)
    rnd = (g.standard_normal(32 * 4096) * np.exp(g.uniform(-40, 40, 32 * 4096))).astype(np.float32)
    rnd[:32] = 0
    rnd[32:64] = 1e-31
    x = np.concatenate(blocks + [rnd])
    q_ref, d_ref = O.quantize_q8(x)
    xd = K.dev(x)
    q = torch.empty(x.size, dtype=torch.int8, device="cuda")
    d = torch.empty(x.size // 32, dtype=torch.float32, device="cuda")
    Q.qmv_quantize_q8(xd, q, d)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), d_ref.view(np.uint32))
    for b in range(5):
        assert q.cpu().numpy()[32 * b:32 * b + 32].tolist() == G.ints(kv[f"block_{'abcde'[b]}_q"])


@pytest.mark.parametrize("wt", [1, 2])
def test_block_dots_bit_exact(wt):
    import torch
    R, C = 77, 4096
    img = K.make_image(600, wt, wt, 1, R, C)
    h = K.upload(img, wt, 1, R, C)
    try:
        xq, _ = O.quantize_q8(K.make_x(600, wt, 1, C))
        xq[:32] = 127
        xq[32:64] = -127
        ref = O.block_dots(img, wt, R, C, xq)
        s = torch.empty((R, C // 32), dtype=torch.int32, device="cuda")
        Q.qmv_block_dots(h, K.dev(xq), s)
        torch.cuda.synchronize()
        assert np.array_equal(s.cpu().numpy(), ref)
    finally:
        Q.qmv_destroy(h)


# ---- argument errors on the GPU ---------------------------------------------

def test_gpu_argument_errors():
    import ctypes
    import torch
    R, C = 64, 256
    img = K.make_image(700, 0, 2, 1, R, C)
    h = K.upload(img, 2, 1, R, C)
    try:
        with pytest.raises(Q.QmvError) as e:
            Q.qmv_upload(h, img)                     # second upload
        assert e.value.status == Q.QMV_E_ARG
        x = torch.zeros(C + 4, dtype=torch.float32, device="cuda")
        y = torch.zeros(R + 4, dtype=torch.float32, device="cuda")
        L = Q.lib()
        bad = ctypes.c_void_p(x.data_ptr() + 4)      # misaligned
        assert L.qmv_gemv(h.ptr, bad, ctypes.c_void_p(y.data_ptr()), 1, None) == Q.QMV_E_ARG
        assert L.qmv_gemv(h.ptr, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                          0, None) == Q.QMV_E_ARG
    finally:
        Q.qmv_destroy(h)


def test_gemm_split_k_is_deterministic():
    # a narrow matrix with a long K takes the split-K path; partial sums are
    # added in slice order, so two runs agree bit for bit
    R, C, B = 256, 8192, 256
    img = K.make_image(450, 0, 1, 0, R, C)
    h = K.upload(img, 1, 0, R, C)
    try:
        xb = K.make_xb(450, 1, B, C)
        a, b = K.gpu_gemm(h, xb), K.gpu_gemm(h, xb)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        sel = np.array([0, 1, 127, 128, 255])
        ref, norm = O.product(img, 1, 0, R, C, xb, sel=sel, threads=K.THREADS)
        close(a[:, sel], ref, norm, "split-K gemm")
    finally:
        Q.qmv_destroy(h)


def test_gemv_group_mixed_types_against_oracle_and_single():
    # one launch over matrices of different storage types sharing x; each
    # output equals the single-matrix product bit for bit (same arithmetic)
    import torch
    C = 1056
    specs = [(2, 1, 300), (1, 1, 77), (2, 0, 129), (1, 0, 1)]
    imgs, hs = [], []
    try:
        for m, (wt, sf, R) in enumerate(specs):
            img = K.make_image(800, m, wt, sf, R, C, lo=-1e-2)
            imgs.append(img)
            hs.append(K.upload(img, wt, sf, R, C))
        for batch in (1, 3, 8):
            x = K.make_x(800, 10 + batch, batch, C)
            xd = K.dev(x)
            ys = [torch.empty((batch, R), dtype=torch.float32, device="cuda") for (_, _, R) in specs]
            Q.qmv_gemv_group(hs, xd, ys)
            torch.cuda.synchronize()
            for (wt, sf, R), img, h, y in zip(specs, imgs, hs, ys):
                yg = y.cpu().numpy()
                ref, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
                close(yg, ref, norm, f"group {wt}/{sf} {R}x{C} b{batch}")
                assert np.array_equal(yg.view(np.uint32), K.gpu_gemv(h, x).view(np.uint32))
    finally:
        for h in hs:
            Q.qmv_destroy(h)


@pytest.mark.parametrize("wt,sf,R,C", [(2, 1, 6200, 4096), (2, 0, 6201, 4096),
                                       (1, 0, 6144, 2048), (1, 1, 6145, 2048)])
def test_gemv_group_streaming_kernel_full(wt, sf, R, C):
    """Two same-type matrices of two-step rows with at least 6144 row pairs
    between them: the one-workgroup-per-compute-unit streaming kernel at
    batch 1 (odd row counts end in a half tile), full oracle."""
    import torch
    imgs = [K.make_image(820, m, wt, sf, R, C, lo=-1e-2) for m in range(2)]
    hs = [K.upload(img, wt, sf, R, C) for img in imgs]
    try:
        x = K.make_x(820, 5, 1, C)
        ys = [torch.empty((1, R), dtype=torch.float32, device="cuda") for _ in hs]
        Q.qmv_gemv_group(hs, K.dev(x), ys)
        torch.cuda.synchronize()
        for img, h, y in zip(imgs, hs, ys):
            ref, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
            close(y.cpu().numpy(), ref, norm, f"stream {wt}/{sf} {R}x{C}")
    finally:
        for h in hs:
            Q.qmv_destroy(h)


def test_gemv_group_rejects_mismatched_cols():
    import torch
    a = K.upload(K.make_image(801, 0, 2, 1, 64, 128), 2, 1, 64, 128)
    b = K.upload(K.make_image(801, 1, 2, 1, 64, 256), 2, 1, 64, 256)
    try:
        x = torch.zeros((1, 256), dtype=torch.float32, device="cuda")
        ys = [torch.zeros((1, 64), dtype=torch.float32, device="cuda") for _ in range(2)]
        with pytest.raises(Q.QmvError) as e:
            Q.qmv_gemv_group([a, b], x, ys)
        assert e.value.status == Q.QMV_E_SHAPE
    finally:
        Q.qmv_destroy(a)
        Q.qmv_destroy(b)


def test_gemv_nonfinite_activation_gives_nan():
    R, C = 64, 128
    img = K.make_image(92, 0, K.Q4, 1, R, C)
    h = K.upload(img, K.Q4, 1, R, C)
    try:
        x = K.make_x(92, 0, 3, C)
        x[0, 37] = np.nan
        x[1, 100] = np.inf
        y = K.gpu_gemv(h, x)
        assert np.all(np.isnan(y[0])) and np.all(np.isnan(y[1]))
        assert np.all(np.isfinite(y[2]))
    finally:
        Q.qmv_destroy(h)


# ---- batched GEMV on the f16 matrix-core path (Q8_0, f16 scales, cols % 256) --

@pytest.mark.parametrize("R,C", [(1, 256), (31, 512), (300, 1024), (1000, 768)])
@pytest.mark.parametrize("batch", [9, 33, 64, 65, 130])
def test_gemv_batched_f16_matrix_core_path(R, C, batch):
    img = K.make_image(300 + R, batch, K.Q8, 1, R, C, lo=-1e-2)   # negative scales too
    h = K.upload(img, K.Q8, 1, R, C)
    try:
        x = K.make_x(300 + R, C + batch, batch, C)
        ref, norm = O.product(img, K.Q8, 1, R, C, x, threads=K.THREADS)
        close(K.gpu_gemv(h, x), ref, norm, f"gemv-f16 {R}x{C} b{batch}")
    finally:
        Q.qmv_destroy(h)


def test_gemv_batched_f16_path_ranges_and_nonfinite():
    # scales up to 1000 (q * d up to 127000, past f16's 65504: the weights are
    # scaled by 2^-k to stay in f16), token rows whose magnitudes differ by
    # 2^40 from token to token and by 2^12 inside a token, and NaN / inf in
    # two tokens
    R, C, B = 200, 512, 20
    img = K.make_image(310, 0, K.Q8, 1, R, C, lo=1.0, hi=1000.0)
    h = K.upload(img, K.Q8, 1, R, C)
    try:
        g = np.random.default_rng(310)
        x = K.make_x(310, 1, B, C).astype(np.float64)
        x *= np.exp2(g.uniform(-20, 20, size=(B, 1)))       # per-token magnitude
        x *= np.exp2(g.uniform(-12, 0, size=(B, C)))        # spread inside a token
        x = x.astype(np.float32)
        ref, norm = O.product(img, K.Q8, 1, R, C, x, threads=K.THREADS)
        close(K.gpu_gemv(h, x), ref, norm, "gemv-f16 ranges")
        x[3, 17] = np.nan
        x[11, 400] = -np.inf
        y = K.gpu_gemv(h, x)
        assert np.all(np.isnan(y[3])) and np.all(np.isnan(y[11]))
        keep = [t for t in range(B) if t not in (3, 11)]
        assert np.all(np.isfinite(y[keep]))
    finally:
        Q.qmv_destroy(h)
