"""Seeded random shapes through every product entry point, against the
oracle: storage and scale types, row counts that end mid-tile, column
counts of any number of blocks, and batches across the vector / matrix-core
boundary."""
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


def draw(seed, max_rows, max_blocks, max_batch):
    g = np.random.default_rng(seed)
    wt = int(g.choice([K.Q8, K.Q4]))
    sf = int(g.integers(0, 2))
    R = int(g.integers(1, max_rows + 1))
    C = 32 * int(g.integers(1, max_blocks + 1))
    B = int(g.integers(1, max_batch + 1))
    return wt, sf, R, C, B


@pytest.mark.parametrize("seed", range(40))
def test_random_gemv(seed):
    wt, sf, R, C, B = draw(3000 + seed, 700, 200, 20)
    img = K.make_image(100 + seed, 0, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        x = K.make_x(100 + seed, 1, B, C)
        ref, norm = O.product(img, wt, sf, R, C, x, threads=K.THREADS)
        ok, worst = O.within_tolerance(K.gpu_gemv(h, x), ref, norm)
        assert ok, (wt, sf, R, C, B, worst)
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("seed", range(20))
def test_random_gemm(seed):
    wt, sf, R, C, B = draw(4000 + seed, 500, 100, 300)
    img = K.make_image(200 + seed, 0, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        xb = K.make_xb(200 + seed, 1, B, C)
        ref, norm = O.product(img, wt, sf, R, C, xb, threads=K.THREADS)
        ok, worst = O.within_tolerance(K.gpu_gemm(h, xb), ref, norm)
        assert ok, (wt, sf, R, C, B, worst)
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("seed", range(20))
def test_random_gated(seed):
    import torch
    wt, sf, R, C, B = draw(5000 + seed, 600, 128, 9)
    act = seed % 2
    img1 = K.make_image(300 + seed, 1, wt, sf, R, C)
    img3 = K.make_image(300 + seed, 3, wt, sf, R, C)
    h1, h3 = K.upload(img1, wt, sf, R, C), K.upload(img3, wt, sf, R, C)
    try:
        x = K.make_x(300 + seed, 2, B, C)
        out = torch.empty((B, R), dtype=torch.float32, device="cuda")
        Q.qmv_gemv_gated(h1, h3, K.dev(x), out, act=act)
        torch.cuda.synchronize()
        href, y1, n1, y3, n3 = O.gated(img1, img3, wt, sf, R, C, x, act, threads=K.THREADS)
        ok, worst = O.gated_within_tolerance(out.cpu().numpy(), href, y1, n1, y3, n3, act)
        assert ok, (wt, sf, R, C, B, act, worst)
    finally:
        Q.qmv_destroy(h1)
        Q.qmv_destroy(h3)


@pytest.mark.parametrize("seed", range(20))
def test_random_q8act(seed):
    import torch
    wt, sf, R, C, B = draw(6000 + seed, 500, 100, 300)
    img = K.make_image(400 + seed, 0, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        x = K.make_x(400 + seed, 1, B, C)
        xq = np.zeros((B, C), dtype=np.int8)
        dx = np.zeros((B, C // 32), dtype=np.float32)
        for t in range(B):
            xq[t], dx[t] = O.quantize_q8(x[t])
        y = torch.empty((B, R), dtype=torch.float32, device="cuda")
        Q.qmv_gemm_q8(h, K.dev(xq), K.dev(dx), y)
        torch.cuda.synchronize()
        ref, bound = O.gemm_q8act(img, wt, sf, R, C, xq, dx, threads=K.THREADS)
        ok, worst = O.q8act_within_tolerance(y.cpu().numpy(), ref, bound, C)
        assert ok, (wt, sf, R, C, B, worst)
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("seed", range(20))
def test_random_batched_classifier(seed):
    """Q8_0 with f16 scales, 512 or 1024 columns, batches above 8: the
    f16 matrix-core path, with rows that end mid-tile and token counts that
    end mid-pass."""
    g = np.random.default_rng(7000 + seed)
    C = int(g.choice([512, 1024]))
    R = int(g.integers(1, 5000))
    B = int(g.integers(9, 200))
    img = K.make_image(500 + seed, 0, K.Q8, 1, R, C)
    h = K.upload(img, K.Q8, 1, R, C)
    try:
        x = K.make_x(500 + seed, 1, B, C)
        ref, norm = O.product(img, K.Q8, 1, R, C, x, threads=K.THREADS)
        ok, worst = O.within_tolerance(K.gpu_gemv(h, x), ref, norm)
        assert ok, (R, C, B, worst)
    finally:
        Q.qmv_destroy(h)
