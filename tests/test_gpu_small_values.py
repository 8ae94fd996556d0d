"""Decode kernels on activations far below their block's largest value, at
the parity bar |y - ref| <= 2e-3 * sum |w||x| per output (the .mlb page's
"Body" product; any finite activations are valid input).

Each block of 32 holds one value 1.0, a number of values far below 1.0
and zeros; the weight that meets the 1.0 is zero, so the output is carried
by the far smaller values alone and any loss of them shows at full size.
The count of such values per block varies from 1 to 31, and they include
"small" ones (below 2^-20 of the block's largest, whose products the kernels
add in float32 after the digit sums), so the one-shot and the streaming
kernels take their small-value pass with up to 31 values per block.  A
second pattern puts values just above and just below that threshold, where
the fixed point keeps the fewest significant bits."""
import numpy as np
import pytest

import cases as K
import oracle as O
from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


COUNTS = [1, 2, 3, 5, 16, 31, 0, 2]


def small_pattern(B, C, seed, mags):
    """Block b of token t: 1.0 at position p (p = (b + t) % 32), then
    COUNTS[b % 8] values of magnitude drawn from mags at seeded positions,
    random signs; zeros elsewhere.  Returns x and the positions of the 1.0."""
    g = np.random.default_rng(seed)
    x = np.zeros((B, C), dtype=np.float32)
    big = np.zeros((B, C // 32), dtype=np.int64)
    for t in range(B):
        for b in range(C // 32):
            p = (b + t) % 32
            big[t, b] = p
            x[t, 32 * b + p] = 1.0
            n = COUNTS[b % len(COUNTS)]
            others = [j for j in range(32) if j != p]
            pos = g.choice(others, size=n, replace=False)
            vals = g.choice(mags, size=n) * g.choice([-1.0, 1.0], size=n)
            x[t, 32 * b + pos] = vals.astype(np.float32)
    return x, big


def zero_at(img, wt, sf, R, C, cols_zero, seed=0):
    """The image with code 0 (Q4_0 nibble 8) in every row at the columns
    cols_zero, seeded nonzero codes elsewhere, scales kept."""
    g = np.random.default_rng(seed + R + C)
    if wt == K.Q8:
        q = g.integers(1, 128, size=(R, C)).astype(np.int8) * g.choice([-1, 1], size=(R, C)).astype(np.int8)
        q[:, cols_zero] = 0
        qb = q.reshape(-1)
    else:
        nib = g.choice([0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15], size=(R, C)).astype(np.uint8)
        nib[:, cols_zero] = 8
        blk = nib.reshape(R, C // 32, 32)
        qb = (blk[:, :, :16] | (blk[:, :, 16:] << 4)).reshape(-1)
    st, s = O.span(wt, sf, R, C)
    d = img[s["d_offset"]:s["d_offset"] + s["d_bytes"]].copy().view(np.float16 if sf else np.float32)
    return O.layout(wt, sf, R, C, qb, d)


# (wtype, scale_f16, rows, cols): one-shot shapes, then shapes that take the
# streaming kernel (two steps of 64 chunks per row and at least 6144 tiles)
SHAPES = [(K.Q4, 1, 300, 4096), (K.Q8, 0, 300, 2048), (K.Q8, 1, 257, 1024),
          (K.Q4, 1, 12800, 4096), (K.Q8, 0, 12800, 2048)]


def check(y, ref, norm, what):
    ok, worst = O.within_tolerance(y, ref, norm, TOL)
    print(f"{what}: worst |y-ref|/norm = {worst:.3e}")
    assert ok, f"{what}: outside 2e-3 * norm (worst ratio {worst:.3e})"


@pytest.mark.parametrize("wt,sf,R,C", SHAPES)
@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("mags", [(1e-12, 1e-7, 3e-6, 2e-4), (9.0e-7, 9.5e-7, 9.6e-7, 1.05e-6)],
                         ids=["far", "threshold"])
def test_gemv_small_values(wt, sf, R, C, B, mags):
    x, big = small_pattern(B, C, 900 + R + B, np.array(mags))
    # the 1.0 of every token meets a zero weight: zero every column that
    # holds a 1.0 in some token
    cols = sorted({32 * b + int(big[t, b]) for t in range(B) for b in range(C // 32)})
    img = zero_at(K.make_image(901, 0, wt, sf, R, C), wt, sf, R, C, cols)
    h = K.upload(img, wt, sf, R, C)
    try:
        sel = K.sample_rows(R, 96, seed=R) if R > 600 else None
        y = K.gpu_gemv(h, x)
        ref, norm = O.product(img, wt, sf, R, C, x, sel=sel, threads=K.THREADS)
        check(y if sel is None else y[:, sel], ref, norm, f"gemv small {wt}/{sf} {R}x{C} b{B}")
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("act", [0, 1])
def test_gated_small_values_match_plain_products(act):
    """The gated launch (streaming kernel) and the two plain products
    (one-shot kernel) add the small values in the same order: the gate and
    up sums agree bit for bit, so the gated output equals act(z1) * z3 up
    to the activation's own rounding."""
    import torch
    wt, sf, R, C, B = K.Q4, 1, 2000, 4096, 2
    x, big = small_pattern(B, C, 950 + act, np.array([1e-7, 1e-5, 2e-4, 2.6e-4]))
    cols = sorted({32 * b + int(big[t, b]) for t in range(B) for b in range(C // 32)})
    img1 = zero_at(K.make_image(951, 1, wt, sf, R, C), wt, sf, R, C, cols, seed=1)
    img3 = zero_at(K.make_image(951, 3, wt, sf, R, C), wt, sf, R, C, cols, seed=3)
    h1, h3 = K.upload(img1, wt, sf, R, C), K.upload(img3, wt, sf, R, C)
    try:
        xd = K.dev(x)
        hd = torch.empty((B, R), dtype=torch.float32, device="cuda")
        Q.qmv_gemv_gated(h1, h3, xd, hd, act=act)
        torch.cuda.synchronize()
        hg = hd.cpu().numpy()
        z1, z3 = K.gpu_gemv(h1, x), K.gpu_gemv(h3, x)
        ref1, n1 = O.product(img1, wt, sf, R, C, x, threads=K.THREADS)
        ref3, n3 = O.product(img3, wt, sf, R, C, x, threads=K.THREADS)
        check(z1, ref1, n1, "w1 small")
        check(z3, ref3, n3, "w3 small")
        z = z1.astype(np.float64)
        with np.errstate(over="ignore"):
            a = np.vectorize(lambda v: O.ffn_act(v, act))(z)
        expect = a * z3.astype(np.float64)
        arg = np.abs(z) if act == 0 else 2 * np.abs(0.7978845608 * (z + 0.044715 * z ** 3))
        rel = 2.0 ** -20 * (1 + arg)
        floor = 2.0 ** -120 * (1 + np.abs(z * z3))
        assert np.all(np.abs(hg - expect) <= rel * np.abs(expect) + floor)
    finally:
        Q.qmv_destroy(h1)
        Q.qmv_destroy(h3)
