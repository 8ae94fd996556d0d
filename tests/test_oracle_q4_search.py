"""Pins of the oracle's Q4_0 least-squares writer (the .mlb page's paragraph
on fitting each Q4_0 block: the largest element mapped to 13 candidate
levels -6.0 .. -8.4, d the x^2-weighted least-squares fit, the smallest
weighted error wins, blocks below 1e-6 scaled up first).

The pins come from outside the oracle's own arithmetic: blocks that are
exactly d times integer levels (recovered exactly), a numpy brute force over
the 13 candidates in float64, the least-squares normal equation, comparison
with the round rule's error, exact power-of-two rescaling, and numpy's f16
rounding."""
import numpy as np
import pytest

import oracle as O


def split(img, rows, cols, sf16):
    """(levels [rows*cols/32][32] as nibble - 8, d as float64 [rows*cols/32])."""
    st, s = O.span(O.Q4_0, sf16, rows, cols)
    nb = rows * cols // 32
    q = img[:s["q_bytes"]].reshape(nb, 16)
    lv = np.concatenate([(q & 15).astype(np.int64), (q >> 4).astype(np.int64)], axis=1) - 8
    raw = img[s["d_offset"]:s["d_offset"] + s["d_bytes"]]
    d = raw.view(np.float16 if sf16 else np.float32).astype(np.float64)
    return lv, d


def weighted_error(x, d, lv):
    x = x.astype(np.float64)
    return np.sum(x * x * (x - d[:, None] * lv) ** 2, axis=1)


def brute_force(x):
    """Per block: the smallest float64 weighted error over the 13 candidates
    (levels from rint(x * L / mx) clamped to [-8, 7], d the weighted fit)."""
    out = []
    for b in x.astype(np.float64):
        a = np.abs(b)
        mx = b[int(np.argmax(a))]
        best = np.inf
        for i in range(13):
            L = -6.0 - 0.2 * i
            lv = np.clip(np.rint(b * (L / mx)), -8, 7)
            w = b * b
            d = np.sum(w * b * lv) / np.sum(w * lv * lv)
            best = min(best, float(np.sum(w * (b - d * lv) ** 2)))
        out.append(best)
    return np.array(out)


def test_exact_blocks_are_recovered():
    """x = d0 * l with integer levels l in [-8, 7] and l = -8 at the largest
    element: some candidate reproduces l with zero error, so the writer
    returns l and d0 exactly (a negative d0 makes the largest element
    positive; the levels are the same)."""
    g = np.random.default_rng(3)
    lv = g.integers(-8, 8, size=(40, 32))
    lv[:, 5] = -8
    for d0 in (0.5, -0.25, 3.0):
        x = (d0 * lv).astype(np.float32)
        st, img = O.quantize_q4_search(0, 40, 32, x)
        assert st == "ok"
        got_l, got_d = split(img, 40, 32, 0)
        assert np.array_equal(got_l, lv)
        assert np.all(got_d == d0)


def test_zero_block_and_sign_of_d():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1] = np.linspace(-1, 2, 32)              # largest element positive
    st, img = O.quantize_q4_search(0, 1, 64, x.reshape(1, 64))
    assert st == "ok"
    lv, d = split(img, 1, 64, 0)
    assert d[0] == 0 and np.all(lv[0] == 0)    # nibbles 8
    assert d[1] < 0 and lv[1, 31] in (-8, -7, -6)


def test_brute_force_minimum_and_normal_equation():
    g = np.random.default_rng(4)
    x = (g.standard_normal((300, 32)) * np.exp(g.uniform(-3, 3, (300, 1)))).astype(np.float32)
    x[::7, 3] *= 9                             # outliers
    st, img = O.quantize_q4_search(0, 300, 32, x)
    assert st == "ok"
    lv, d = split(img, 300, 32, 0)
    e = weighted_error(x, d, lv)
    best = brute_force(x)
    scale = np.sum(x.astype(np.float64) ** 4, axis=1)
    assert np.all(e <= best + 1e-6 * scale)
    # d solves the weighted normal equation for its levels
    xd = x.astype(np.float64)
    w = xd * xd
    resid = np.sum(w * (xd - d[:, None] * lv) * lv, axis=1)
    assert np.all(np.abs(resid) <= 1e-5 * np.sum(w * np.abs(xd * lv), axis=1))


def test_no_worse_than_the_round_rule():
    g = np.random.default_rng(5)
    x = g.standard_normal((50, 4096)).astype(np.float32)
    st, img = O.quantize_q4_search(0, 50, 4096, x)
    st2, img2 = O.quantize_weights(O.Q4_0, 0, 50, 4096, x)
    assert st == st2 == "ok"
    xb = x.reshape(-1, 32)
    ls, ds = split(img, 50, 4096, 0)
    lr, dr = split(img2, 50, 4096, 0)
    e_s = weighted_error(xb, ds, ls)
    e_r = weighted_error(xb, dr, lr)
    assert np.all(e_s <= e_r * (1 + 1e-5) + 1e-30)
    assert np.mean(e_s) < 0.9 * np.mean(e_r)   # and clearly better on average


def test_tiny_blocks_are_scaled_up():
    """A block whose largest magnitude is 1, and the same block times 2^-40
    (below 1e-6): identical nibbles, d scaled by exactly 2^-40."""
    g = np.random.default_rng(6)
    x = g.uniform(-1, 1, (20, 32)).astype(np.float32)
    x[:, 0] = -1.0
    st, a = O.quantize_q4_search(0, 20, 32, x)
    st2, b = O.quantize_q4_search(0, 20, 32, x * np.float32(2.0 ** -40))
    assert st == st2 == "ok"
    la, da = split(a, 20, 32, 0)
    lb, db = split(b, 20, 32, 0)
    assert np.array_equal(la, lb)
    assert np.array_equal(db, da * 2.0 ** -40)


def test_f16_scales_and_refusals():
    g = np.random.default_rng(7)
    x = (g.standard_normal((8, 64)) * 30).astype(np.float32)
    st, a = O.quantize_q4_search(0, 8, 64, x)
    st2, b = O.quantize_q4_search(1, 8, 64, x)
    assert st == st2 == "ok"
    la, da = split(a, 8, 64, 0)
    lb, db = split(b, 8, 64, 1)
    assert np.array_equal(la, lb)
    assert np.array_equal(db, da.astype(np.float32).astype(np.float16).astype(np.float64))
    big = x.copy()
    big[0, 0] = 9e5                            # d near -1.1e5: no f16 holds it
    assert O.quantize_q4_search(1, 8, 64, big)[0] == "format"
    assert O.quantize_q4_search(0, 8, 64, big)[0] == "ok"
    huge = x.copy()
    huge[3, 40] = 1e13                         # cubes overflow float32
    assert O.quantize_q4_search(0, 8, 64, huge)[0] == "format"


def test_scaling_threshold_is_1e_minus_6():
    """Blocks with largest magnitude between 1e-7 and 1e-6 are fitted as
    the block divided by that magnitude, d multiplied back; at 2e-6 they
    are fitted as they are (the same as with no scaling rule)."""
    g = np.random.default_rng(8)
    base = g.standard_normal((64, 32)).astype(np.float32)
    for c, scaled in ((3.7e-7, True), (2.3e-6, False)):
        xt = (base * np.float32(c / np.abs(base).max())).astype(np.float32)
        amax = np.abs(xt).max(axis=1)
        st, img = O.quantize_q4_search(0, 64, 32, xt)
        assert st == "ok"
        lt, dt = split(img, 64, 32, 0)
        v = (xt / amax[:, None]).astype(np.float32)
        st2, img2 = O.quantize_q4_search(0, 64, 32, v)
        lv, dv = split(img2, 64, 32, 0)
        expect = (dv.astype(np.float32) * amax).astype(np.float64)
        same = np.array_equal(lt, lv) and np.array_equal(dt, expect)
        assert same == scaled
