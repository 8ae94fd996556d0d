"""Pins of the oracle's product on Q8_0-quantized activations (the .mlb
page's CPU path: activations quantized per block by the "Quantization rule",
then per-block integer dot products combined with the two scales).

Pinned against: exact rational arithmetic from the bit patterns, the pinned
float64 product when the activation scales are powers of two (then
xq * dx is exact in float32), and the quantizer's error bound against the
product on the original activations."""
from fractions import Fraction

import numpy as np
import pytest

import cases as K
import oracle as O


@pytest.mark.parametrize("wt", [K.Q4, K.Q8])
def test_exact_rationals(wt):
    R, C, B = 5, 96, 3
    img = K.make_image(90, wt, wt, 1, R, C)       # f16 scales: fl32(v d) is exact
    g = np.random.default_rng(90 + wt)
    xq = g.integers(-127, 128, (B, C)).astype(np.int8)
    dx = g.uniform(1e-3, 1e-1, (B, C // 32)).astype(np.float32)
    ref, bound = O.gemm_q8act(img, wt, 1, R, C, xq, dx)
    W = O.dequant_rows(img, wt, 1, R, C, np.arange(R, dtype=np.int64))
    for t in range(B):
        for r in range(R):
            exact = Fraction(0)
            absum = Fraction(0)
            for b in range(C // 32):
                sb = sum(Fraction(float(W[r, 32 * b + j])) * int(xq[t, 32 * b + j])
                         for j in range(32))
                term = sb * Fraction(float(dx[t, b]))
                exact += term
                absum += abs(term)
            assert abs(Fraction(ref[t, r]) - exact) <= Fraction(1, 2 ** 50) * absum
            assert abs(Fraction(bound[t, r]) - absum) <= Fraction(1, 2 ** 50) * absum


@pytest.mark.parametrize("wt,sf", [(K.Q4, 1), (K.Q8, 0)])
def test_power_of_two_scales_equal_the_plain_product(wt, sf):
    R, C, B = 40, 256, 4
    img = K.make_image(91, wt, wt, sf, R, C)
    g = np.random.default_rng(91)
    xq = g.integers(-127, 128, (B, C)).astype(np.int8)
    dx = np.float32(2.0) ** g.integers(-20, 4, (B, C // 32)).astype(np.float32)
    x = (xq.astype(np.float32) * np.repeat(dx, 32, axis=1)).astype(np.float32)
    ref, bound = O.gemm_q8act(img, wt, sf, R, C, xq, dx)
    ref2, norm = O.product(img, wt, sf, R, C, x)
    assert np.all(np.abs(ref - ref2) <= 1e-13 * norm)
    assert np.all(bound <= norm * (1 + 1e-12))
    assert np.all(np.abs(ref) <= bound * (1 + 1e-12))


def test_quantized_activations_stay_within_the_quantizer_bound():
    """With xq, dx from the quantizer, the result differs from the product on
    the original activations by at most sum_b |w| dx_b (0.5 + 1e-4)."""
    R, C = 30, 512
    img = K.make_image(92, K.Q4, K.Q4, 1, R, C)
    x = K.make_x(92, 1, 2, C)
    xq = np.zeros(x.shape, dtype=np.int8)
    dx = np.zeros((2, C // 32), dtype=np.float32)
    for t in range(2):
        q, d = O.quantize_q8(x[t])
        xq[t], dx[t] = q, d
    ref, _ = O.gemm_q8act(img, K.Q4, 1, R, C, xq, dx)
    ref_x, _ = O.product(img, K.Q4, 1, R, C, x)
    W = np.abs(O.dequant_rows(img, K.Q4, 1, R, C, np.arange(R, dtype=np.int64)).astype(np.float64))
    for t in range(2):
        lim = W @ (np.repeat(dx[t].astype(np.float64), 32) * (0.5 + 1e-4))
        assert np.all(np.abs(ref[t] - ref_x[t]) <= lim)
        assert np.any(ref[t] != ref_x[t])          # the quantization does change it


def test_tolerance_predicate():
    ref = np.array([[1.0, -2.0]])
    bound = np.array([[10.0, 4.0]])
    tol = (128 // 32 + 2) * 2.0 ** -23 * bound
    assert O.q8act_within_tolerance(ref + 0.9 * tol, ref, bound, 128)[0]
    assert not O.q8act_within_tolerance(ref + 2.0 * tol, ref, bound, 128)[0]
    assert not O.q8act_within_tolerance(np.array([[np.nan, -2.0]]), ref, bound, 128)[0]
