"""Pins of the oracle's gated feed-forward output h = act(W1 x) * (W3 x)
(the .mlb page's header field "act": code 0 selects SiLU, code 1 the tanh
form of GELU; w1 = gate, w3 = up in its body table).

The activations are pinned to facts outside the oracle's own formulas:
library routines (scipy's logistic function and normal CDF), the identity
f(a) - f(-a) = a that both gates a * s(a) satisfy because s(a) + s(-a) = 1,
a closed value (sigmoid(ln 3) = 3/4), and the published size of the tanh
approximation's deviation from the exact GELU.  The gated product is pinned
against numpy matrix products of the dequantized weights."""
import math

import numpy as np
import pytest
from scipy.special import expit, ndtr

import cases as K
import oracle as O


def test_silu_library_closed_form_and_identity():
    a = np.linspace(-60, 60, 2401)
    s = np.array([O.ffn_act(v, O.ACT_SILU) for v in a])
    assert np.allclose(s, a * expit(a), rtol=1e-14, atol=1e-300)
    sm = np.array([O.ffn_act(-v, O.ACT_SILU) for v in a])
    assert np.allclose(s - sm, a, rtol=1e-13, atol=1e-13)
    assert O.ffn_act(math.log(3.0), O.ACT_SILU) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert O.ffn_act(0.0, O.ACT_SILU) == 0.0
    assert O.ffn_act(-800.0, O.ACT_SILU) == 0.0        # e^800 overflows: a / inf


def test_gelu_tanh_negative_tail_relative_accuracy():
    """Far in the negative tail the tanh form is a * e^(2u) to first order
    (u = sqrt(2/pi)(a + 0.044715 a^3)); the oracle keeps full relative
    precision there, where 1 + tanh(u) in binary64 is 0."""
    for a in (-6.0, -8.0, -12.0):
        u = math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3)
        tail = a * math.exp(2 * u)
        assert O.ffn_act(a, O.ACT_GELU_TANH) == pytest.approx(tail, rel=1e-9)
        assert O.ffn_act(a, O.ACT_GELU_TANH) != 0.0


def test_gelu_tanh_near_exact_gelu_and_identity():
    a = np.linspace(-12, 12, 4801)
    g = np.array([O.ffn_act(v, O.ACT_GELU_TANH) for v in a])
    dev = np.abs(g - a * ndtr(a))
    # the tanh form stays within 4.8e-4 of a * Phi(a) and is not Phi itself
    assert dev.max() <= 4.8e-4
    assert dev.max() >= 4.5e-4
    gm = np.array([O.ffn_act(-v, O.ACT_GELU_TANH) for v in a])
    assert np.allclose(g - gm, a, rtol=1e-13, atol=1e-13)
    assert O.ffn_act(0.0, O.ACT_GELU_TANH) == 0.0


@pytest.mark.parametrize("act", [O.ACT_SILU, O.ACT_GELU_TANH])
def test_lipschitz_constant_of_the_tolerance(act):
    """The gated tolerance uses L = 1.13 >= max |act'|; a finite-difference
    scan shows the bound holds and is not loose by more than 3%."""
    a = np.linspace(-20, 20, 40001)
    f = np.array([O.ffn_act(v, act) for v in a])
    slope = np.abs(np.diff(f) / np.diff(a))
    assert slope.max() <= O.ACT_LIPSCHITZ
    assert slope.max() >= O.ACT_LIPSCHITZ - 0.035


@pytest.mark.parametrize("act", [O.ACT_SILU, O.ACT_GELU_TANH])
@pytest.mark.parametrize("wt,sf", [(K.Q4, 1), (K.Q8, 1)])
def test_gated_against_numpy_products(act, wt, sf):
    """f16 scales, so the float32 dequantized weights are the exact ones."""
    R, C, B = 23, 128, 3
    img1 = K.make_image(71, 1, wt, sf, R, C)
    img3 = K.make_image(71, 3, wt, sf, R, C)
    x = K.make_x(71, 5, B, C)
    h, y1, n1, y3, n3 = O.gated(img1, img3, wt, sf, R, C, x, act)
    ids = np.arange(R, dtype=np.int64)
    W1 = O.dequant_rows(img1, wt, sf, R, C, ids).astype(np.float64)
    W3 = O.dequant_rows(img3, wt, sf, R, C, ids).astype(np.float64)
    z1 = x.astype(np.float64) @ W1.T
    z3 = x.astype(np.float64) @ W3.T
    if act == O.ACT_SILU:
        gate = z1 * expit(z1)
    else:   # within the tanh form's distance from a * Phi(a)
        gate = z1 * ndtr(z1)
    tol = 1e-12 if act == O.ACT_SILU else 4.8e-4
    assert np.allclose(h, gate * z3, rtol=1e-12, atol=tol * np.abs(z3).max())
    assert np.allclose(y1, z1, rtol=1e-12, atol=1e-12)
    assert np.allclose(y3, z3, rtol=1e-12, atol=1e-12)
    assert np.allclose(n1, np.abs(x.astype(np.float64)) @ np.abs(W1).T, rtol=1e-12)
    # swapping the matrices changes the result (gate and up are not symmetric)
    hs = O.gated(img3, img1, wt, sf, R, C, x, act)[0]
    assert not np.allclose(hs, h)


def test_gated_tolerance_predicate():
    """Accepts the exact value and errors inside the propagated bound;
    rejects NaN and an error of twice the bound."""
    y1 = np.array([[1.5, -3.0, 0.0]])
    y3 = np.array([[2.0, 0.5, -4.0]])
    n1 = np.array([[10.0, 10.0, 10.0]])
    n3 = np.array([[5.0, 5.0, 5.0]])
    href = np.array([[O.ffn_act(a, 0) * b for a, b in zip(y1[0], y3[0])]])
    assert O.gated_within_tolerance(href, href, y1, n1, y3, n3, 0)[0]
    e1, e3 = 2e-3 * n1, 2e-3 * n3
    a1 = np.abs([[O.ffn_act(a, 0) for a in y1[0]]])
    bound = O.ACT_LIPSCHITZ * e1 * (np.abs(y3) + e3) + a1 * e3
    assert O.gated_within_tolerance(href + 0.9 * bound, href, y1, n1, y3, n3, 0)[0]
    assert not O.gated_within_tolerance(href + 2.0 * bound, href, y1, n1, y3, n3, 0)[0]
    bad = href.copy()
    bad[0, 1] = np.nan
    assert not O.gated_within_tolerance(bad, href, y1, n1, y3, n3, 0)[0]
