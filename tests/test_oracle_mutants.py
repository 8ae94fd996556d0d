"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source, plants one mistake by text
substitution, compiles the copy (on the CPU) and runs every pin of
test_oracle.py against it; at least one pin must fail.  The committed oracle
itself is never changed."""
import subprocess

import numpy as np
import pytest

import oracle as O
import test_oracle as P

MUTANTS = [
    ("nibbles swapped",
     "(j < 16) ? (byte & 0xF) : (byte >> 4)", "(j < 16) ? (byte >> 4) : (byte & 0xF)"),
    ("Q4 offset 8 dropped", "return nib - 8;", "return nib;"),
    ("Q8 read unsigned", "(int)(int8_t)img[r * cols + c]", "(int)img[r * cols + c]"),
    ("Q8 row stride wrong", "(int)(int8_t)img[r * cols + c]", "(int)(int8_t)img[r * 32 + c]"),
    ("scales in column-major block order",
     "r * (cols / 32) + c / 32);\n                double w",
     "(c / 32) * rows + r);\n                double w"),
    ("padding to 32", "((n + 63) / 64) * 64", "((n + 31) / 32) * 32"),
    ("f16 exponent bias", "e - 25", "e - 24"),
    ("f16 subnormal scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("-128 not rejected", "if (img[i] == 0x80) return ORC_FORMAT;", "(void)0;"),
    ("norm without absolute values", "nrm += fabs(w) * fabs(a);", "nrm += w * a;"),
    ("quantizer divides last",
     "volatile float t = xb[j] * id;", "volatile float t = (xb[j] * 127.0f) / amax;"),
    ("quantizer rounds half to even",
     "float tr = truncf(u);", "float tr = rintf(t);"),
    ("quantizer threshold", "if (amax < 1e-30f)", "if (amax <= 0.0f)"),
    ("quantizer scale 1/128", "d[b] = amax / 127.0f;", "d[b] = amax / 128.0f;"),
    ("bf16 widened wrongly", "(uint32_t)b << 16", "(uint32_t)b << 15"),
    ("dequantized subnormals flushed",
     "float w = (float)v * d;",
     "float w = (float)v * d; if (fabsf(w) < 1.17549435e-38f) w = 0.0f;"),
    ("shared classifier ignored",
     "if (shared_classifier && (class_bit == 1 || class_bit == 2)) bits = 1u | 2u;",
     "(void)shared_classifier;"),
    ("block dot over 31 elements", "for (uint64_t j = 0; j < 32; ++j) {\n                acc +=",
     "for (uint64_t j = 0; j < 31; ++j) {\n                acc +="),
    ("limit 2^24 not enforced",
     "if (rows > ORC_DIM_LIMIT || cols > ORC_DIM_LIMIT) return ORC_SHAPE;", ""),
]


def _pins():
    out = []
    for n in P.FIXTURES_W:
        out.append((P.test_fixture_dequantized_values, (n,)))
    for n in P.FIXTURES_Y:
        out.append((P.test_fixture_products, (n,)))
    out += [(P.test_fixture_product_bf16_activations, ()),
            (P.test_quantizer_fixture, ()),
            (P.test_quantizer_properties, ()),
            (P.test_sizes_printed_on_pages, ()),
            (P.test_rejects_fixture, ()),
            (P.test_class_rule_hand_cases, ()),
            (P.test_block_dots_hand_and_brute_force, ()),
            (P.test_product_invariants, ())]
    for wt, sf in [(1, 0), (2, 1)]:
        out.append((P.test_product_exact_rational_brute_force, (wt, sf)))
    return out


def test_f16_decoder_mutant_fails_exhaustive_check(tmp_path, monkeypatch):
    _install(tmp_path, monkeypatch, "e - 25", "e - 24")
    with pytest.raises(AssertionError):
        P.test_f16_decoder_exhaustive_against_numpy()


def _install(tmp_path, monkeypatch, old, new):
    src = open(O._SRC).read()
    assert src.count(old) >= 1, old
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC",
                           "-shared", "-o", str(so), str(path), "-lm"])
    monkeypatch.setattr(O, "_lib", None)
    monkeypatch.setattr(O, "_LIB_PATH", str(so))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    _install(tmp_path, monkeypatch, old, new)
    failed = []
    for fn, args in _pins():
        try:
            fn(*args)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            failed.append(fn.__name__)
    assert failed, f"no pin catches: {name}"


# ---- the GGUF reader and the weight writer ----------------------------------

import test_oracle_writer_gguf as W  # noqa: E402

MUTANTS_WG = [
    ("gguf quants read from the scale", "memcpy(img + k * qb, b + 2, qb);",
     "memcpy(img + k * qb, b, qb);"),
    ("gguf Q8 block of 32 bytes", "uint64_t bsize = (wtype == ORC_Q8_0) ? 34 : 18;",
     "uint64_t bsize = (wtype == ORC_Q8_0) ? 32 : 18;"),
    ("gguf -128 not rejected", "if (src[34 * k + 2 + j] == 0x80) return ORC_FORMAT;", "(void)0;"),
    ("writer f16 quants against the unrounded scale", "float id = 1.0f / d16;",
     "float id = 127.0f / amax;"),
    ("writer f16 overflow not refused",
     "if ((dbits16 & 0x7FFFu) >= 0x7C00u) return ORC_FORMAT; /* > 65504 */", ""),
    ("writer Q4 unsigned maximum", "if (a > amax) { amax = a; mx = x[j]; }",
     "if (a > amax) { amax = a; mx = a; }"),
    ("writer Q4 offset 8.0", "float l0 = truncf(t0 + 8.5f), l1 = truncf(t1 + 8.5f);",
     "float l0 = truncf(t0 + 8.0f), l1 = truncf(t1 + 8.0f);"),
    ("writer Q4 nibbles swapped", "qb[j] = (uint8_t)((unsigned)l0 | ((unsigned)l1 << 4));",
     "qb[j] = (uint8_t)((unsigned)l1 | ((unsigned)l0 << 4));"),
    ("writer Q4 scale +8", "float d = mx / -8.0f;", "float d = mx / 8.0f;"),
    ("f16 rounding truncates", "if (rem > half || (rem == half && (q & 1u))) ++q;", "(void)0;"),
    ("f16 ties away from zero", "if (rem > half || (rem == half && (q & 1u))) ++q;",
     "if (rem >= half) ++q;"),
]


def _pins_wg():
    return [(W.test_gguf_sizes_printed_on_page, ()), (W.test_gguf_hand_built_blocks, ()),
            (W.test_gguf_round_trip_is_the_two_array_image, (O.Q8_0,)),
            (W.test_gguf_round_trip_is_the_two_array_image, (O.Q4_0,)),
            (W.test_gguf_checks, ()), (W.test_f16_rounding_matches_numpy, ()),
            (W.test_q8_f32_writer_is_the_activation_quantizer, ()),
            (W.test_q8_f16_writer_closed_forms, ()), (W.test_q8_f16_writer_properties, ()),
            (W.test_q4_round_writer_exact_recovery, ()), (W.test_q4_round_writer_properties, ())]


@pytest.mark.parametrize("name,old,new", MUTANTS_WG, ids=[m[0] for m in MUTANTS_WG])
def test_planted_writer_or_gguf_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    _install(tmp_path, monkeypatch, old, new)
    failed = []
    for fn, args in _pins_wg():
        try:
            fn(*args)
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(fn.__name__)
    assert failed, f"no pin catches: {name}"


# ---- the gated feed-forward output ------------------------------------------

import test_oracle_gated as G  # noqa: E402

MUTANTS_G = [
    ("SiLU with e^+a", "return a / (1.0 + exp(-a));", "return a / (1.0 + exp(a));"),
    ("GELU cubic coefficient", "0.044715 * a * a * a", "0.44715 * a * a * a"),
    ("GELU with e^-u", "return a / (1.0 + exp(-2.0 * u));", "return a / (1.0 + exp(-u));"),
    ("GELU constant 2/pi", "sqrt(2.0 / 3.14159265358979323846)", "(2.0 / 3.14159265358979323846)"),
    ("gate taken from the up projection", "orc_ffn_act(y1[i], act) * y3[i]",
     "orc_ffn_act(y3[i], act) * y1[i]"),
]


def _pins_g():
    out = [(G.test_silu_library_closed_form_and_identity, ()),
           (G.test_gelu_tanh_near_exact_gelu_and_identity, ())]
    for act in (0, 1):
        out.append((G.test_lipschitz_constant_of_the_tolerance, (act,)))
        for wt, sf in ((2, 1), (1, 1)):
            out.append((G.test_gated_against_numpy_products, (act, wt, sf)))
    return out


@pytest.mark.parametrize("name,old,new", MUTANTS_G, ids=[m[0] for m in MUTANTS_G])
def test_planted_gated_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    _install(tmp_path, monkeypatch, old, new)
    failed = []
    for fn, args in _pins_g():
        try:
            fn(*args)
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(fn.__name__)
    assert failed, f"no pin catches: {name}"


# ---- the Q4_0 least-squares writer ------------------------------------------

import test_oracle_q4_search as S  # noqa: E402

MUTANTS_S = [
    ("candidate step 0.25", "-6.2f, -6.4f, -6.6f", "-6.25f, -6.4f, -6.6f"),
    ("12 candidates", "for (int i = 0; i < 13; ++i) {\n                orc_lsq_levels",
     "for (int i = 0; i < 12; ++i) {\n                orc_lsq_levels"),
    ("weights |x| instead of x^2", "wt[j] = v[j] * v[j];", "wt[j] = fabsf(v[j]);"),
    ("levels truncated", "float t = rintf(v[j] * iscale);", "float t = truncf(v[j] * iscale);"),
    ("levels clamped to 8", "if (t > 7.0f) t = 7.0f;", "if (t > 8.0f) t = 8.0f;"),
    ("tiny threshold 1e-7", "const int tiny = amax < 1e-6f;", "const int tiny = amax < 1e-7f;"),
    ("tiny d not scaled back", "if (tiny) d = d * amax;", "(void)0;"),
    ("largest error wins", "if (i == 0 || e < best_e) {", "if (i == 0 || e > best_e) {"),
    ("unweighted fit", "sxl += cube[j] * l[j];\n                    sll += wt[j] * (l[j] * l[j]);",
     "sxl += v[j] * l[j];\n                    sll += l[j] * l[j];"),
]


def _pins_s():
    return [(S.test_exact_blocks_are_recovered, ()), (S.test_zero_block_and_sign_of_d, ()),
            (S.test_brute_force_minimum_and_normal_equation, ()),
            (S.test_no_worse_than_the_round_rule, ()), (S.test_tiny_blocks_are_scaled_up, ()),
            (S.test_f16_scales_and_refusals, ()), (S.test_scaling_threshold_is_1e_minus_6, ())]


@pytest.mark.parametrize("name,old,new", MUTANTS_S, ids=[m[0] for m in MUTANTS_S])
def test_planted_search_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    _install(tmp_path, monkeypatch, old, new)
    failed = []
    for fn, args in _pins_s():
        try:
            fn(*args)
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(fn.__name__)
    assert failed, f"no pin catches: {name}"


# ---- the product on Q8_0-quantized activations -------------------------------

import test_oracle_q8act as A8  # noqa: E402

MUTANTS_A = [
    ("activation scale of token 0", "(double)dx[t * nb + b]", "(double)dx[b]"),
    ("next block's weight scale", "orc_scale(img, span[1], scale_f16, r * nb + b)",
     "orc_scale(img, span[1], scale_f16, r * nb + (b + 1) % nb)"),
    ("bound without absolute values", "bnd += fabs(term);", "bnd += term;"),
    ("activation quants unsigned", "(int32_t)xq[t * cols + 32 * b + j]",
     "(int32_t)(uint8_t)xq[t * cols + 32 * b + j]"),
    ("block of 31", "for (uint64_t j = 0; j < 32; ++j)\n                    sb +=",
     "for (uint64_t j = 0; j < 31; ++j)\n                    sb +="),
]


def _pins_a():
    out = [(A8.test_quantized_activations_stay_within_the_quantizer_bound, ())]
    for wt in (2, 1):
        out.append((A8.test_exact_rationals, (wt,)))
    for wt, sf in ((2, 1), (1, 0)):
        out.append((A8.test_power_of_two_scales_equal_the_plain_product, (wt, sf)))
    return out


@pytest.mark.parametrize("name,old,new", MUTANTS_A, ids=[m[0] for m in MUTANTS_A])
def test_planted_q8act_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    _install(tmp_path, monkeypatch, old, new)
    failed = []
    for fn, args in _pins_a():
        try:
            fn(*args)
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(fn.__name__)
    assert failed, f"no pin catches: {name}"
