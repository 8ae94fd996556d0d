"""Pins of the oracle's GGUF block reader and weight writer to facts that do
not come from the oracle: the byte counts the minfer GGUF page prints, hand-
built blocks, byte-exact round trips through independently packed data, the
page's own statement that the Q8_0 writer and the activation quantizer use
the same operations, numpy's IEEE binary16 rounding, and closed forms of the
writer rules on blocks built so that the answer is known."""
import numpy as np
import pytest

import oracle as O

Q8, Q4 = O.Q8_0, O.Q4_0


def pack_gguf(wt, q, d16):
    """BlockQ4_0 / BlockQ8_0 records (f16 scale, then the block's quant
    bytes) from per-row quant bytes and f16 scale bits - written here, apart
    from the oracle."""
    qb = np.ascontiguousarray(q).view(np.uint8).reshape(-1)
    per = 32 if wt == Q8 else 16
    nblk = qb.size // per
    rec = np.zeros((nblk, 2 + per), dtype=np.uint8)
    rec[:, 0:2] = np.ascontiguousarray(d16, dtype=np.uint16).reshape(-1, 1).view(np.uint8)
    rec[:, 2:] = qb.reshape(nblk, per)
    return rec.reshape(-1)


# ---- GGUF ----------------------------------------------------------------

def test_gguf_sizes_printed_on_page():
    # minfer "GGUF load" page, section 3.2 (g): output.weight Q8_0 151936 x 896
    # is 144,643,072 bytes; token_embd.weight Q4_0 of the same shape follows
    # and the next tensor starts at 221,218,816.  Section 2.4: an 896-wide
    # Q4_0 row is 28 blocks x 18 bytes = 504 bytes.
    assert O.gguf_span(Q8, 151936, 896) == ("ok", 144_643_072)
    assert O.gguf_span(Q4, 151936, 896) == ("ok", 76_575_744)
    assert 144_643_072 + O.gguf_span(Q4, 151936, 896)[1] == 221_218_816
    assert O.gguf_span(Q4, 1, 896) == ("ok", 504)
    assert O.gguf_span(Q4, 4, 33)[0] == "shape"
    assert O.gguf_span(3, 4, 32)[0] == "format"


def test_gguf_hand_built_blocks():
    # one Q4_0 row of 64 weights: block 0 scale 0.5 (f16 0x3800), block 1
    # scale -2 (0xC000); quant byte j of block 0 is (j << 4) | (15 - j)
    d16 = np.array([0x3800, 0xC000], dtype=np.uint16)
    q = np.zeros(32, dtype=np.uint8)
    q[:16] = [(j << 4) | (15 - j) for j in range(16)]
    q[16:] = 0x81                              # low 1, high 8 in every byte
    img = O.gguf_to_image(Q4, 1, 64, pack_gguf(Q4, q, d16))
    w = O.dequant_rows(img, Q4, 1, 1, 64, np.array([0]))[0]
    want = [((15 - j) - 8) * 0.5 for j in range(16)] + [(j - 8) * 0.5 for j in range(16)]
    want += [(1 - 8) * -2.0] * 16 + [(8 - 8) * -2.0] * 16
    assert w.tolist() == want
    # one Q8_0 block: scale 0.25 (0x3400), quants -127 .. 127 step 8 and more
    qq = np.array([-127 + 8 * j for j in range(32)], dtype=np.int8)
    img = O.gguf_to_image(Q8, 1, 32, pack_gguf(Q8, qq, np.array([0x3400], np.uint16)))
    w = O.dequant_rows(img, Q8, 1, 1, 32, np.array([0]))[0]
    assert w.tolist() == [(-127 + 8 * j) * 0.25 for j in range(32)]


@pytest.mark.parametrize("wt", [Q8, Q4])
def test_gguf_round_trip_is_the_two_array_image(wt):
    g = np.random.default_rng(3)
    R, C = 7, 96
    if wt == Q8:
        q = g.integers(-127, 128, size=(R, C)).astype(np.int8)
    else:
        q = g.integers(0, 256, size=(R, C // 2)).astype(np.uint8)
    d = g.uniform(-4, 4, size=R * C // 32).astype(np.float16)
    img = O.gguf_to_image(wt, R, C, pack_gguf(wt, q, d.view(np.uint16)))
    assert np.array_equal(img, O.layout(wt, 1, R, C, q, d))


def test_gguf_checks():
    R, C = 3, 64
    q = np.ones((R, C), dtype=np.int8)
    blob = pack_gguf(Q8, q, np.full(R * 2, 0x3C00, np.uint16))
    assert O.check_gguf(Q8, R, C, blob) == "ok"
    assert O.check_gguf(Q8, R, C, blob, blob.size - 1) == "format"
    bad = blob.copy()
    bad[34 * 4 + 2 + 31] = 0x80              # last quant of block 4
    assert O.check_gguf(Q8, R, C, bad) == "format"
    bad = blob.copy()
    bad[34 * 4] = 0x80                       # a scale byte of 0x80 is fine
    assert O.check_gguf(Q8, R, C, bad) == "ok"
    q4 = np.full((R, C // 2), 0x80, dtype=np.uint8)   # Q4_0: every byte legal
    assert O.check_gguf(Q4, R, C, pack_gguf(Q4, q4, np.zeros(R * 2, np.uint16))) == "ok"


# ---- weight writer ---------------------------------------------------------

def split_image(img, wt, sf, R, C):
    st, s = O.span(wt, sf, R, C)
    q = img[:s["q_bytes"]]
    d = img[s["d_offset"]:s["d_offset"] + s["d_bytes"]].view(np.float16 if sf else np.float32)
    return (q.view(np.int8) if wt == Q8 else q), d, s


def test_f16_rounding_matches_numpy():
    g = np.random.default_rng(5)
    x = (g.standard_normal(50000) * np.exp(g.uniform(-35, 13, 50000))).astype(np.float32)
    x = np.concatenate([x, np.float32([65504, 65519.99, 65520, 65536, 2.0 ** -24, 2.0 ** -25,
                                       2.0 ** -25 * 1.0000001, 6.1e-5, -0.0, 0.0])])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([O.f16_bits(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_q8_f32_writer_is_the_activation_quantizer():
    # the .mlb page, "Quantization rule": the Q8_0 writer and the runtime's
    # activation quantizer share the same float32 steps
    g = np.random.default_rng(7)
    R, C = 9, 256
    w = (g.standard_normal((R, C)) * np.exp(g.uniform(-80, 30, (R, 1)))).astype(np.float32)
    w[0, :32] = 0
    w[1, :32] = 1e-31
    st, img = O.quantize_weights(Q8, 0, R, C, w)
    assert st == "ok"
    q, d, _ = split_image(img, Q8, 0, R, C)
    q_ref, d_ref = O.quantize_q8(w.reshape(-1))
    assert np.array_equal(q, q_ref)
    assert np.array_equal(d.view(np.uint32), d_ref.view(np.uint32))


def test_q8_f16_writer_closed_forms():
    # amax = 127 / 16: d = 1/16 exactly in f32 and f16, so q is x * 16 rounded
    # half away from zero
    x = np.zeros(32, dtype=np.float32)
    x[:8] = [127 / 16, -127 / 16, 1 / 32, -1 / 32, 3 / 32, -3 / 32, 0.5, 0.0]
    st, img = O.quantize_weights(Q8, 1, 1, 32, x)
    q, d, _ = split_image(img, Q8, 1, 1, 32)
    assert d.tolist() == [1 / 16]
    assert q[:8].tolist() == [127, -127, 1, -1, 2, -2, 8, 0]
    # the largest storable scale, and the first one that is not
    ok = np.full(32, 127 * 65504.0, dtype=np.float32)
    assert O.quantize_weights(Q8, 1, 1, 32, ok)[0] == "ok"
    big = np.full(32, 127 * 65536.0, dtype=np.float32)
    assert O.quantize_weights(Q8, 1, 1, 32, big) == ("format", None)
    assert O.quantize_weights(Q8, 0, 1, 32, big)[0] == "ok"       # f32 scales store it
    # below 1e-30 the block is zero
    tiny = np.full(32, 9e-31, dtype=np.float32)
    st, img = O.quantize_weights(Q8, 1, 1, 32, tiny)
    q, d, _ = split_image(img, Q8, 1, 1, 32)
    assert d.tolist() == [0.0] and not q.any()


def test_q8_f16_writer_properties():
    g = np.random.default_rng(11)
    R, C = 64, 512
    w = (g.standard_normal((R, C)) * np.exp(g.uniform(-12, 9, (R, 1)))).astype(np.float32)
    st, img = O.quantize_weights(Q8, 1, R, C, w)
    assert st == "ok"
    q, d, _ = split_image(img, Q8, 1, R, C)
    blocks = w.reshape(-1, 32)
    amax = np.abs(blocks).max(axis=1)
    # the scale is amax / 127 (float32) rounded to f16 by numpy
    assert np.array_equal(d.view(np.uint16), (amax / np.float32(127)).astype(np.float16).view(np.uint16))
    # every weight is within half a step of its value, unless clamped
    dq = q.reshape(-1, 32).astype(np.float64) * d.astype(np.float64)[:, None]
    err = np.abs(dq - blocks)
    ratio = np.abs(blocks) / d.astype(np.float64)[:, None]
    free = ratio < 126.5
    assert np.all(err[free] <= d.astype(np.float64).repeat(32).reshape(-1, 32)[free] * (0.5 + 1e-6))
    assert np.abs(q).max() <= 127


def test_q4_round_writer_exact_recovery():
    # x = k * c with integer k in [-8, 7] and the largest magnitude at k = -8:
    # d = -8c / -8 = c and every nibble is k + 8
    g = np.random.default_rng(13)
    for sign in (1, -1):
        k = g.integers(-7, 8, size=32)
        k[5] = -8
        c = np.float32(0.375) * sign
        x = (k * c).astype(np.float32)
        for sf in (0, 1):
            st, img = O.quantize_weights(Q4, sf, 1, 32, x)
            q, d, _ = split_image(img, Q4, sf, 1, 32)
            nib = np.concatenate([q & 15, q >> 4]).astype(int)
            # the largest magnitude is -8c, so d = c (negative when c is) and
            # x / d = k in both cases
            assert d.tolist() == [0.375 * sign] and nib.tolist() == (k + 8).tolist()
    # a block so small that 1 / d overflows writes as zeros: nibbles 8
    tiny = np.full(32, 1e-40, dtype=np.float32)
    st, img = O.quantize_weights(Q4, 0, 1, 32, tiny)
    q, d, _ = split_image(img, Q4, 0, 1, 32)
    assert d.tolist() == [np.float32(1e-40) / np.float32(-8)] and set(q.tolist()) == {0x88}
    # an all-zero block: d = -0.0 (0 / -8), every nibble 8, every weight 0
    st, img = O.quantize_weights(Q4, 0, 1, 32, np.zeros(32, np.float32))
    q, d, _ = split_image(img, Q4, 0, 1, 32)
    assert d.view(np.uint32).tolist() == [0x80000000] and set(q.tolist()) == {0x88}


def test_q4_round_writer_properties():
    g = np.random.default_rng(17)
    R, C = 64, 512
    w = (g.standard_normal((R, C)) * np.exp(g.uniform(-10, 8, (R, 1)))).astype(np.float32)
    for sf in (0, 1):
        st, img = O.quantize_weights(Q4, sf, R, C, w)
        assert st == "ok"
        q, d, _ = split_image(img, Q4, sf, R, C)
        blocks = w.reshape(-1, 32)
        qb = q.reshape(-1, 16)
        nib = np.concatenate([qb & 15, qb >> 4], axis=1).astype(np.int64)
        idx = np.abs(blocks).argmax(axis=1)              # first largest magnitude
        mx = blocks[np.arange(blocks.shape[0]), idx]
        d32 = mx / np.float32(-8)
        if sf:
            assert np.array_equal(d.view(np.uint16), d32.astype(np.float16).view(np.uint16))
        else:
            assert np.array_equal(d.view(np.uint32), d32.view(np.uint32))
        assert np.all(nib[np.arange(nib.shape[0]), idx] == 0)   # the largest maps to -8
        # within half a step (of the float32 d) unless clamped at 15
        t = blocks.astype(np.float64) / d32.astype(np.float64)[:, None]
        err = np.abs((nib - 8) - t)
        assert np.all(err[nib < 15] <= 0.5 + 1e-5)
        assert np.all(t[nib == 15] >= 6.5 - 1e-5)
