"""Python face of the plain CPU oracle (oracle/qmv_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are its only users.  Nothing in block_quant_weight_amd/
imports it, and it imports nothing from there.

The C file holds every rule, each cited there against Krafla's ".mlb model,
version 1" format page; this module only builds and loads it, marshals numpy
arrays, and lays out a matrix image (q array, zero pad to 64 bytes, d array)
from the oracle's own span arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqmv_oracle.so")
# a sanitizer build of the same source, loaded instead when set (the
# sanitizer test runs the oracle's pins against it in a child process)
_LIB_OVERRIDE = os.environ.get("QMV_ORACLE_LIB")

Q8_0 = 1
Q4_0 = 2
OUTCOME = {0: "ok", 1: "arg", 2: "format", 3: "shape"}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain scalar C, no fused multiply-add)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build()
            L = ctypes.CDLL(_LIB_PATH)
        u32, u64, i32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
        vp = ctypes.c_void_p
        L.orc_span.argtypes = [u32, u32, u64, u64, vp]
        L.orc_span.restype = i32
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_f16_value.restype = ctypes.c_double
        L.orc_quant_at.argtypes = [vp, u32, u64, u64, u64]
        L.orc_quant_at.restype = i32
        L.orc_scale_at.argtypes = [vp, u64, u32, u64]
        L.orc_scale_at.restype = ctypes.c_float
        L.orc_dequant_rows.argtypes = [vp, u32, u32, u64, u64, vp, u64, vp]
        L.orc_dequant_rows.restype = None
        L.orc_product.argtypes = [vp, u32, u32, u64, u64, vp, i32, u64, vp, u64, vp, vp]
        L.orc_product.restype = None
        L.orc_quantize_q8.argtypes = [vp, u64, vp, vp]
        L.orc_quantize_q8.restype = None
        L.orc_block_dots.argtypes = [vp, u32, u64, u64, vp, vp]
        L.orc_block_dots.restype = None
        L.orc_gemm_q8act.argtypes = [vp, u32, u32, u64, u64, vp, vp, u64, vp, u64, vp, vp]
        L.orc_gemm_q8act.restype = None
        L.orc_class_wtype.argtypes = [u32, u32, u32, u32, ctypes.POINTER(u32)]
        L.orc_class_wtype.restype = i32
        L.orc_check_image.argtypes = [u32, u32, u64, u64, vp, u64]
        L.orc_check_image.restype = i32
        L.orc_gguf_span.argtypes = [u32, u64, u64, ctypes.POINTER(u64)]
        L.orc_gguf_span.restype = i32
        L.orc_check_gguf.argtypes = [u32, u64, u64, vp, u64]
        L.orc_check_gguf.restype = i32
        L.orc_gguf_to_image.argtypes = [u32, u64, u64, vp, vp]
        L.orc_gguf_to_image.restype = i32
        L.orc_f16_bits.argtypes = [ctypes.c_float]
        L.orc_f16_bits.restype = ctypes.c_uint16
        L.orc_quantize_weights.argtypes = [u32, u32, u64, u64, vp, vp]
        L.orc_quantize_weights.restype = i32
        L.orc_quantize_q4_search.argtypes = [u32, u64, u64, vp, vp]
        L.orc_quantize_q4_search.restype = i32
        L.orc_ffn_act.argtypes = [ctypes.c_double, u32]
        L.orc_ffn_act.restype = ctypes.c_double
        L.orc_gated.argtypes = [vp, vp, u64, u32, vp]
        L.orc_gated.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def span(wtype, scale_f16, rows, cols):
    """(outcome, dict) with q_bytes, d_offset, d_bytes, min_span, full_span."""
    out = np.zeros(5, dtype=np.uint64)
    st = lib().orc_span(wtype, scale_f16, rows, cols, _ptr(out))
    if st != 0:
        return OUTCOME[st], None
    keys = ("q_bytes", "d_offset", "d_bytes", "min_span", "full_span")
    return "ok", {k: int(v) for k, v in zip(keys, out)}


def f16_value(bits: int) -> float:
    return lib().orc_f16_value(bits)


def layout(wtype, scale_f16, rows, cols, q: np.ndarray, d: np.ndarray,
           trailing_pad: bool = True) -> np.ndarray:
    """A matrix image as the file holds it: q, zeros up to the d offset, d,
    and (optionally) zeros up to a multiple of 64."""
    st, s = span(wtype, scale_f16, rows, cols)
    if st != "ok":
        raise ValueError(f"span: {st}")
    qb = np.ascontiguousarray(q).view(np.uint8).reshape(-1)
    db = np.ascontiguousarray(d).view(np.uint8).reshape(-1)
    if qb.size != s["q_bytes"] or db.size != s["d_bytes"]:
        raise ValueError("q or d has the wrong size for this shape")
    n = s["full_span"] if trailing_pad else s["min_span"]
    img = np.zeros(n, dtype=np.uint8)
    img[:qb.size] = qb
    img[s["d_offset"]:s["d_offset"] + db.size] = db
    return img


def quant_at(img, wtype, cols, r, c) -> int:
    return lib().orc_quant_at(_ptr(img), wtype, cols, r, c)


def scale_at(img, wtype, scale_f16, rows, cols, k) -> float:
    st, s = span(wtype, scale_f16, rows, cols)
    return lib().orc_scale_at(_ptr(img), s["d_offset"], scale_f16, k)


def dequant_rows(img, wtype, scale_f16, rows, cols, ids) -> np.ndarray:
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    out = np.zeros((ids.size, cols), dtype=np.float32)
    lib().orc_dequant_rows(_ptr(img), wtype, scale_f16, rows, cols, _ptr(ids),
                           ids.size, _ptr(out))
    return out


def product(img, wtype, scale_f16, rows, cols, x, sel=None, threads: int = 1):
    """(ref, norm), each float64 [batch][len(sel)].  x is float32 [batch][cols]
    or bfloat16 bits as uint16 [batch][cols].  sel defaults to every row.
    threads > 1 splits the selected rows over threads (the C code releases
    the interpreter lock while it runs)."""
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    if x.dtype == np.float32:
        x_bf16 = 0
    elif x.dtype == np.uint16:
        x_bf16 = 1
    else:
        raise TypeError("x must be float32 or bfloat16 bits (uint16)")
    batch = x.shape[0]
    assert x.shape[1] == cols
    if sel is None:
        sel = np.arange(rows, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    L = lib()

    def run(part):
        s = np.ascontiguousarray(part)
        ref = np.zeros((batch, s.size), dtype=np.float64)
        nrm = np.zeros((batch, s.size), dtype=np.float64)
        L.orc_product(_ptr(img), wtype, scale_f16, rows, cols, _ptr(x), x_bf16,
                      batch, _ptr(s), s.size, _ptr(ref), _ptr(nrm))
        return ref, nrm

    if threads <= 1 or sel.size < 2 * threads:
        return run(sel)
    parts = np.array_split(sel, threads)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(run, parts))
    return (np.concatenate([r for r, _ in res], axis=1),
            np.concatenate([n for _, n in res], axis=1))


def quantize_q8(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    assert x.size % 32 == 0
    q = np.zeros(x.size, dtype=np.int8)
    d = np.zeros(x.size // 32, dtype=np.float32)
    lib().orc_quantize_q8(_ptr(x), x.size, _ptr(q), _ptr(d))
    return q, d


def block_dots(img, wtype, rows, cols, xq: np.ndarray) -> np.ndarray:
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    assert xq.size == cols
    s = np.zeros((rows, cols // 32), dtype=np.int32)
    lib().orc_block_dots(_ptr(img), wtype, rows, cols, _ptr(xq), _ptr(s))
    return s


def gemm_q8act(img, wtype, scale_f16, rows, cols, xq, dx, sel=None, threads: int = 1):
    """(ref, bound), float64 [batch][len(sel)]: the product on Q8_0-quantized
    activations (xq int8 [batch][cols], dx float32 [batch][cols/32])."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    dx = np.ascontiguousarray(dx, dtype=np.float32)
    if xq.ndim == 1:
        xq = xq.reshape(1, -1)
    batch = xq.shape[0]
    assert xq.shape[1] == cols and dx.size == batch * (cols // 32)
    if sel is None:
        sel = np.arange(rows, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    L = lib()

    def run(part):
        p = np.ascontiguousarray(part)
        ref = np.zeros((batch, p.size), dtype=np.float64)
        bnd = np.zeros((batch, p.size), dtype=np.float64)
        L.orc_gemm_q8act(_ptr(img), wtype, scale_f16, rows, cols, _ptr(xq), _ptr(dx), batch,
                         _ptr(p), p.size, _ptr(ref), _ptr(bnd))
        return ref, bnd

    if threads <= 1 or sel.size < 2 * threads:
        return run(sel)
    parts = np.array_split(sel, threads)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(run, parts))
    return (np.concatenate([r for r, _ in res], axis=1),
            np.concatenate([b for _, b in res], axis=1))


def q8act_within_tolerance(y, ref, bound, cols):
    """Parity predicate of the product on quantized activations: the block
    sums are exact integers, so the only error is float32 rounding of the
    combine, each block's fl(dw dx) and its multiply-add into the running
    sum: |y - ref| <= (nb + 2) 2^-23 bound, nb = cols / 32 blocks (twice
    the first-order bound).  Returns (ok, worst ratio err / tolerance)."""
    y = np.asarray(y, dtype=np.float64)
    tol = (cols // 32 + 2) * 2.0 ** -23 * bound
    err = np.abs(y - ref)
    ok = bool((err <= tol).all())
    pos = tol > 0
    worst = float((err[pos] / tol[pos]).max()) if pos.any() else 0.0
    return ok, worst


def class_wtype(file_wtype, q8_mask, class_bit, shared_classifier):
    out = ctypes.c_uint32(0)
    st = lib().orc_class_wtype(file_wtype, q8_mask, class_bit,
                               shared_classifier, ctypes.byref(out))
    return OUTCOME[st], (out.value if st == 0 else None)


def check_image(wtype, scale_f16, rows, cols, img, nbytes=None) -> str:
    if img is None:
        ptr, n = None, 0
    else:
        ptr = _ptr(img)
        n = img.size if nbytes is None else nbytes
    return OUTCOME[lib().orc_check_image(wtype, scale_f16, rows, cols, ptr, n)]


def within_tolerance(y, ref, norm, rel: float = 2e-3):
    """The parity predicate on float outputs: |y - ref| <= rel * norm per
    output, in float64; a NaN fails; a zero norm demands an exact zero.
    Returns (ok, worst ratio |y - ref| / norm over outputs with norm > 0)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - ref)
    bad = ~(err <= rel * norm)          # NaN compares false -> bad
    ok = not bool(bad.any())
    pos = norm > 0
    worst = float((err[pos] / norm[pos]).max()) if pos.any() else 0.0
    return ok, worst


# ---- gated feed-forward pair: act(W1 x) * (W3 x) ----

ACT_SILU = 0
ACT_GELU_TANH = 1
# max |act'(a)| over all a: SiLU 1.0998 (a = 2.40), GELU-tanh 1.1290 (a = 1.50)
ACT_LIPSCHITZ = 1.13


def ffn_act(a: float, act: int) -> float:
    return float(lib().orc_ffn_act(float(a), act))


def gated(img1, img3, wtype, scale_f16, rows, cols, x, act, sel=None, threads: int = 1):
    """(h, y1, n1, y3, n3), each float64 [batch][len(sel)]: the two products
    with their norms, and h = act(y1) * y3."""
    y1, n1 = product(img1, wtype, scale_f16, rows, cols, x, sel, threads)
    y3, n3 = product(img3, wtype, scale_f16, rows, cols, x, sel, threads)
    h = np.zeros_like(y1)
    lib().orc_gated(_ptr(y1), _ptr(y3), y1.size, act, _ptr(h))
    return h, y1, n1, y3, n3


def gated_within_tolerance(h, href, y1, n1, y3, n3, act, rel: float = 2e-3):
    """Parity predicate on a gated output, propagated from the products'
    bound e = rel * norm: |h - href| <= L e1 (|y3| + e3) + |act(y1)| e3 plus
    2^-20 of (|act(y1)| + L e1)(|y3| + e3) for the float32 activation and
    multiply, with L = max |act'|.  Returns (ok, worst ratio err / bound)."""
    h = np.asarray(h, dtype=np.float64)
    e1, e3 = rel * n1, rel * n3
    with np.errstate(over="ignore"):   # e^-a overflows to inf for the far tail: act -> 0
        a1 = np.abs(np.vectorize(lambda v: ffn_act(v, act))(y1)) if y1.size else y1
    L = ACT_LIPSCHITZ
    bound = L * e1 * (np.abs(y3) + e3) + a1 * e3
    bound = bound + 2.0 ** -20 * (a1 + L * e1) * (np.abs(y3) + e3)
    err = np.abs(h - href)
    ok = bool((err <= bound).all())
    pos = bound > 0
    worst = float((err[pos] / bound[pos]).max()) if pos.any() else 0.0
    return ok, worst


# ---- GGUF block data (the minfer GGUF page's BlockQ4_0 / BlockQ8_0) ----

def gguf_span(wtype, rows, cols):
    """(outcome, bytes): rows * cols / 32 blocks of 18 (Q4_0) or 34 (Q8_0)."""
    out = ctypes.c_uint64(0)
    st = lib().orc_gguf_span(wtype, rows, cols, ctypes.byref(out))
    return OUTCOME[st], (out.value if st == 0 else None)


def check_gguf(wtype, rows, cols, src, nbytes=None) -> str:
    a = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    n = a.size if nbytes is None else nbytes
    return OUTCOME[lib().orc_check_gguf(wtype, rows, cols, _ptr(a), n)]


def gguf_to_image(wtype, rows, cols, src) -> np.ndarray:
    """The .mlb image (f16 scales, both pads) holding the GGUF blocks' weights."""
    st, s = span(wtype, 1, rows, cols)
    if st != "ok":
        raise ValueError(f"span: {st}")
    a = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    ok, need = gguf_span(wtype, rows, cols)
    if ok != "ok" or a.size < need:
        raise ValueError("gguf data too short")
    img = np.zeros(s["full_span"], dtype=np.uint8)
    st = lib().orc_gguf_to_image(wtype, rows, cols, _ptr(a), _ptr(img))
    if st != 0:
        raise ValueError(OUTCOME[st])
    return img


# ---- weight writer (the .mlb page's quantization rules) ----

def f16_bits(x: float) -> int:
    """The oracle's own float32 -> binary16 rounding (nearest even)."""
    return int(lib().orc_f16_bits(float(np.float32(x))))


def quantize_weights(wtype, scale_f16, rows, cols, w: np.ndarray):
    """(outcome, image): the full_span .mlb bytes of float32 w [rows][cols]
    quantized by the writer's rule; outcome 'format' when a scale does not
    fit f16 (image None)."""
    st, s = span(wtype, scale_f16, rows, cols)
    if st != "ok":
        return st, None
    wf = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if wf.size != rows * cols:
        raise ValueError("w has the wrong size")
    img = np.zeros(s["full_span"], dtype=np.uint8)
    st = lib().orc_quantize_weights(wtype, scale_f16, rows, cols, _ptr(wf), _ptr(img))
    return OUTCOME[st], (img if st == 0 else None)


def quantize_q4_search(scale_f16, rows, cols, w: np.ndarray):
    """(outcome, image): Q4_0 by the least-squares search (13 candidate
    levels, weights x^2); outcome 'format' for a refused block."""
    st, s = span(Q4_0, scale_f16, rows, cols)
    if st != "ok":
        return st, None
    wf = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if wf.size != rows * cols:
        raise ValueError("w has the wrong size")
    img = np.zeros(s["full_span"], dtype=np.uint8)
    st = lib().orc_quantize_q4_search(scale_f16, rows, cols, _ptr(wf), _ptr(img))
    return OUTCOME[st], (img if st == 0 else None)
