"""CPU checks of the C-ABI library: it loads, exports every function that
include/qmv.h declares, and its host-only rules (spans, class rule, byte
checks, argument errors) agree with the oracle.  No kernel is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from block_quant_weight_amd import qmv as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CODES = {"ok": Q.QMV_OK, "arg": Q.QMV_E_ARG, "format": Q.QMV_E_FORMAT,
         "shape": Q.QMV_E_SHAPE}


def header_functions():
    txt = open(os.path.join(ROOT, "include", "qmv.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    L = Q.lib()
    declared = header_functions()
    assert len(declared) == 20
    assert sorted(Q.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_span_matches_oracle():
    shapes = [(1, 32), (3, 32), (5, 96), (4096, 4096), (11008, 4096), (4096, 11008),
              (248320, 1024), (151936, 896), (7, 4064), (16777216, 32), (1, 16777216)]
    for wt in (1, 2):
        for sf in (0, 1):
            for R, C in shapes:
                st, s = O.span(wt, sf, R, C)
                got = Q.qmv_span(wt, sf, R, C)
                for k in ("q_bytes", "d_offset", "d_bytes", "min_span"):
                    assert got[k] == s[k], (wt, sf, R, C, k)


@pytest.mark.parametrize("args", [(3, 0, 1, 32), (0, 0, 1, 32), (1, 2, 1, 32),
                                  (1, 0, 1, 48), (1, 0, 0, 32), (1, 0, 1, 0),
                                  (2, 1, 16777217, 32), (2, 1, 32, 16777248)])
def test_span_rejects_like_oracle(args):
    st, _ = O.span(*args)
    with pytest.raises(Q.QmvError) as e:
        Q.qmv_span(*args)
    assert e.value.status == CODES[st]


def test_class_rule_matches_oracle_exhaustively():
    for fw in (0, 1, 2, 3):
        for mask in range(128):
            for cls in (0, 1, 2, 3, 4, 8, 16, 32, 64, 128):
                for shared in (0, 1):
                    st, want = O.class_wtype(fw, mask, cls, shared)
                    if st == "ok":
                        assert Q.qmv_class_wtype(fw, mask, cls, shared) == want
                    else:
                        with pytest.raises(Q.QmvError) as e:
                            Q.qmv_class_wtype(fw, mask, cls, shared)
                        assert e.value.status == CODES[st]


def test_create_rejects_and_destroy():
    with pytest.raises(Q.QmvError) as e:
        Q.qmv_create(4, 0, 32, 32)
    assert e.value.status == Q.QMV_E_FORMAT
    with pytest.raises(Q.QmvError) as e:
        Q.qmv_create(1, 0, 32, 40)
    assert e.value.status == Q.QMV_E_SHAPE
    h = Q.qmv_create(2, 1, 64, 128)
    assert Q.lib().qmv_create(None, 1, 0, 1, 32) == Q.QMV_E_ARG
    Q.qmv_destroy(h)
    assert Q.lib().qmv_destroy(None) == Q.QMV_OK


def test_upload_byte_checks_before_any_device_use():
    # The checks of the loader's table run on the host before anything
    # touches a device, so they can be exercised here.
    kv_cases = [(1, 0, 1, 32, "short"), (1, 0, 1, 32, "m128@0"), (1, 1, 2, 96, "m128@150"),
                (2, 0, 1, 32, "short")]
    for wt, sf, R, C, case in kv_cases:
        _, s = O.span(wt, sf, R, C)
        img = np.zeros(s["full_span"], dtype=np.uint8)
        n = img.size
        if case == "short":
            n = s["min_span"] - 1
        else:
            img[int(case[5:])] = 0x80
        assert O.check_image(wt, sf, R, C, img, n) == "format"
        h = Q.qmv_create(wt, sf, R, C)
        try:
            with pytest.raises(Q.QmvError) as e:
                Q.qmv_upload(h, img, nbytes=n, stream=0)
            assert e.value.status == Q.QMV_E_FORMAT
        finally:
            Q.qmv_destroy(h)
    h = Q.qmv_create(1, 0, 1, 32)
    assert Q.lib().qmv_upload(h.ptr, None, 100, None) == Q.QMV_E_ARG
    Q.qmv_destroy(h)


def test_compute_before_upload_is_an_argument_error():
    h = Q.qmv_create(2, 1, 64, 64)
    L = Q.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert L.qmv_gemv(h.ptr, p, p, 1, None) == Q.QMV_E_ARG
    assert L.qmv_gemm(h.ptr, p, p, 1, None) == Q.QMV_E_ARG
    assert L.qmv_embed_rows(h.ptr, p, 1, p, None) == Q.QMV_E_ARG
    assert L.qmv_block_dots(h.ptr, p, p, None) == Q.QMV_E_ARG
    assert L.qmv_gemv(None, p, p, 1, None) == Q.QMV_E_ARG
    assert L.qmv_quantize_q8(p, 48, p, p, None) == Q.QMV_E_SHAPE
    assert L.qmv_quantize_q8(None, 64, p, p, None) == Q.QMV_E_ARG
    Q.qmv_destroy(h)


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(Q.qmv_status_str(st), str) and Q.qmv_status_str(st)


def test_oracle_and_product_share_no_code():
    # Neither side includes, imports or links the other: check the include
    # and import statements of both.
    def code_refs(path):
        refs = []
        for line in open(path):
            t = line.strip()
            if t.startswith("#include") or t.startswith("import ") or t.startswith("from "):
                refs.append(t)
        return refs
    csrc = os.path.join(ROOT, "block_quant_weight_amd", "csrc")
    pkg = os.path.join(ROOT, "block_quant_weight_amd")
    for path in [os.path.join(csrc, f) for f in os.listdir(csrc)] + \
            [os.path.join(pkg, f) for f in os.listdir(pkg) if f.endswith(".py")]:
        for ref in code_refs(path):
            assert "oracle" not in ref, (path, ref)
    for f in ("qmv_oracle.c", "__init__.py"):
        for ref in code_refs(os.path.join(ROOT, "oracle", f)):
            assert "block_quant_weight_amd" not in ref and "qmv.h" not in ref, (f, ref)


def test_gguf_span_matches_oracle_and_page():
    for wt in (1, 2):
        for R, C in [(1, 32), (7, 96), (151936, 896), (248320, 1024), (16777216, 32)]:
            st, n = O.gguf_span(wt, R, C)
            assert Q.qmv_gguf_span(wt, R, C) == n
    # the minfer page's byte counts (section 3.2 (g))
    assert Q.qmv_gguf_span(1, 151936, 896) == 144_643_072
    assert Q.qmv_gguf_span(2, 151936, 896) == 76_575_744
    for args in [(3, 1, 32), (1, 1, 48), (1, 0, 32), (2, 16777217, 32)]:
        st, _ = O.gguf_span(*args)
        with pytest.raises(Q.QmvError) as e:
            Q.qmv_gguf_span(*args)
        assert e.value.status == CODES[st]
    assert Q.lib().qmv_gguf_span(1, 1, 32, None) == Q.QMV_E_ARG


def test_gguf_upload_host_checks():
    # rejected on the host, before any device call: f32-scale handle, short
    # data, a -128 quant (on this CPU-only machine a handle can be created but
    # not uploaded, so only the refusals are checked here)
    L = Q.lib()
    R, C = 2, 64
    blob = np.zeros(Q.qmv_gguf_span(1, R, C), dtype=np.uint8)
    ptr = blob.ctypes.data_as(ctypes.c_void_p)
    h32 = Q.qmv_create(1, 0, R, C)
    try:
        assert L.qmv_upload_gguf(h32.ptr, ptr, blob.size, None) == Q.QMV_E_FORMAT
    finally:
        Q.qmv_destroy(h32)
    h = Q.qmv_create(1, 1, R, C)
    try:
        assert L.qmv_upload_gguf(h.ptr, ptr, blob.size - 1, None) == Q.QMV_E_FORMAT
        bad = blob.copy()
        bad[34 * 3 + 2 + 7] = 0x80
        assert O.check_gguf(1, R, C, bad) == "format"
        assert L.qmv_upload_gguf(h.ptr, bad.ctypes.data_as(ctypes.c_void_p), bad.size,
                                 None) == Q.QMV_E_FORMAT
        assert L.qmv_upload_gguf(h.ptr, None, 0, None) == Q.QMV_E_ARG
    finally:
        Q.qmv_destroy(h)


def test_quantize_weights_host_checks():
    L = Q.lib()
    p = ctypes.c_void_p(4096)
    assert L.qmv_quantize_weights(3, 0, 0, 1, 32, p, p, 1 << 20, p, None) == Q.QMV_E_FORMAT
    assert L.qmv_quantize_weights(1, 2, 0, 1, 32, p, p, 1 << 20, p, None) == Q.QMV_E_FORMAT
    assert L.qmv_quantize_weights(1, 0, 0, 1, 48, p, p, 1 << 20, p, None) == Q.QMV_E_SHAPE
    assert L.qmv_quantize_weights(1, 0, 0, 1, 32, None, p, 1 << 20, p, None) == Q.QMV_E_ARG
    assert L.qmv_quantize_weights(1, 0, 0, 1, 32, p, p, 1 << 20, None, None) == Q.QMV_E_ARG
    assert L.qmv_quantize_weights(1, 0, 0, 1, 32, ctypes.c_void_p(4100), p, 1 << 20, p,
                                  None) == Q.QMV_E_ARG
    assert L.qmv_quantize_weights(1, 0, 0, 1, 32, p, p, 1 << 20, ctypes.c_void_p(4098),
                                  None) == Q.QMV_E_ARG
    need = Q.qmv_span(1, 1, 1, 32)["min_span"]
    assert L.qmv_quantize_weights(1, 1, 0, 1, 32, p, p, need - 1, p, None) == Q.QMV_E_ARG
    # the least-squares search is a Q4_0 rule; rules above 1 do not exist
    assert L.qmv_quantize_weights(1, 0, 1, 1, 32, p, p, 1 << 20, p, None) == Q.QMV_E_ARG
    assert L.qmv_quantize_weights(2, 0, 2, 1, 32, p, p, 1 << 20, p, None) == Q.QMV_E_ARG
