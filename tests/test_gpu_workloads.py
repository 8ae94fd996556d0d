"""GPU parity at the full sizes of the five workloads, through the same entry
points the benchmark times.  Outputs the oracle can afford are compared in
full; the large products on seeded samples of rows (first, last, tile edges
and random rows, every token)."""
import numpy as np
import pytest

import cases as K
import oracle as O
from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu
TOL = 2e-3


def close(y, ref, norm, what):
    ok, worst = O.within_tolerance(y, ref, norm, TOL)
    print(f"{what}: worst |y-ref|/norm = {worst:.3e}")
    assert ok, f"{what}: outside 2e-3 * norm (worst ratio {worst:.3e})"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_q8_gemv_512_f32_scales():
    R = C = 512
    img = K.make_image(1, 0, K.Q8, 0, R, C)
    h = K.upload(img, K.Q8, 0, R, C)
    try:
        x = K.make_x(1, 0, 1, C)
        ref, norm = O.product(img, K.Q8, 0, R, C, x)
        close(K.gpu_gemv(h, x), ref, norm, "Q8_0 512x512 f32 scales")
    finally:
        Q.qmv_destroy(h)


def test_q4_gemv_4096_f16_scales():
    R = C = 4096
    img = K.make_image(2, 0, K.Q4, 1, R, C)
    h = K.upload(img, K.Q4, 1, R, C)
    try:
        x = K.make_x(2, 0, 1, C)
        ref, norm = O.product(img, K.Q4, 1, R, C, x, threads=K.THREADS)
        close(K.gpu_gemv(h, x), ref, norm, "Q4_0 4096x4096 f16 scales")
    finally:
        Q.qmv_destroy(h)


def test_mixed_decode_layer():
    for m, (name, cls, R, C) in enumerate(K.LAYER):
        wt = Q.qmv_class_wtype(K.Q4, K.LAYER_Q8_MASK, cls, 0)
        assert O.class_wtype(K.Q4, K.LAYER_Q8_MASK, cls, 0) == ("ok", wt)
        assert wt == (K.Q8 if name in ("wv", "w2") else K.Q4)
        img = K.make_image(3, m, wt, 1, R, C)
        h = K.upload(img, wt, 1, R, C)
        try:
            x = K.make_x(3, m, 1, C)
            ref, norm = O.product(img, wt, 1, R, C, x, threads=K.THREADS)
            close(K.gpu_gemv(h, x), ref, norm, f"layer {name} {R}x{C} wtype {wt}")
        finally:
            Q.qmv_destroy(h)


def test_mixed_decode_layer_fused_launches():
    # the layer as it runs: wq | wk | wv share the attention input, wo its
    # own, w1 | w3 share the FFN input, w2 its own: four launches
    import torch
    hs, imgs = {}, {}
    try:
        for m, (name, cls, R, C) in enumerate(K.LAYER):
            wt = Q.qmv_class_wtype(K.Q4, K.LAYER_Q8_MASK, cls, 0)
            imgs[name] = (K.make_image(3, m, wt, 1, R, C), wt, R, C)
            hs[name] = K.upload(imgs[name][0], wt, 1, R, C)
        for group, xm in ((("wq", "wk", "wv"), 20), (("wo",), 21), (("w1", "w3"), 22), (("w2",), 23)):
            C = imgs[group[0]][3]
            x = K.make_x(3, xm, 1, C)
            ys = [torch.empty((1, imgs[n][2]), dtype=torch.float32, device="cuda") for n in group]
            Q.qmv_gemv_group([hs[n] for n in group], K.dev(x), ys)
            torch.cuda.synchronize()
            for n, y in zip(group, ys):
                img, wt, R, C = imgs[n]
                ref, norm = O.product(img, wt, 1, R, C, x, threads=K.THREADS)
                close(y.cpu().numpy(), ref, norm, f"fused layer {n}")
    finally:
        for h in hs.values():
            Q.qmv_destroy(h)


@pytest.mark.parametrize("which", ["q4_14336x4096", "q8_4096x14336"])
def test_prefill_gemm_512_tokens(which):
    if which == "q4_14336x4096":
        m, wt, sf, R, C = 0, K.Q4, 1, 14336, 4096
    else:
        m, wt, sf, R, C = 1, K.Q8, 0, 4096, 14336
    B = 512
    img = K.make_image(4, m, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        xb = K.make_xb(4, m, B, C)
        y = K.gpu_gemm(h, xb)
        sel = K.sample_rows(R, 48, seed=m)
        ref, norm = O.product(img, wt, sf, R, C, xb, sel=sel, threads=K.THREADS)
        close(y[:, sel], ref, norm, f"gemm {which} x 512 tokens ({sel.size} rows)")
    finally:
        Q.qmv_destroy(h)


def test_shared_classifier_lm_head_and_gather():
    wt = Q.qmv_class_wtype(K.Q4, 1 | 2, 1, 1)        # tok_emb, shared classifier
    assert wt == K.Q8
    R, C = K.VOCAB, K.HIDDEN
    img = K.make_image(5, 0, wt, 1, R, C)
    h = K.upload(img, wt, 1, R, C)
    try:
        # batch 1: every row
        x = K.make_x(5, 0, 1, C)
        ref, norm = O.product(img, wt, 1, R, C, x, threads=K.THREADS)
        close(K.gpu_gemv(h, x), ref, norm, "LM head batch 1")
        # batch 64 hidden states (float32): sampled rows, every token
        x = K.make_x(5, 1, 64, C)
        y = K.gpu_gemv(h, x)
        sel = K.sample_rows(R, 384, seed=5)
        ref, norm = O.product(img, wt, 1, R, C, x, sel=sel, threads=K.THREADS)
        close(y[:, sel], ref, norm, f"LM head batch 64 ({sel.size} rows)")
        # gather of 64 token ids in [3, 248319], bit for bit
        from block_quant_weight_amd import synth
        ids = synth.token_ids(synth.rng(5, 0, synth.STREAM_IDS), 64, 3, R - 1)
        out = K.gpu_embed(h, ids)
        ref_rows = O.dequant_rows(img, wt, 1, R, C, ids.astype(np.int64))
        assert np.array_equal(out.view(np.uint32), ref_rows.view(np.uint32))
    finally:
        Q.qmv_destroy(h)
