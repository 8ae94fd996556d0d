"""Every entry point captured in a HIP graph: each replay must reproduce the
eager result bit for bit, with other eager work (which overwrites the same
outputs) and synchronisations between the replays.  The calls enqueue
kernels only (the writer clears its status word and padding with a kernel,
not a memset), so nothing in a captured graph depends on host work."""
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


def check_graph(call, outputs, disturb):
    """call(stream) enqueues the work; outputs: tensors it writes; disturb()
    overwrites them eagerly.  Eager result, then three replays."""
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(s)              # eager (also allocates any per-stream workspace)
        call(s)
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    for _ in range(3):
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o.view(torch.uint8) if o.dtype != torch.uint8 else o,
                               w.view(torch.uint8) if w.dtype != torch.uint8 else w)
    del g


def garbage(*ts):
    import torch

    def f():
        for t in ts:
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(7)
    return f


@pytest.mark.parametrize("wt,sf,R,C,B", [(2, 1, 4096, 4096, 1), (1, 1, 11008, 4096, 1),
                                         (1, 1, 1000, 1024, 16), (2, 0, 300, 1024, 70)])
def test_graph_gemv(wt, sf, R, C, B):
    import torch
    h = K.upload(K.make_image(500, 0, wt, sf, R, C), wt, sf, R, C)
    try:
        x = K.dev(K.make_x(500, 1, B, C))
        y = torch.empty((B, R), dtype=torch.float32, device="cuda")
        check_graph(lambda s: Q.qmv_gemv(h, x, y, stream=s), [y], garbage(y))
    finally:
        Q.qmv_destroy(h)


def test_graph_group_and_gated():
    import torch
    mats = [(2, 1, 4096, 4096), (2, 1, 1024, 4096), (1, 1, 1024, 4096)]
    hs = [K.upload(K.make_image(501, i, *m), *m) for i, m in enumerate(mats)]
    w1 = K.upload(K.make_image(502, 1, 2, 1, 11008, 4096), 2, 1, 11008, 4096)
    w3 = K.upload(K.make_image(502, 3, 2, 1, 11008, 4096), 2, 1, 11008, 4096)
    try:
        x = K.dev(K.make_x(501, 1, 1, 4096))
        ys = [torch.empty((1, m[2]), dtype=torch.float32, device="cuda") for m in mats]
        check_graph(lambda s: Q.qmv_gemv_group(hs, x, ys, stream=s), ys, garbage(*ys))
        h = torch.empty((1, 11008), dtype=torch.float32, device="cuda")
        check_graph(lambda s: Q.qmv_gemv_gated(w1, w3, x, h, act=0, stream=s), [h], garbage(h))
    finally:
        for m in hs + [w1, w3]:
            Q.qmv_destroy(m)


@pytest.mark.parametrize("wt,sf,R,C,B", [(2, 1, 14336, 4096, 512), (1, 0, 256, 8192, 256),
                                         (1, 1, 300, 1024, 100)])
def test_graph_gemm(wt, sf, R, C, B):
    """The large-tile kernel, its split-K form (workspace and reduction) and
    the small-batch kernel."""
    import torch
    h = K.upload(K.make_image(503, 0, wt, sf, R, C), wt, sf, R, C)
    try:
        xb = K.make_xb(503, 1, B, C)
        xd = K.dev(xb.view(np.int16)).view(torch.bfloat16)
        y = torch.empty((B, R), dtype=torch.float32, device="cuda")
        check_graph(lambda s: Q.qmv_gemm(h, xd, y, stream=s), [y], garbage(y))
    finally:
        Q.qmv_destroy(h)


def test_graph_int8_path_and_gather():
    import torch
    R, C, B = 2048, 4096, 256
    h = K.upload(K.make_image(504, 0, 2, 1, R, C), 2, 1, R, C)
    try:
        x = K.dev(K.make_x(504, 1, B, C))
        xq = torch.empty((B, C), dtype=torch.int8, device="cuda")
        dx = torch.empty((B, C // 32), dtype=torch.float32, device="cuda")
        y = torch.empty((B, R), dtype=torch.float32, device="cuda")

        def call(s):
            Q.qmv_quantize_q8(x, xq, dx, stream=s)
            Q.qmv_gemm_q8(h, xq, dx, y, stream=s)
        check_graph(call, [xq, dx, y], garbage(xq, dx, y))
        ids = K.dev(np.array([0, 5, R - 1, 77], dtype=np.int32))
        out = torch.empty((4, C), dtype=torch.float32, device="cuda")
        check_graph(lambda s: Q.qmv_embed_rows(h, ids, out, stream=s), [out], garbage(out))
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("wt,sf,rule", [(1, 1, 0), (2, 1, 0), (2, 0, 1)])
def test_graph_writer(wt, sf, rule):
    import torch
    R, C = 300, 1024
    w = torch.from_numpy(np.random.default_rng(505).standard_normal((R, C)).astype(np.float32)).cuda()
    n = Q.qmv_span(wt, sf, R, C)["min_span"]
    img = torch.empty(n, dtype=torch.uint8, device="cuda")
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    check_graph(lambda s: Q.qmv_quantize_weights(wt, sf, w, img, status=st, stream=s, rule=rule),
                [img, st], garbage(img, st))
    assert int(st[0].item()) == 0
    ref = (O.quantize_q4_search(sf, R, C, w.cpu().numpy())[1] if rule
           else O.quantize_weights(wt, sf, R, C, w.cpu().numpy())[1])
    assert np.array_equal(img.cpu().numpy(), ref[:n])
