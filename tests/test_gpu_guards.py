"""Output bounds: every output buffer (y, out, h, the writer's image) sits
between two guard bands of 4 KiB filled with a sentinel pattern, on ragged
shapes of every entry point that writes device memory; after the call the
bands must be untouched and the output itself fully written (no sentinel
word left inside it)."""
import numpy as np
import pytest

import cases as K
from block_quant_weight_amd import qmv as Q

pytestmark = pytest.mark.gpu
GUARD = 1024          # 32-bit words on each side (4 KiB, keeps 16-byte alignment)
SENTINEL = 0x7FA5A5A5  # a NaN pattern no kernel writes


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


class Guarded:
    """A device buffer of n elements of a 4- or 1-byte dtype between guard
    bands; .t is the inner tensor (shaped)."""

    def __init__(self, shape, dtype):
        import torch
        n = int(np.prod(shape))
        esize = torch.empty(0, dtype=dtype).element_size()
        words = -(-n * esize // 4)
        self.full = torch.full((words + 2 * GUARD,), SENTINEL, dtype=torch.int32, device="cuda")
        inner = self.full[GUARD:GUARD + words].view(torch.uint8)[:n * esize]
        self.t = inner.view(dtype).view(*shape)
        self.words, self.n, self.esize = words, n, esize

    def check(self, what, full_write=True):
        import torch
        torch.cuda.synchronize()
        f = self.full.cpu().numpy().view(np.uint32)
        assert np.all(f[:GUARD] == SENTINEL), f"{what}: guard band before the output written"
        assert np.all(f[GUARD + self.words:] == SENTINEL), f"{what}: guard band after the output written"
        if full_write and self.esize == 4:
            inner = f[GUARD:GUARD + self.words]
            assert not np.any(inner == SENTINEL), f"{what}: part of the output not written"


# ragged rows / columns / batches of the vector, grouped, matrix-core and
# prefill paths
GEMV = [(K.Q4, 1, 37, 96, 1), (K.Q8, 0, 1001, 2048, 3), (K.Q4, 0, 129, 4096, 8),
        (K.Q8, 1, 300, 1024, 9), (K.Q4, 1, 77, 8192, 65), (K.Q8, 1, 513, 1024, 64),
        (K.Q4, 1, 12289, 4096, 1)]


@pytest.mark.parametrize("wt,sf,R,C,B", GEMV)
def test_gemv_guards(wt, sf, R, C, B):
    img = K.make_image(40 + R, 0, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        x = K.dev(K.make_x(40, 1, B, C))
        import torch
        y = Guarded((B, R), torch.float32)
        Q.qmv_gemv(h, x, y.t)
        y.check(f"gemv {wt}/{sf} {R}x{C} b{B}")
    finally:
        Q.qmv_destroy(h)


@pytest.mark.parametrize("wt,sf,R,C,B", [(K.Q4, 1, 1001, 4096, 37), (K.Q8, 0, 257, 2048, 300),
                                         (K.Q8, 1, 130, 14336, 9)])
def test_gemm_guards(wt, sf, R, C, B):
    import torch
    img = K.make_image(50 + R, 0, wt, sf, R, C)
    h = K.upload(img, wt, sf, R, C)
    try:
        xb = K.make_xb(50, 1, B, C)
        xd = K.dev(xb.view(np.int16)).view(torch.bfloat16)
        for fn in (Q.qmv_gemm, Q.qmv_gemm_noalloc):
            y = Guarded((B, R), torch.float32)
            fn(h, xd, y.t)
            y.check(f"{fn.__name__} {wt}/{sf} {R}x{C} b{B}")
        xq = torch.empty((B, C), dtype=torch.int8, device="cuda")
        dx = torch.empty((B, C // 32), dtype=torch.float32, device="cuda")
        Q.qmv_quantize_q8(K.dev(K.make_x(50, 2, B, C)), xq, dx)
        y = Guarded((B, R), torch.float32)
        Q.qmv_gemm_q8(h, xq, dx, y.t)
        y.check(f"gemm_q8 {wt}/{sf} {R}x{C} b{B}")
    finally:
        Q.qmv_destroy(h)


def test_group_and_gated_guards():
    import torch
    C = 4096
    shapes = [(K.Q4, 1, 301), (K.Q8, 1, 97), (K.Q4, 1, 1025)]
    hs = [K.upload(K.make_image(60, i, wt, sf, R, C), wt, sf, R, C)
          for i, (wt, sf, R) in enumerate(shapes)]
    try:
        for B in (1, 3):
            x = K.dev(K.make_x(60, 9, B, C))
            ys = [Guarded((B, R), torch.float32) for (_, _, R) in shapes]
            Q.qmv_gemv_group(hs, x, [g.t for g in ys])
            for g, s in zip(ys, shapes):
                g.check(f"group {s} b{B}")
        w1 = K.upload(K.make_image(61, 1, K.Q4, 1, 1001, C), K.Q4, 1, 1001, C)
        w3 = K.upload(K.make_image(61, 3, K.Q4, 1, 1001, C), K.Q4, 1, 1001, C)
        try:
            for B in (1, 5):
                x = K.dev(K.make_x(61, 9, B, C))
                hh = Guarded((B, 1001), torch.float32)
                Q.qmv_gemv_gated(w1, w3, x, hh.t)
                hh.check(f"gated b{B}")
        finally:
            Q.qmv_destroy(w1)
            Q.qmv_destroy(w3)
    finally:
        for h in hs:
            Q.qmv_destroy(h)


def test_embed_and_writer_guards():
    import torch
    R, C = 1000, 96
    img = K.make_image(70, 0, K.Q8, 1, R, C)
    h = K.upload(img, K.Q8, 1, R, C)
    try:
        ids = K.dev(np.array([0, 999, 5, -1, 1000, 3], dtype=np.int32))
        out = Guarded((6, C), torch.float32)
        Q.qmv_embed_rows(h, ids, out.t)
        out.check("embed")
    finally:
        Q.qmv_destroy(h)
    for wt, sf, rule, (R, C) in [(K.Q4, 1, Q.QMV_Q4_ROUND, (37, 96)), (K.Q8, 0, Q.QMV_Q4_ROUND, (5, 4064)),
                                 (K.Q4, 0, Q.QMV_Q4_SEARCH, (3, 160))]:
        w = K.dev(K.make_x(71, 0, R, C))
        n = Q.qmv_span(wt, sf, R, C)["min_span"]
        image = Guarded((n,), torch.uint8)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        Q.qmv_quantize_weights(wt, sf, w, image.t, status=status, rule=rule)
        image.check(f"writer {wt}/{sf}/{rule} {R}x{C}", full_write=False)
        assert int(status[0].item()) == 0
