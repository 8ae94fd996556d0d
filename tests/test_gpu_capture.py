"""The split-K workspace under graph capture: the first call that needs it on
a stream cannot allocate while that stream is being captured, so it returns
QMV_E_ARG and enqueues nothing; after one eager call on the stream, the
same call captures, and every replay matches the eager result bit for bit.
Each case uses a stream of its own, created here, so no earlier call has
given it a workspace."""
import ctypes

import numpy as np
import pytest

import cases as K
import oracle as O
from block_quant_weight_amd import qmv as Q

pytestmark = [pytest.mark.gpu,
              # the refused capture records nothing: torch warns of an empty graph
              pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.fixture(scope="module")
def _streams():
    """Streams created here, all kept until the module ends: a destroyed
    stream's handle can come back from the next create, and the library
    keys workspaces by handle."""
    import torch
    torch.cuda.init()
    # the HIP runtime torch has loaded, by its soname (a bare
    # "libamdhip64.so" could load a second runtime from another path)
    hip = ctypes.CDLL("libamdhip64.so.7")
    mapped = {line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line}
    assert len(mapped) == 1, f"more than one HIP runtime mapped: {mapped}"
    handles = []

    def create():
        handle = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(handle)) == 0
        assert all(handle.value != h.value for h in handles)
        handles.append(handle)
        return torch.cuda.ExternalStream(handle.value)
    yield create
    torch.cuda.synchronize()
    for handle in handles:
        hip.hipStreamDestroy(handle)


@pytest.fixture
def fresh_stream(_streams):
    return _streams()


def capture_refused_then_replays(call, y):
    import torch

    def capture(s):
        g = torch.cuda.CUDAGraph()
        err = None
        with torch.cuda.graph(g, stream=s):
            try:
                call(s)
            except Q.QmvError as e:
                err = e
        return g, err

    s = call.stream
    g, err = capture(s)
    assert err is not None and err.status == Q.QMV_E_ARG, "capture before any eager call must be refused"
    del g
    with torch.cuda.stream(s):
        call(s)                      # eager: allocates the stream's workspace
    torch.cuda.synchronize()
    want = y.clone()
    g, err = capture(s)
    assert err is None
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), want.view(torch.int32))
    del g
    return want


def test_gemm_split_k_capture(fresh_stream):
    import torch
    R, C, B = 256, 4096, 256            # 2 row tiles, one token tile: K split in 8
    img = K.make_image(601, 0, K.Q4, 1, R, C)
    h = K.upload(img, K.Q4, 1, R, C)
    try:
        xb = K.make_xb(601, 1, B, C)
        xd = K.dev(xb.view(np.int16)).view(torch.bfloat16)
        y = torch.empty((B, R), dtype=torch.float32, device="cuda")

        def call(s):
            Q.qmv_gemm(h, xd, y, stream=s)
        call.stream = fresh_stream
        got = capture_refused_then_replays(call, y).cpu().numpy()
        ref, norm = O.product(img, K.Q4, 1, R, C, xb, threads=K.THREADS)
        assert O.within_tolerance(got, ref, norm, 2e-3)[0]
    finally:
        Q.qmv_destroy(h)


def test_q8act_split_k_capture(fresh_stream):
    import torch
    R, C, B = 300, 1024, 130            # 3 row tiles x 2 token tiles: K split in 2
    img = K.make_image(602, 0, K.Q8, 0, R, C)
    h = K.upload(img, K.Q8, 0, R, C)
    try:
        x = K.make_x(602, 1, B, C)
        xq = np.zeros((B, C), dtype=np.int8)
        dx = np.zeros((B, C // 32), dtype=np.float32)
        for t in range(B):
            xq[t], dx[t] = O.quantize_q8(x[t])
        xqd, dxd = K.dev(xq), K.dev(dx)
        y = torch.empty((B, R), dtype=torch.float32, device="cuda")

        def call(s):
            Q.qmv_gemm_q8(h, xqd, dxd, y, stream=s)
        call.stream = fresh_stream
        got = capture_refused_then_replays(call, y).cpu().numpy()
        ref, bound = O.gemm_q8act(img, K.Q8, 0, R, C, xq, dx, threads=K.THREADS)
        assert O.q8act_within_tolerance(got, ref, bound, C)[0]
    finally:
        Q.qmv_destroy(h)
