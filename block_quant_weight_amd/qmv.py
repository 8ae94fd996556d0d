"""Thin Python binding of libqmv (include/qmv.h): the same entry points, with
arguments marshalled from PyTorch tensors (device memory) and streams.  All
computation happens in the HIP library; if libqmv.so is missing, loading it
raises instead of falling back to anything else."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmv.so")

QMV_Q8_0 = 1
QMV_Q4_0 = 2
QMV_OK = 0
QMV_E_ARG = -1
QMV_E_FORMAT = -2
QMV_E_SHAPE = -3
QMV_E_DEVICE = -4
QMV_E_NOMEM = -5

# every symbol include/qmv.h declares
EXPORTS = ("qmv_span", "qmv_class_wtype", "qmv_create", "qmv_upload",
           "qmv_destroy", "qmv_gemv", "qmv_gemv_group", "qmv_gemm", "qmv_embed_rows",
           "qmv_quantize_q8", "qmv_block_dots", "qmv_status_str", "qmv_gguf_span",
           "qmv_upload_gguf", "qmv_quantize_weights", "qmv_gemv_gated", "qmv_gemm_q8",
           "qmv_read_probe", "qmv_gemm_noalloc", "qmv_mfma_probe")

_lib = None


class QmvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {qmv_status_str(status)} ({status})")
        self.status = status


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built: run `python -m block_quant_weight_amd.build`")
        # torch first: its HIP runtime must be the one the library binds to
        # (a second runtime loaded ahead of it would not know torch's streams
        # or memory)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        u32, u64, i32, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        pu64 = ctypes.POINTER(u64)
        sig = {
            "qmv_span": ([u32, u32, u32, u32, pu64, pu64, pu64, pu64], i32),
            "qmv_class_wtype": ([u32, u32, u32, u32, ctypes.POINTER(u32)], i32),
            "qmv_create": ([ctypes.POINTER(vp), u32, u32, u32, u32], i32),
            "qmv_upload": ([vp, vp, u64, vp], i32),
            "qmv_destroy": ([vp], i32),
            "qmv_gemv": ([vp, vp, vp, u32, vp], i32),
            "qmv_gemv_group": ([vp, u32, vp, vp, u32, vp], i32),
            "qmv_gemm": ([vp, vp, vp, u32, vp], i32),
            "qmv_embed_rows": ([vp, vp, u32, vp, vp], i32),
            "qmv_quantize_q8": ([vp, u64, vp, vp, vp], i32),
            "qmv_block_dots": ([vp, vp, vp, vp], i32),
            "qmv_status_str": ([i32], ctypes.c_char_p),
            "qmv_gguf_span": ([u32, u32, u32, pu64], i32),
            "qmv_upload_gguf": ([vp, vp, u64, vp], i32),
            "qmv_quantize_weights": ([u32, u32, u32, u32, u32, vp, vp, u64, vp, vp], i32),
            "qmv_gemv_gated": ([vp, vp, u32, vp, vp, u32, vp], i32),
            "qmv_gemm_q8": ([vp, vp, vp, vp, u32, vp], i32),
            "qmv_read_probe": ([vp, u64, vp, vp], i32),
            "qmv_gemm_noalloc": ([vp, vp, vp, u32, vp], i32),
            "qmv_mfma_probe": ([u32, u32, u32, vp, vp, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def qmv_status_str(status: int) -> str:
    return lib().qmv_status_str(status).decode()


def _check(status: int, what: str):
    if status != QMV_OK:
        raise QmvError(status, what)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t, dtype, numel, what):
    """Device pointer of a contiguous GPU tensor of at least `numel` elements."""
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{what} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


class QmvHandle:
    """A matrix handle: the C pointer plus the shape it was created with."""

    def __init__(self, ptr, wtype, scale_f16, rows, cols):
        self.ptr = ptr
        self.wtype, self.scale_f16, self.rows, self.cols = wtype, scale_f16, rows, cols

    def __repr__(self):
        kind = {1: "Q8_0", 2: "Q4_0"}.get(self.wtype, "?")
        return f"QmvHandle({kind}, f16 scales={bool(self.scale_f16)}, {self.rows}x{self.cols})"


def qmv_span(wtype, scale_f16, rows, cols):
    """dict(q_bytes, d_offset, d_bytes, min_span); raises QmvError."""
    out = [ctypes.c_uint64(0) for _ in range(4)]
    _check(lib().qmv_span(wtype, scale_f16, rows, cols, *[ctypes.byref(o) for o in out]),
           "qmv_span")
    return dict(zip(("q_bytes", "d_offset", "d_bytes", "min_span"), (o.value for o in out)))


def qmv_gguf_span(wtype, rows, cols) -> int:
    """Bytes of a Q4_0 / Q8_0 tensor's GGUF block data; raises QmvError."""
    out = ctypes.c_uint64(0)
    _check(lib().qmv_gguf_span(wtype, rows, cols, ctypes.byref(out)), "qmv_gguf_span")
    return out.value


def qmv_class_wtype(file_wtype, q8_mask, class_bit, shared_classifier=0) -> int:
    out = ctypes.c_uint32(0)
    _check(lib().qmv_class_wtype(file_wtype, q8_mask, class_bit, shared_classifier,
                                 ctypes.byref(out)), "qmv_class_wtype")
    return out.value


def qmv_create(wtype, scale_f16, rows, cols) -> QmvHandle:
    p = ctypes.c_void_p(None)
    _check(lib().qmv_create(ctypes.byref(p), wtype, scale_f16, rows, cols), "qmv_create")
    return QmvHandle(p, wtype, scale_f16, rows, cols)


def qmv_upload(h: QmvHandle, src, nbytes=None, stream=None):
    """src: a host buffer (bytes, bytearray, numpy array) holding the matrix's
    bytes from its q array on."""
    import numpy as np
    a = np.ascontiguousarray(np.frombuffer(src, dtype=np.uint8)
                             if isinstance(src, (bytes, bytearray, memoryview))
                             else np.asarray(src).view(np.uint8).reshape(-1))
    n = a.size if nbytes is None else int(nbytes)
    if n > a.size:
        raise ValueError("nbytes exceeds the buffer")
    st = lib().qmv_upload(h.ptr, a.ctypes.data_as(ctypes.c_void_p), n, _stream(stream))
    _check(st, "qmv_upload")


def qmv_upload_gguf(h: QmvHandle, src, nbytes=None, stream=None):
    """src: a host buffer holding the matrix's GGUF block data."""
    import numpy as np
    a = np.ascontiguousarray(np.frombuffer(src, dtype=np.uint8)
                             if isinstance(src, (bytes, bytearray, memoryview))
                             else np.asarray(src).view(np.uint8).reshape(-1))
    n = a.size if nbytes is None else int(nbytes)
    if n > a.size:
        raise ValueError("nbytes exceeds the buffer")
    st = lib().qmv_upload_gguf(h.ptr, a.ctypes.data_as(ctypes.c_void_p), n, _stream(stream))
    _check(st, "qmv_upload_gguf")


QMV_Q4_ROUND = 0
QMV_Q4_SEARCH = 1


def qmv_quantize_weights(wtype, scale_f16, w, image, status=None, stream=None,
                         rule=QMV_Q4_ROUND):
    """w: float32 [rows, cols] on the GPU; image: uint8 GPU tensor of at least
    min_span bytes, receiving the .mlb bytes; rule QMV_Q4_SEARCH selects the
    Q4_0 least-squares writer.  With status (an int32/uint32 GPU tensor of
    >= 1 element) the call only enqueues work and status[0] tells, once done,
    whether a scale could not be stored (1); without it the call waits and
    raises QmvError(QMV_E_FORMAT) in that case."""
    import torch
    rows, cols = w.shape
    pw = _dev(w, torch.float32, rows * cols, "w")
    if image.dtype != torch.uint8:
        raise TypeError("image must be uint8")
    pi = _dev(image, torch.uint8, 0, "image")
    own = status is None
    if own:
        status = torch.empty(1, dtype=torch.int32, device=image.device)
    ps = _dev(status, status.dtype, 1, "status")
    st = lib().qmv_quantize_weights(wtype, scale_f16, rule, rows, cols, pw, pi, image.numel(),
                                    ps, _stream(stream))
    _check(st, "qmv_quantize_weights")
    if own:
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
        if int(status[0].item()) != 0:
            raise QmvError(QMV_E_FORMAT, "qmv_quantize_weights: a scale cannot be stored")


def qmv_destroy(h: QmvHandle):
    if h is not None and h.ptr:
        lib().qmv_destroy(h.ptr)
        h.ptr = ctypes.c_void_p(None)


def qmv_gemv(h: QmvHandle, x, y, batch=None, stream=None):
    """x: float32 [batch, cols] on the GPU; y: float32 [batch, rows]."""
    import torch
    b = x.shape[0] if (batch is None and x.dim() == 2) else (batch or 1)
    px = _dev(x, torch.float32, b * h.cols, "x")
    py = _dev(y, torch.float32, b * h.rows, "y")
    _check(lib().qmv_gemv(h.ptr, px, py, b, _stream(stream)), "qmv_gemv")


def qmv_gemv_group(hs, x, ys, batch=None, stream=None):
    """hs: list of handles with the same cols; x: float32 [batch, cols] on the
    GPU; ys: list of float32 [batch, rows_i] GPU tensors."""
    import torch
    if len(hs) != len(ys):
        raise ValueError("one output per handle")
    cols = hs[0].cols
    b = x.shape[0] if (batch is None and x.dim() == 2) else (batch or 1)
    px = _dev(x, torch.float32, b * cols, "x")
    n = len(hs)
    harr = (ctypes.c_void_p * n)(*[h.ptr.value if isinstance(h.ptr, ctypes.c_void_p) else h.ptr
                                   for h in hs])
    yarr = (ctypes.c_void_p * n)(*[_dev(y, torch.float32, b * h.rows, f"ys[{i}]").value
                                   for i, (h, y) in enumerate(zip(hs, ys))])
    _check(lib().qmv_gemv_group(ctypes.cast(harr, ctypes.c_void_p), n, px,
                                ctypes.cast(yarr, ctypes.c_void_p), b, _stream(stream)),
           "qmv_gemv_group")


def qmv_gemm_q8(h: QmvHandle, xq, dx, y, batch=None, stream=None):
    """Product on Q8_0-quantized activations: xq int8 [batch, cols], dx
    float32 [batch, cols/32] (from qmv_quantize_q8), y float32 [batch, rows],
    all on the GPU."""
    import torch
    b = xq.shape[0] if (batch is None and xq.dim() == 2) else (batch or 1)
    pq = _dev(xq, torch.int8, b * h.cols, "xq")
    pd = _dev(dx, torch.float32, b * (h.cols // 32), "dx")
    py = _dev(y, torch.float32, b * h.rows, "y")
    _check(lib().qmv_gemm_q8(h.ptr, pq, pd, py, b, _stream(stream)), "qmv_gemm_q8")


ACT_SILU = 0
ACT_GELU_TANH = 1


def qmv_gemv_gated(w1: QmvHandle, w3: QmvHandle, x, h, act=ACT_SILU, batch=None, stream=None):
    """h = act(W1 x) * (W3 x) per row; x: float32 [batch, cols] on the GPU,
    h: float32 [batch, rows]; act 0 = SiLU, 1 = GELU (tanh form)."""
    import torch
    b = x.shape[0] if (batch is None and x.dim() == 2) else (batch or 1)
    px = _dev(x, torch.float32, b * w1.cols, "x")
    ph = _dev(h, torch.float32, b * w1.rows, "h")
    _check(lib().qmv_gemv_gated(w1.ptr, w3.ptr, act, px, ph, b, _stream(stream)),
           "qmv_gemv_gated")


def qmv_gemm(h: QmvHandle, x_bf16, y, batch=None, stream=None):
    """x_bf16: bfloat16 (or int16/uint16 bit patterns) [batch, cols] on the
    GPU; y: float32 [batch, rows]."""
    import torch
    b = x_bf16.shape[0] if batch is None else batch
    if x_bf16.dtype in (torch.int16, torch.uint16):
        x_bf16 = x_bf16.view(torch.bfloat16)
    px = _dev(x_bf16, torch.bfloat16, b * h.cols, "x_bf16")
    py = _dev(y, torch.float32, b * h.rows, "y")
    _check(lib().qmv_gemm(h.ptr, px, py, b, _stream(stream)), "qmv_gemm")


def qmv_gemm_noalloc(h: QmvHandle, x_bf16, y, batch=None, stream=None):
    """qmv_gemm on the library's fixed scratch (no allocation); calls that
    overlap on one GPU race."""
    import torch
    b = batch if batch is not None else x_bf16.shape[0]
    px = _dev(x_bf16, torch.bfloat16, b * h.cols, "x_bf16")
    py = _dev(y, torch.float32, b * h.rows, "y")
    _check(lib().qmv_gemm_noalloc(h.ptr, px, py, b, _stream(stream)), "qmv_gemm_noalloc")


def qmv_embed_rows(h: QmvHandle, ids, out, stream=None):
    """ids: int32 [n] on the GPU; out: float32 [n, cols]."""
    import torch
    n = ids.numel()
    pi = _dev(ids, torch.int32, n, "ids")
    po = _dev(out, torch.float32, n * h.cols, "out")
    _check(lib().qmv_embed_rows(h.ptr, pi, n, po, _stream(stream)), "qmv_embed_rows")


def qmv_quantize_q8(x, q, d, stream=None):
    """x: float32 [n]; q: int8 [n]; d: float32 [n/32]; all on the GPU."""
    import torch
    n = x.numel()
    px = _dev(x, torch.float32, n, "x")
    pq = _dev(q, torch.int8, n, "q")
    pd = _dev(d, torch.float32, n // 32, "d")
    _check(lib().qmv_quantize_q8(px, n, pq, pd, _stream(stream)), "qmv_quantize_q8")


def qmv_block_dots(h: QmvHandle, xq, s, stream=None):
    """xq: int8 [cols]; s: int32 [rows, cols/32]; on the GPU."""
    import torch
    px = _dev(xq, torch.int8, h.cols, "xq")
    ps = _dev(s, torch.int32, h.rows * (h.cols // 32), "s")
    _check(lib().qmv_block_dots(h.ptr, px, ps, _stream(stream)), "qmv_block_dots")


def qmv_read_probe(src, nbytes, sink, stream=None):
    """Reads nbytes of the GPU tensor src (from its start; a measurement
    aid); sink: int32 or uint32 GPU tensor of at least 64 elements."""
    import torch
    if not (src.is_cuda and sink.is_cuda) or sink.numel() < 64 or sink.element_size() != 4:
        raise QmvError(QMV_E_ARG, "qmv_read_probe")
    if nbytes > src.numel() * src.element_size():
        raise QmvError(QMV_E_ARG, "qmv_read_probe")
    _check(lib().qmv_read_probe(src.data_ptr(), nbytes, sink.data_ptr(), _stream(stream)),
           "qmv_read_probe")


def qmv_mfma_probe(random_operands, waves_per_simd, iters, clocks, sink, stream=None):
    """Back-to-back matrix-core products (a measurement aid): clocks, int64
    GPU tensor of 2 * 1024 * waves_per_simd elements (cycles and 100 MHz
    ticks per wave); sink, float32 GPU tensor of 64 * 1024 * waves_per_simd."""
    import torch
    waves = 1024 * waves_per_simd
    if not (clocks.is_cuda and sink.is_cuda) or clocks.dtype != torch.int64 or sink.dtype != torch.float32:
        raise QmvError(QMV_E_ARG, "qmv_mfma_probe")
    if clocks.numel() < 2 * waves or sink.numel() < 64 * waves:
        raise QmvError(QMV_E_ARG, "qmv_mfma_probe")
    _check(lib().qmv_mfma_probe(int(random_operands), int(waves_per_simd), int(iters), clocks.data_ptr(),
                                sink.data_ptr(), _stream(stream)), "qmv_mfma_probe")
