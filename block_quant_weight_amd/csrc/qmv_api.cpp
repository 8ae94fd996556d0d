// C-ABI entry points of libqmv: matrix handles, upload, and the compute
// calls that validate their arguments on the host and enqueue the gfx950
// kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"
#include "qmv.h"
#include "qmv_layout.h"

struct qmv_mat {
    qmv::Layout layout;
    // One hipMalloc: q at dev, d at dev + d_offset (the file image, d's
    // padding zeroed), then at rexp_offset one int32 per row: the exponent
    // of the row's largest finite scale magnitude.
    uint8_t* dev = nullptr;
    uint64_t rexp_offset = 0;
    int device = -1;
    int32_t dexp = 0;        // the same exponent over the whole matrix
};

namespace {

bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int device_status(hipError_t e) {
    if (e == hipSuccess) return QMV_OK;
    if (e == hipErrorOutOfMemory) return QMV_E_NOMEM;
    return QMV_E_DEVICE;
}

// The launchers check their launches with hipGetLastError, which also
// returns an error left by any earlier failed runtime call of this thread
// (a failed allocation, say); each call that launches clears it first.
void clear_stale_error() { (void)hipGetLastError(); }

// Common checks of a compute call on an uploaded handle.  The call must run
// on the device that holds the matrix.
int ready(const qmv_mat* h) {
    if (h == nullptr || h->dev == nullptr) return QMV_E_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return QMV_E_DEVICE;
    if (cur != h->device) return QMV_E_ARG;
    clear_stale_error();
    return QMV_OK;
}

// Split-K workspace, one per (device, stream): work on one stream runs in
// order, so every call on that stream may reuse it; calls on other streams
// get their own.  It grows on demand.  A replaced buffer is never freed (a
// graph captured earlier may still name it); all live until the process
// ends.
struct Workspace {
    int device;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;

int workspace_for(hipStream_t stream, size_t bytes, void** out) {
    *out = nullptr;
    if (bytes == 0) return QMV_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace* w = nullptr;
    for (auto& e : g_ws)
        if (e.device == dev && e.stream == stream) w = &e;
    if (w != nullptr && w->bytes >= bytes) {
        *out = w->ptr;
        return QMV_OK;
    }
    // Growing allocates: not allowed while the stream is being captured into
    // a graph (run the call once on that stream before capturing it).
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return QMV_E_DEVICE;
    if (cap != hipStreamCaptureStatusNone) return QMV_E_ARG;
    void* p = nullptr;
    const hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return e == hipErrorOutOfMemory ? QMV_E_NOMEM : QMV_E_DEVICE;
    if (w != nullptr) {
        w->ptr = p;  // the old buffer stays allocated (see above)
        w->bytes = bytes;
    } else {
        g_ws.push_back(Workspace{dev, stream, p, bytes});
    }
    *out = p;
    return QMV_OK;
}

qmv::MatView view(const qmv_mat* h) {
    const qmv::Layout& L = h->layout;
    return qmv::MatView{h->dev, h->dev + L.d_offset,
                        reinterpret_cast<const int32_t*>(h->dev + h->rexp_offset), L.wtype,
                        L.scale_f16, L.rows, L.cols, h->dexp};
}

// Bytes of a handle's device allocation: the image with d's padding, then
// the row exponents from a 64-byte boundary.
bool device_bytes(const qmv::Layout& L, uint64_t* rexp_off, uint64_t* total) {
    const uint64_t off = (L.full_span + 63) & ~uint64_t{63};
    if (off < L.full_span) return false;
    const uint64_t t = off + uint64_t{L.rows} * 4;
    if (t < off) return false;
    *rexp_off = off;
    *total = t;
    return true;
}

// The row exponents of a checked host buffer (image or GGUF blocks), copied
// behind the image on `s`; the host vector must live until the stream is
// synchronised.
hipError_t upload_row_exponents(const qmv::Layout& L, const void* src, bool gguf, uint8_t* dst,
                                std::vector<int32_t>& rexp, int32_t* dexp, hipStream_t s) {
    rexp.resize(L.rows);
    qmv::scale_exponents(L, src, gguf, rexp.data(), dexp);
    return hipMemcpyAsync(dst, rexp.data(), uint64_t{L.rows} * 4, hipMemcpyHostToDevice, s);
}

}  // namespace

extern "C" {

int qmv_create(qmv_handle* out, uint32_t wtype, uint32_t scale_f16,
               uint32_t rows, uint32_t cols) {
    if (out == nullptr) return QMV_E_ARG;
    *out = nullptr;
    qmv::Layout L;
    const int st = qmv::compute_layout(wtype, scale_f16, rows, cols, &L);
    if (st != QMV_OK) return st;
    qmv_mat* h = new (std::nothrow) qmv_mat;
    if (h == nullptr) return QMV_E_NOMEM;
    h->layout = L;
    *out = h;
    return QMV_OK;
}

int qmv_upload(qmv_handle h, const void* src, uint64_t nbytes, void* stream) {
    if (h == nullptr || src == nullptr) return QMV_E_ARG;
    if (h->dev != nullptr) return QMV_E_ARG;  // uploaded once, then read-only
    const qmv::Layout& L = h->layout;
    const int st = qmv::check_bytes(L, src, nbytes);
    if (st != QMV_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_DEVICE;
    uint64_t rexp_off = 0, total = 0;
    if (!device_bytes(L, &rexp_off, &total)) return QMV_E_SHAPE;
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, total);
    if (e != hipSuccess) return device_status(e);
    uint8_t* d = static_cast<uint8_t*>(p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> rexp;
    int32_t dexp = 0;
    e = hipMemcpyAsync(d, src, L.min_span, hipMemcpyHostToDevice, s);
    // The device image always carries d's zero padding, whether or not the
    // caller's buffer held it.
    if (e == hipSuccess && rexp_off > L.min_span)
        e = hipMemsetAsync(d + L.min_span, 0, rexp_off - L.min_span, s);
    if (e == hipSuccess) e = upload_row_exponents(L, src, false, d + rexp_off, rexp, &dexp, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return device_status(e);
    }
    h->dev = d;
    h->rexp_offset = rexp_off;
    h->device = dev;
    h->dexp = dexp;
    return QMV_OK;
}

int qmv_upload_gguf(qmv_handle h, const void* src, uint64_t nbytes, void* stream) {
    clear_stale_error();
    if (h == nullptr || src == nullptr) return QMV_E_ARG;
    if (h->dev != nullptr) return QMV_E_ARG;  // uploaded once, then read-only
    const qmv::Layout& L = h->layout;
    if (L.scale_f16 != 1) return QMV_E_FORMAT;  // GGUF Q4_0 / Q8_0 scales are f16
    int st = qmv::check_gguf(L, src, nbytes);
    if (st != QMV_OK) return st;
    uint64_t gb = 0;
    st = qmv::gguf_bytes(L.wtype, L.rows, L.cols, &gb);
    if (st != QMV_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_DEVICE;
    uint64_t rexp_off = 0, total = 0;
    if (!device_bytes(L, &rexp_off, &total)) return QMV_E_SHAPE;
    void* img = nullptr;
    void* raw = nullptr;
    hipError_t e = hipMalloc(&img, total);
    if (e != hipSuccess) return device_status(e);
    e = hipMalloc(&raw, gb);
    if (e != hipSuccess) {
        (void)hipFree(img);
        return device_status(e);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* d = static_cast<uint8_t*>(img);
    // the raw blocks to the device, the image zeroed (its padding), then
    // each block's quants and scale moved to the two arrays
    std::vector<int32_t> rexp;
    int32_t dexp = 0;
    e = hipMemcpyAsync(raw, src, gb, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemsetAsync(img, 0, rexp_off, s);
    if (e == hipSuccess)
        e = qmv::launch_gguf_repack(L.wtype, raw, uint64_t{L.rows} * (L.cols / 32), d,
                                    reinterpret_cast<uint16_t*>(d + L.d_offset), s);
    if (e == hipSuccess) e = upload_row_exponents(L, src, true, d + rexp_off, rexp, &dexp, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)hipFree(raw);
    if (e != hipSuccess) {
        (void)hipFree(img);
        return device_status(e);
    }
    h->dev = d;
    h->rexp_offset = rexp_off;
    h->device = dev;
    h->dexp = dexp;
    return QMV_OK;
}

int qmv_destroy(qmv_handle h) {
    if (h == nullptr) return QMV_OK;
    if (h->dev != nullptr) {
        int cur = -1;
        const bool switched = hipGetDevice(&cur) == hipSuccess && cur != h->device &&
                              hipSetDevice(h->device) == hipSuccess;
        (void)hipFree(h->dev);
        if (switched) (void)hipSetDevice(cur);
    }
    delete h;
    return QMV_OK;
}

int qmv_gemv(qmv_handle h, const float* x, float* y, uint32_t batch,
             void* stream) {
    int st = ready(h);
    if (st != QMV_OK) return st;
    if (x == nullptr || y == nullptr || batch == 0) return QMV_E_ARG;
    if (!aligned16(x) || !aligned16(y)) return QMV_E_ARG;
    const qmv::MatView v = view(h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    st = workspace_for(s, qmv::gemv_workspace_bytes(v, batch), &ws);
    if (st != QMV_OK) return st;
    const hipError_t e = qmv::launch_gemv(v, x, y, batch, ws, s);
    if (e == hipErrorNotSupported) return QMV_E_SHAPE;
    return device_status(e);
}

int qmv_gemv_group(const qmv_handle* hs, uint32_t n, const float* x, float* const* ys,
                   uint32_t batch, void* stream) {
    if (hs == nullptr || ys == nullptr || x == nullptr || n == 0 || n > 8 || batch == 0)
        return QMV_E_ARG;
    if (!aligned16(x)) return QMV_E_ARG;
    qmv::MatView ms[8];
    size_t wsb = 0;
    for (uint32_t i = 0; i < n; ++i) {
        const int st = ready(hs[i]);
        if (st != QMV_OK) return st;
        if (ys[i] == nullptr || !aligned16(ys[i])) return QMV_E_ARG;
        ms[i] = view(hs[i]);
        if (ms[i].cols != ms[0].cols) return QMV_E_SHAPE;
        const size_t b = qmv::gemv_workspace_bytes(ms[i], batch);
        wsb = b > wsb ? b : wsb;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    const int st = workspace_for(s, wsb, &ws);
    if (st != QMV_OK) return st;
    return device_status(qmv::launch_gemv_group(ms, n, x, ys, batch, ws, s));
}

int qmv_gemv_gated(qmv_handle w1, qmv_handle w3, uint32_t act, const float* x, float* h,
                   uint32_t batch, void* stream) {
    int st = ready(w1);
    if (st != QMV_OK) return st;
    st = ready(w3);
    if (st != QMV_OK) return st;
    if (x == nullptr || h == nullptr || batch == 0 || act > 1) return QMV_E_ARG;
    if (!aligned16(x) || !aligned16(h)) return QMV_E_ARG;
    const qmv::MatView a = view(w1), b = view(w3);
    if (a.rows != b.rows || a.cols != b.cols) return QMV_E_SHAPE;
    if (a.wtype != b.wtype || a.scale_f16 != b.scale_f16) return QMV_E_FORMAT;
    if (!qmv::gemv_gated_fits(a, b)) return QMV_E_SHAPE;
    return device_status(qmv::launch_gemv_gated(a, b, act, x, h, batch,
                                                static_cast<hipStream_t>(stream)));
}

int qmv_gemm(qmv_handle h, const uint16_t* x_bf16, float* y, uint32_t batch,
             void* stream) {
    int st = ready(h);
    if (st != QMV_OK) return st;
    if (x_bf16 == nullptr || y == nullptr || batch == 0) return QMV_E_ARG;
    if (!aligned16(x_bf16) || !aligned16(y)) return QMV_E_ARG;
    const qmv::MatView v = view(h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    st = workspace_for(s, qmv::gemm_workspace_bytes(v, batch, false), &ws);
    if (st != QMV_OK) return st;
    const hipError_t e = qmv::launch_gemm(v, x_bf16, false, y, batch, ws, s);
    if (e == hipErrorNotSupported) return QMV_E_SHAPE;
    return device_status(e);
}

int qmv_gemm_noalloc(qmv_handle h, const uint16_t* x_bf16, float* y, uint32_t batch,
                     void* stream) {
    int st = ready(h);
    if (st != QMV_OK) return st;
    if (x_bf16 == nullptr || y == nullptr || batch == 0) return QMV_E_ARG;
    if (!aligned16(x_bf16) || !aligned16(y)) return QMV_E_ARG;
    void* ws = nullptr;
    size_t wsb = 0;
    hipError_t e = qmv::gemm_scratch(&ws, &wsb);
    if (e != hipSuccess) return QMV_E_DEVICE;
    e = qmv::launch_gemm_within(view(h), x_bf16, false, y, batch, ws, wsb,
                                static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return QMV_E_SHAPE;
    return device_status(e);
}

int qmv_gemm_q8(qmv_handle h, const int8_t* xq, const float* dx, float* y, uint32_t batch,
                void* stream) {
    int st = ready(h);
    if (st != QMV_OK) return st;
    if (xq == nullptr || dx == nullptr || y == nullptr || batch == 0) return QMV_E_ARG;
    if (!aligned16(xq) || !aligned16(dx) || !aligned16(y)) return QMV_E_ARG;
    const qmv::MatView v = view(h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    st = workspace_for(s, qmv::gemm_q8act_workspace_bytes(v, batch), &ws);
    if (st != QMV_OK) return st;
    const hipError_t e = qmv::launch_gemm_q8act(v, xq, dx, y, batch, static_cast<float*>(ws), s);
    if (e == hipErrorNotSupported) return QMV_E_SHAPE;
    return device_status(e);
}

int qmv_embed_rows(qmv_handle h, const int32_t* ids, uint32_t n, float* out,
                   void* stream) {
    int st = ready(h);
    if (st != QMV_OK) return st;
    if (ids == nullptr || out == nullptr || n == 0) return QMV_E_ARG;
    if (!aligned16(ids) || !aligned16(out)) return QMV_E_ARG;
    return device_status(qmv::launch_embed(view(h), ids, n, out,
                                           static_cast<hipStream_t>(stream)));
}

int qmv_quantize_weights(uint32_t wtype, uint32_t scale_f16, uint32_t rule, uint32_t rows,
                         uint32_t cols, const float* w, void* image, uint64_t image_bytes,
                         uint32_t* status, void* stream) {
    clear_stale_error();
    qmv::Layout L;
    int st = qmv::compute_layout(wtype, scale_f16, rows, cols, &L);
    if (st != QMV_OK) return st;
    if (rule > 1 || (rule == 1 && wtype != QMV_Q4_0)) return QMV_E_ARG;
    if (w == nullptr || image == nullptr || status == nullptr) return QMV_E_ARG;
    if (!aligned16(w) || !aligned16(image) || image_bytes < L.min_span) return QMV_E_ARG;
    if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) return QMV_E_ARG;
    uint8_t* img = static_cast<uint8_t*>(image);
    return device_status(qmv::launch_quantize_weights(
        wtype, scale_f16, rule, w, uint64_t{rows} * (cols / 32), img,
        static_cast<uint32_t>(L.d_offset - L.q_bytes), img + L.d_offset, status,
        static_cast<hipStream_t>(stream)));
}

int qmv_quantize_q8(const float* x, uint64_t n, int8_t* q, float* d,
                    void* stream) {
    clear_stale_error();
    if (x == nullptr || q == nullptr || d == nullptr || n == 0) return QMV_E_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned16(d)) return QMV_E_ARG;
    if (n % 32 != 0) return QMV_E_SHAPE;
    return device_status(qmv::launch_quantize_q8(x, n, q, d,
                                                 static_cast<hipStream_t>(stream)));
}

int qmv_block_dots(qmv_handle h, const int8_t* xq, int32_t* s, void* stream) {
    int st = ready(h);
    if (st != QMV_OK) return st;
    if (xq == nullptr || s == nullptr) return QMV_E_ARG;
    if (!aligned16(xq) || !aligned16(s)) return QMV_E_ARG;
    return device_status(qmv::launch_block_dots(view(h), xq, s,
                                                static_cast<hipStream_t>(stream)));
}

int qmv_read_probe(const void* src, uint64_t nbytes, uint32_t* sink, void* stream) {
    clear_stale_error();
    if (src == nullptr || sink == nullptr || nbytes == 0 || nbytes % 16 != 0) return QMV_E_ARG;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return QMV_E_ARG;
    return device_status(qmv::launch_read_probe(src, nbytes / 16, sink,
                                                static_cast<hipStream_t>(stream)));
}

int qmv_mfma_probe(uint32_t random_operands, uint32_t waves_per_simd, uint32_t iters, uint64_t* clocks,
                   float* sink, void* stream) {
    clear_stale_error();
    if (clocks == nullptr || sink == nullptr || random_operands > 1) return QMV_E_ARG;
    if (waves_per_simd < 1 || waves_per_simd > 2 || iters < 1 || iters > (1u << 20)) return QMV_E_ARG;
    if ((reinterpret_cast<uintptr_t>(clocks) & 7u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return QMV_E_ARG;
    return device_status(qmv::launch_mfma_probe(random_operands != 0, waves_per_simd, iters, clocks, sink,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
