// C-ABI entry points of libqmv: matrix handles, upload, and the compute
// calls that validate their arguments on the host and enqueue the gfx950
// kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>

#include "kernels.h"
#include "qmv.h"
#include "qmv_layout.h"

struct qmv_mat {
    qmv::Layout layout;
    uint8_t* dev = nullptr;  // q at dev, d at dev + d_offset (hipMalloc'd)
    int device = -1;
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

// Common checks of a compute call on an uploaded handle.  The call must run
// on the device that holds the matrix.
int ready(const qmv_mat* h) {
    if (h == nullptr || h->dev == nullptr) return QMV_E_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return QMV_E_DEVICE;
    if (cur != h->device) return QMV_E_ARG;
    return QMV_OK;
}

qmv::MatView view(const qmv_mat* h) {
    const qmv::Layout& L = h->layout;
    return qmv::MatView{h->dev, h->dev + L.d_offset, L.wtype, L.scale_f16,
                        L.rows, L.cols};
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
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, L.full_span);
    if (e != hipSuccess) return device_status(e);
    uint8_t* d = static_cast<uint8_t*>(p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    e = hipMemcpyAsync(d, src, L.min_span, hipMemcpyHostToDevice, s);
    // The device image always carries d's zero padding, whether or not the
    // caller's buffer held it.
    if (e == hipSuccess && L.full_span > L.min_span)
        e = hipMemsetAsync(d + L.min_span, 0, L.full_span - L.min_span, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return device_status(e);
    }
    h->dev = d;
    h->device = dev;
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
    return device_status(qmv::launch_gemv(view(h), x, y, batch,
                                          static_cast<hipStream_t>(stream)));
}

int qmv_gemm(qmv_handle h, const uint16_t* x_bf16, float* y, uint32_t batch,
             void* stream) {
    int st = ready(h);
    if (st != QMV_OK) return st;
    if (x_bf16 == nullptr || y == nullptr || batch == 0) return QMV_E_ARG;
    if (!aligned16(x_bf16) || !aligned16(y)) return QMV_E_ARG;
    return device_status(qmv::launch_gemm(view(h), x_bf16, false, y, batch,
                                          static_cast<hipStream_t>(stream)));
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

int qmv_quantize_q8(const float* x, uint64_t n, int8_t* q, float* d,
                    void* stream) {
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

}  // extern "C"
