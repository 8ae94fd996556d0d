// Host-side rules of the qmv library that need no GPU: array sizes, the
// q8_mask class rule, the checks applied to a matrix's bytes, status text.
// This translation unit makes no HIP call, so these rules can be exercised
// on a machine without a GPU.
//
// Source: Krafla, ".mlb model, version 1" format page - "Body" (the
// two-array quantized matrix, 64-byte padding), "Q8_0" (no -128 quant), the
// q8_mask paragraph, and "Validation done by the loader" (error classes,
// overflow-checked size arithmetic).
#include <cstddef>
#include <cmath>
#include <cstdint>

#include "qmv.h"
#include "qmv_layout.h"

namespace qmv {

namespace {
constexpr uint64_t kDimLimit = uint64_t{1} << 24;

// a + b and a * b with overflow detection (u64).
bool add_ok(uint64_t a, uint64_t b, uint64_t* out) {
    return !__builtin_add_overflow(a, b, out);
}
bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
    return !__builtin_mul_overflow(a, b, out);
}
bool round_up64(uint64_t n, uint64_t* out) {
    uint64_t t;
    if (!add_ok(n, 63, &t)) return false;
    *out = t & ~uint64_t{63};
    return true;
}
}  // namespace

int compute_layout(uint32_t wtype, uint32_t scale_f16, uint32_t rows,
                   uint32_t cols, Layout* L) {
    if (wtype != QMV_Q8_0 && wtype != QMV_Q4_0) return QMV_E_FORMAT;
    if (scale_f16 > 1) return QMV_E_FORMAT;
    if (rows == 0 || cols == 0 || (cols & 31) != 0) return QMV_E_SHAPE;
    if (rows > kDimLimit || cols > kDimLimit) return QMV_E_SHAPE;
    uint64_t elems, q_bytes, d_bytes, d_off, min_span, d_pad, full;
    if (!mul_ok(rows, cols, &elems)) return QMV_E_SHAPE;
    q_bytes = (wtype == QMV_Q8_0) ? elems : elems / 2;
    if (!mul_ok(elems / 32, scale_f16 ? 2 : 4, &d_bytes)) return QMV_E_SHAPE;
    if (!round_up64(q_bytes, &d_off)) return QMV_E_SHAPE;
    if (!add_ok(d_off, d_bytes, &min_span)) return QMV_E_SHAPE;
    if (!round_up64(d_bytes, &d_pad) || !add_ok(d_off, d_pad, &full))
        return QMV_E_SHAPE;
    L->wtype = wtype;
    L->scale_f16 = scale_f16;
    L->rows = rows;
    L->cols = cols;
    L->q_bytes = q_bytes;
    L->d_offset = d_off;
    L->d_bytes = d_bytes;
    L->min_span = min_span;
    L->full_span = full;
    return QMV_OK;
}

int check_bytes(const Layout& L, const void* src, uint64_t nbytes) {
    if (src == nullptr) return QMV_E_ARG;
    if (nbytes < L.min_span) return QMV_E_FORMAT;
    if (L.wtype == QMV_Q8_0) {
        // A Q8_0 quant of -128 (byte 0x80) is refused; the scan reads the q
        // array eight bytes at a time.
        const uint8_t* p = static_cast<const uint8_t*>(src);
        uint64_t i = 0;
        for (; i + 8 <= L.q_bytes; i += 8) {
            uint64_t w;
            __builtin_memcpy(&w, p + i, 8);
            // a byte equals 0x80 iff (b ^ 0x80) == 0: classic zero-byte test
            uint64_t v = w ^ 0x8080808080808080ull;
            if ((v - 0x0101010101010101ull) & ~v & 0x8080808080808080ull) {
                for (uint64_t j = i; j < i + 8; ++j)
                    if (p[j] == 0x80) return QMV_E_FORMAT;
            }
        }
        for (; i < L.q_bytes; ++i)
            if (p[i] == 0x80) return QMV_E_FORMAT;
    }
    return QMV_OK;
}

int gguf_bytes(uint32_t wtype, uint32_t rows, uint32_t cols, uint64_t* bytes) {
    Layout L;
    const int st = compute_layout(wtype, 1, rows, cols, &L);
    if (st != QMV_OK) return st;
    uint64_t n;
    if (!mul_ok(uint64_t{rows} * (cols / 32), wtype == QMV_Q8_0 ? 34 : 18, &n)) return QMV_E_SHAPE;
    *bytes = n;
    return QMV_OK;
}

int check_gguf(const Layout& L, const void* src, uint64_t nbytes) {
    if (src == nullptr) return QMV_E_ARG;
    uint64_t need;
    const int st = gguf_bytes(L.wtype, L.rows, L.cols, &need);
    if (st != QMV_OK) return st;
    if (nbytes < need) return QMV_E_FORMAT;
    if (L.wtype == QMV_Q8_0) {
        const uint8_t* p = static_cast<const uint8_t*>(src);
        const uint64_t blocks = need / 34;
        for (uint64_t k = 0; k < blocks; ++k) {
            const uint8_t* b = p + 34 * k + 2;
            for (int j = 0; j < 32; ++j)
                if (b[j] == 0x80) return QMV_E_FORMAT;
        }
    }
    return QMV_OK;
}

namespace {
// Binary exponent E of a finite magnitude a > 0 (a in [2^(E-1), 2^E)).
int32_t exponent_of(float a) {
    int e = 0;
    (void)std::frexp(a, &e);
    return e;
}

// Largest finite magnitude among scales held as f16 bits (low 15 bits
// compared as integers: binary16 magnitudes order like their bit patterns),
// or 0 when there is none.
struct F16Max {
    uint16_t m = 0;
    void add(uint16_t b) {
        b &= 0x7FFF;
        if (b < 0x7C00 && b > m) m = b;  // inf and NaN patterns are skipped
    }
    int32_t exponent() const {
        if (m == 0) return 0;
        const int e = m >> 10, f = m & 0x3FF;
        const float a = e == 0 ? std::ldexp(static_cast<float>(f), -24)
                               : std::ldexp(static_cast<float>(1024 + f), e - 25);
        return exponent_of(a);
    }
};

// The same for float32 scales (magnitudes order like their low 31 bits).
struct F32Max {
    uint32_t m = 0;
    void add(uint32_t b) {
        b &= 0x7FFFFFFFu;
        if (b < 0x7F800000u && b > m) m = b;
    }
    int32_t exponent() const {
        if (m == 0) return 0;
        float a;
        __builtin_memcpy(&a, &m, 4);
        return exponent_of(a);
    }
};
}  // namespace

void scale_exponents(const Layout& L, const void* src, bool gguf, int32_t* row_exp,
                     int32_t* mat_exp) {
    const uint8_t* p = static_cast<const uint8_t*>(src);
    const uint64_t nblk = L.cols / 32;
    if (gguf || L.scale_f16) {
        // GGUF: the f16 scale opens each 18- or 34-byte block; .mlb: the d array
        const uint64_t stride = gguf ? (L.wtype == QMV_Q8_0 ? 34 : 18) : 2;
        const uint8_t* d = gguf ? p : p + L.d_offset;
        F16Max all;
        for (uint64_t r = 0; r < L.rows; ++r) {
            F16Max row;
            const uint8_t* dr = d + r * nblk * stride;
            for (uint64_t b = 0; b < nblk; ++b) {
                uint16_t v;
                __builtin_memcpy(&v, dr + b * stride, 2);
                row.add(v);
            }
            all.add(row.m);
            if (row_exp) row_exp[r] = row.exponent();
        }
        *mat_exp = all.exponent();
        return;
    }
    const uint8_t* d = p + L.d_offset;
    F32Max all;
    for (uint64_t r = 0; r < L.rows; ++r) {
        F32Max row;
        const uint8_t* dr = d + r * nblk * 4;
        for (uint64_t b = 0; b < nblk; ++b) {
            uint32_t v;
            __builtin_memcpy(&v, dr + b * 4, 4);
            row.add(v);
        }
        all.add(row.m);
        if (row_exp) row_exp[r] = row.exponent();
    }
    *mat_exp = all.exponent();
}

}  // namespace qmv

extern "C" {

int qmv_span(uint32_t wtype, uint32_t scale_f16, uint32_t rows, uint32_t cols,
             uint64_t* q_bytes, uint64_t* d_offset, uint64_t* d_bytes,
             uint64_t* min_span) {
    qmv::Layout L;
    int st = qmv::compute_layout(wtype, scale_f16, rows, cols, &L);
    if (st != QMV_OK) return st;
    if (q_bytes) *q_bytes = L.q_bytes;
    if (d_offset) *d_offset = L.d_offset;
    if (d_bytes) *d_bytes = L.d_bytes;
    if (min_span) *min_span = L.min_span;
    return QMV_OK;
}

int qmv_gguf_span(uint32_t wtype, uint32_t rows, uint32_t cols, uint64_t* bytes) {
    if (bytes == nullptr) return QMV_E_ARG;
    return qmv::gguf_bytes(wtype, rows, cols, bytes);
}

int qmv_class_wtype(uint32_t file_wtype, uint32_t q8_mask, uint32_t class_bit,
                    uint32_t shared_classifier, uint32_t* wtype_out) {
    if (wtype_out == nullptr) return QMV_E_ARG;
    if (file_wtype != QMV_Q8_0 && file_wtype != QMV_Q4_0) return QMV_E_FORMAT;
    // exactly one of the seven class bits
    if (class_bit == 0 || class_bit > 64 || (class_bit & (class_bit - 1)) != 0)
        return QMV_E_ARG;
    if (file_wtype == QMV_Q8_0) {
        *wtype_out = QMV_Q8_0;
        return QMV_OK;
    }
    uint32_t mask_bits = class_bit;
    // With a shared classifier the embedding matrix is the classifier too:
    // either of its two class bits selects Q8_0 for it.
    if (shared_classifier != 0 && class_bit <= 2) mask_bits = 3;
    *wtype_out = (q8_mask & mask_bits) ? QMV_Q8_0 : QMV_Q4_0;
    return QMV_OK;
}

const char* qmv_status_str(int status) {
    switch (status) {
        case QMV_OK: return "ok";
        case QMV_E_ARG: return "invalid argument";
        case QMV_E_FORMAT: return "bad matrix format or bytes";
        case QMV_E_SHAPE: return "bad matrix shape";
        case QMV_E_DEVICE: return "HIP runtime error";
        case QMV_E_NOMEM: return "out of memory";
        default: return "unknown status";
    }
}

}  // extern "C"
