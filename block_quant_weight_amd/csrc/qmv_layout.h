// Shape and byte layout of one quantized matrix (no HIP types).
#pragma once
#include <cstdint>

namespace qmv {

// The two arrays of a quantized matrix as the .mlb format lays them out:
// q (quants) at byte 0, d (one scale per 32 weights) at d_offset =
// pad64(q_bytes); min_span = d_offset + d_bytes, full_span adds d's padding.
struct Layout {
    uint32_t wtype = 0, scale_f16 = 0, rows = 0, cols = 0;
    uint64_t q_bytes = 0, d_offset = 0, d_bytes = 0, min_span = 0, full_span = 0;
};

// QMV_OK or QMV_E_FORMAT / QMV_E_SHAPE; fills *L on success.
int compute_layout(uint32_t wtype, uint32_t scale_f16, uint32_t rows,
                   uint32_t cols, Layout* L);

// Checks a host buffer holding the matrix's bytes: long enough, and no
// Q8_0 quant equal to -128.  QMV_OK, QMV_E_ARG or QMV_E_FORMAT.
int check_bytes(const Layout& L, const void* src, uint64_t nbytes);

// GGUF block data of a Q4_0 / Q8_0 matrix: rows * cols / 32 blocks of 18 /
// 34 bytes (an f16 scale, then the quants).  QMV_OK or QMV_E_FORMAT /
// QMV_E_SHAPE; *bytes on success.
int gguf_bytes(uint32_t wtype, uint32_t rows, uint32_t cols, uint64_t* bytes);

// Checks GGUF block data for a matrix of layout L (f16 scales): long enough,
// no Q8_0 quant equal to -128.  QMV_OK, QMV_E_ARG or QMV_E_FORMAT.
int check_gguf(const Layout& L, const void* src, uint64_t nbytes);

// Binary exponent E (largest magnitude in [2^(E-1), 2^E)) of the largest
// finite scale magnitude of each row (row_exp[r], if row_exp is not null)
// and of the whole matrix (*mat_exp) of a checked buffer: the two-array
// image (gguf false) or GGUF block data (gguf true, the f16 scale at the
// start of each block).  0 where every finite scale is zero.  Non-finite
// scales are skipped: their products are non-finite however the weights
// are scaled.  Kernels that hold weights in f16 scale a row by 2^(8 - E),
// so that its largest weight stays below 2^15.
void scale_exponents(const Layout& L, const void* src, bool gguf, int32_t* row_exp,
                     int32_t* mat_exp);

}  // namespace qmv
