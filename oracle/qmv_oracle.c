/*
 * Plain CPU oracle for the block-quantized weight matrix x activation product.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  It shares
 * no code, header, table or constant with the HIP library under
 * block_quant_weight_amd/: the two are written separately from the format
 * description so that each checks the other.
 *
 * Source of every rule: Krafla, "File formats: .mlb model, version 1, and
 * .mlt tokenizer" (called "the .mlb page" below), in particular
 *   - "Body": row-major matrices, y[r] = sum_c W[r][c] x[c];
 *   - the two-array quantized matrix (q, then d; one scale per 32 consecutive
 *     weights of a row; f32, or IEEE f16 when scale_f16 is 1) and the
 *     64-byte zero padding of each array;
 *   - "Q8_0" (w = q x d, a byte of -128 is rejected);
 *   - "Q4_0" (elements 0..15 of a block in the low four bits of its 16
 *     bytes, elements 16..31 in the high four bits, w = (nibble - 8) x d);
 *   - "Quantization rule" (activation quantizer, exact float32 operations);
 *   - the header table ("wtype", "scale_f16", "q8_mask", "shared_classifier")
 *     and the q8_mask class-bit paragraph;
 *   - "Validation done by the loader" (ML_E_FORMAT / ML_E_SHAPE classes and
 *     overflow-checked size arithmetic).
 *
 * Everything is scalar, written in the order the page states it, and the
 * products are accumulated in IEEE binary64 in column order.  Build with
 * -ffp-contract=off so that no multiply-add is fused.
 *
 * Readings where the page leaves a step open (all listed in the design notes
 * of the repository):
 *   - blocks (and their scales) are in row-major order: row r's C/32 blocks
 *     are consecutive, block k = r*(C/32) + c/32;
 *   - a dequantized weight is one float32 multiply fl32(v * d) (round to
 *     nearest even, signed zero and subnormals per IEEE); the exact value
 *     v * d (at most 7 + 24 significant bits) is what the f64 product uses;
 *   - rows and cols are each limited to 2^24 (the only limit that survives
 *     in the page's garbled limits sentence); cols must be a multiple of 32.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* Outcome classes of the oracle's checks; the Python wrapper maps them to
 * names ("ok", "arg", "format", "shape"). */
#define ORC_OK 0
#define ORC_ARG 1
#define ORC_FORMAT 2
#define ORC_SHAPE 3

#define ORC_Q8_0 1 /* header "wtype": 1 = Q8_0 */
#define ORC_Q4_0 2 /* header "wtype": 2 = Q4_0 */

static const uint64_t ORC_DIM_LIMIT = (uint64_t)1 << 24;

/* Round n up to a multiple of 64 (the arrays' zero padding). */
static uint64_t orc_pad64(uint64_t n) { return ((n + 63) / 64) * 64; }

/*
 * Sizes of one quantized matrix's two arrays.
 * out[0] = bytes of q, out[1] = offset of d (q padded to 64),
 * out[2] = bytes of d, out[3] = smallest legal span (d offset + d bytes,
 * the trailing padding being optional), out[4] = span with trailing pad.
 */
int orc_span(uint32_t wtype, uint32_t scale_f16, uint64_t rows, uint64_t cols,
             uint64_t out[5]) {
    if (wtype != ORC_Q8_0 && wtype != ORC_Q4_0) return ORC_FORMAT;
    if (scale_f16 != 0 && scale_f16 != 1) return ORC_FORMAT;
    if (rows == 0 || cols == 0) return ORC_SHAPE;
    if (cols % 32 != 0) return ORC_SHAPE;
    if (rows > ORC_DIM_LIMIT || cols > ORC_DIM_LIMIT) return ORC_SHAPE;
    /* With both factors at most 2^24 the products below stay under 2^50,
     * far inside uint64_t; they are still checked. */
    uint64_t n = rows * cols;
    if (n / rows != cols) return ORC_SHAPE;
    uint64_t q_bytes = (wtype == ORC_Q8_0) ? n : n / 2;
    uint64_t n_blocks = n / 32;
    uint64_t d_bytes = n_blocks * (scale_f16 ? 2u : 4u);
    uint64_t d_off = orc_pad64(q_bytes);
    if (d_off < q_bytes) return ORC_SHAPE;
    uint64_t min_span = d_off + d_bytes;
    if (min_span < d_off) return ORC_SHAPE;
    uint64_t full = d_off + orc_pad64(d_bytes);
    if (full < d_off) return ORC_SHAPE;
    out[0] = q_bytes;
    out[1] = d_off;
    out[2] = d_bytes;
    out[3] = min_span;
    out[4] = full;
    return ORC_OK;
}

/*
 * IEEE binary16 -> exact value, written out from the format's definition:
 * 1 sign bit, 5 exponent bits with bias 15, 10 fraction bits; exponent 0 is
 * zero or subnormal (fraction * 2^-24), exponent 31 is infinity or NaN.
 */
double orc_f16_value(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25);
    }
    return sign ? -v : v;
}

/* Read little-endian integers byte by byte, so the result does not depend on
 * the host's byte order ("Everything is little-endian"). */
static uint16_t orc_le16(const uint8_t *p) {
    return (uint16_t)(p[0] | ((uint16_t)p[1] << 8));
}
static uint32_t orc_le32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
           ((uint32_t)p[3] << 24);
}

/* Scale k of the d array, as the float32 the runtime uses. */
static float orc_scale(const uint8_t *img, uint64_t d_off, uint32_t scale_f16,
                       uint64_t k) {
    if (scale_f16) {
        uint16_t h = orc_le16(img + d_off + 2 * k);
        /* The conversion to f32 is exact: every binary16 value is a binary32
         * value. */
        return (float)orc_f16_value(h);
    }
    uint32_t bits = orc_le32(img + d_off + 4 * k);
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* Integer quant v of element (r, c): Q8_0 is the int8 byte; Q4_0 is the
 * nibble minus 8, low nibble for elements 0..15 of the block, high nibble
 * for elements 16..31. */
static int orc_quant(const uint8_t *img, uint32_t wtype, uint64_t cols,
                     uint64_t r, uint64_t c) {
    if (wtype == ORC_Q8_0) {
        return (int)(int8_t)img[r * cols + c];
    }
    uint64_t k = r * (cols / 32) + c / 32;
    uint64_t j = c % 32;
    uint8_t byte = img[16 * k + (j % 16)];
    int nib = (j < 16) ? (byte & 0xF) : (byte >> 4);
    return nib - 8;
}

/* Public form of the quant accessor for tests: v at (r, c). */
int orc_quant_at(const uint8_t *img, uint32_t wtype, uint64_t cols, uint64_t r,
                 uint64_t c) {
    return orc_quant(img, wtype, cols, r, c);
}

/* Public form of the scale accessor for tests: d of block k, as f32. */
float orc_scale_at(const uint8_t *img, uint64_t d_off, uint32_t scale_f16,
                   uint64_t k) {
    return orc_scale(img, d_off, scale_f16, k);
}

/*
 * Dequantized rows: out[i][c] = fl32(v * d) for row ids[i], one float32
 * multiply.  This is the value an embedding-row gather returns.
 */
void orc_dequant_rows(const uint8_t *img, uint32_t wtype, uint32_t scale_f16,
                      uint64_t rows, uint64_t cols, const int64_t *ids,
                      uint64_t n, float *out) {
    uint64_t span[5];
    if (orc_span(wtype, scale_f16, rows, cols, span) != ORC_OK) return;
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t r = (uint64_t)ids[i];
        for (uint64_t c = 0; c < cols; ++c) {
            int v = orc_quant(img, wtype, cols, r, c);
            float d = orc_scale(img, span[1], scale_f16, r * (cols / 32) + c / 32);
            float w = (float)v * d;
            out[i * cols + c] = w;
        }
    }
}

/* Activation element (t, c): float32, or bfloat16 bits widened exactly
 * (a bfloat16 is the top half of a float32). */
static double orc_act(const void *x, int x_bf16, uint64_t cols, uint64_t t,
                      uint64_t c) {
    if (x_bf16) {
        uint16_t b = ((const uint16_t *)x)[t * cols + c];
        uint32_t bits = (uint32_t)b << 16;
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    return (double)((const float *)x)[t * cols + c];
}

/*
 * The product y[t][r] = sum_c W[r][c] * x[t][c] for the selected rows,
 * computed in binary64 in column order from the exact weights (double)v *
 * (double)d, together with the per-row norm sum_c |W[r][c]| |x[t][c]| that
 * the tolerance is stated against.  ref and norm are [batch][n_sel].
 */
void orc_product(const uint8_t *img, uint32_t wtype, uint32_t scale_f16,
                 uint64_t rows, uint64_t cols, const void *x, int x_bf16,
                 uint64_t batch, const int64_t *sel, uint64_t n_sel,
                 double *ref, double *norm) {
    uint64_t span[5];
    if (orc_span(wtype, scale_f16, rows, cols, span) != ORC_OK) return;
    for (uint64_t t = 0; t < batch; ++t) {
        for (uint64_t i = 0; i < n_sel; ++i) {
            uint64_t r = (uint64_t)sel[i];
            double acc = 0.0, nrm = 0.0;
            for (uint64_t c = 0; c < cols; ++c) {
                int v = orc_quant(img, wtype, cols, r, c);
                float d = orc_scale(img, span[1], scale_f16, r * (cols / 32) + c / 32);
                double w = (double)v * (double)d;
                double a = orc_act(x, x_bf16, cols, t, c);
                acc += w * a;
                nrm += fabs(w) * fabs(a);
            }
            ref[t * n_sel + i] = acc;
            norm[t * n_sel + i] = nrm;
        }
    }
}

/*
 * Feed-forward activation of the .mlb header field "act" (code 0 selects
 * SiLU, code 1 the tanh form of GELU, the Gemma convention), in binary64:
 *   SiLU(a) = a / (1 + e^-a)   (a times the logistic sigmoid);
 *   GELU(a) = a/2 * (1 + tanh(u)),  u = sqrt(2/pi) * (a + 0.044715 a^3)
 *             (Hendrycks and Gimpel's tanh approximation of a * Phi(a)),
 *             written as a / (1 + e^(-2u)): the same function, because
 *             1 + tanh(u) = 2 / (1 + e^(-2u)), without the cancellation of
 *             1 + tanh(u) that leaves no correct digit even in binary64 once
 *             u < -19.
 * The gated hidden state of a layer is act(w1 . x) * (w3 . x): w1 is the
 * gate and w3 the up projection in the page's body table.
 */
double orc_ffn_act(double a, uint32_t act) {
    if (act == 0) return a / (1.0 + exp(-a));
    const double k = sqrt(2.0 / 3.14159265358979323846);
    const double u = k * (a + 0.044715 * a * a * a);
    return a / (1.0 + exp(-2.0 * u));
}

/* h[i] = act(y1[i]) * y3[i] for n elements (the gated output from the two
 * products of orc_product). */
void orc_gated(const double *y1, const double *y3, uint64_t n, uint32_t act, double *h) {
    for (uint64_t i = 0; i < n; ++i) h[i] = orc_ffn_act(y1[i], act) * y3[i];
}

/*
 * Activation quantizer (the .mlb page, "Quantization rule" section), per
 * block of 32 values, in float32: the block's scale is its largest
 * magnitude divided by 127 (zero, with all codes zero, when that magnitude
 * is below 1e-30); each code is the value times the reciprocal of the scale
 * (127 over the largest magnitude), rounded to the nearest integer with
 * halves away from zero, and kept within [-127, 127].  The operations come
 * in the order the section gives them, each rounded on its own (no fused
 * multiply-add).  n must be a multiple of 32.
 */
void orc_quantize_q8(const float *x, uint64_t n, int8_t *q, float *d) {
    for (uint64_t b = 0; b < n / 32; ++b) {
        const float *xb = x + 32 * b;
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            float a = fabsf(xb[j]);
            if (a > amax) amax = a;
        }
        if (amax < 1e-30f) {
            d[b] = 0.0f;
            for (int j = 0; j < 32; ++j) q[32 * b + j] = 0;
            continue;
        }
        d[b] = amax / 127.0f;
        float id = 127.0f / amax;
        for (int j = 0; j < 32; ++j) {
            volatile float t = xb[j] * id; /* separate rounding of the product */
            float u = t + copysignf(0.5f, xb[j]);
            float tr = truncf(u);
            int qi;
            if (tr > 127.0f) qi = 127;
            else if (tr < -127.0f) qi = -127;
            else qi = (int)tr;
            q[32 * b + j] = (int8_t)qi;
        }
    }
}

/*
 * Per-block integer dot products of the weight quants with quantized
 * activations: s[r][b] = sum_{j<32} v[r][32b+j] * xq[32b+j], exact in int32
 * (|s| <= 32 * 127 * 127).
 */
void orc_block_dots(const uint8_t *img, uint32_t wtype, uint64_t rows,
                    uint64_t cols, const int8_t *xq, int32_t *s) {
    uint64_t nb = cols / 32;
    for (uint64_t r = 0; r < rows; ++r) {
        for (uint64_t b = 0; b < nb; ++b) {
            int32_t acc = 0;
            for (uint64_t j = 0; j < 32; ++j) {
                acc += orc_quant(img, wtype, cols, r, 32 * b + j) * (int32_t)xq[32 * b + j];
            }
            s[r * nb + b] = acc;
        }
    }
}

/*
 * Product on Q8_0-quantized activations (the page's CPU path: activations
 * quantized per block of 32 by the "Quantization rule", then per-block
 * integer dot products): for each selected row r and token t,
 *   ref[t][r]   = sum_b dw[r,b] * dx[t,b] * s[t,r,b],
 *   bound[t][r] = sum_b |dw[r,b] * dx[t,b] * s[t,r,b]|,
 *   s[t,r,b]    = sum_j v[r,32b+j] * xq[t,32b+j]   (exact, int32),
 * in binary64 in block order, dw the decoded scale and dx[t,b] the
 * activation block's scale.  xq is int8 [batch][cols], dx float32
 * [batch][cols/32]; ref and bound are [batch][n_sel].
 */
void orc_gemm_q8act(const uint8_t *img, uint32_t wtype, uint32_t scale_f16,
                    uint64_t rows, uint64_t cols, const int8_t *xq, const float *dx,
                    uint64_t batch, const int64_t *sel, uint64_t n_sel, double *ref,
                    double *bound) {
    uint64_t span[5];
    if (orc_span(wtype, scale_f16, rows, cols, span) != ORC_OK) return;
    uint64_t nb = cols / 32;
    for (uint64_t t = 0; t < batch; ++t) {
        for (uint64_t i = 0; i < n_sel; ++i) {
            uint64_t r = (uint64_t)sel[i];
            double acc = 0.0, bnd = 0.0;
            for (uint64_t b = 0; b < nb; ++b) {
                int32_t sb = 0;
                for (uint64_t j = 0; j < 32; ++j)
                    sb += orc_quant(img, wtype, cols, r, 32 * b + j) *
                          (int32_t)xq[t * cols + 32 * b + j];
                double dw = (double)orc_scale(img, span[1], scale_f16, r * nb + b);
                double term = dw * (double)dx[t * nb + b] * (double)sb;
                acc += term;
                bnd += fabs(term);
            }
            ref[t * n_sel + i] = acc;
            bound[t * n_sel + i] = bnd;
        }
    }
}

/*
 * Storage type of one matrix class (the q8_mask paragraph).  Class bits:
 * 1 tok_emb, 2 wcls, 4 wq/wk (wg, lqkv), 8 wv (lz), 16 wo (lout),
 * 32 w1/w3, 64 w2.  A Q8_0 file stores every matrix as Q8_0.  In a Q4_0
 * file a set class bit stores the class as Q8_0; with a shared classifier
 * the embedding (which is then also the classifier) is Q8_0 if bit 1 or
 * bit 2 is set.  Reading: asking for the classifier class of a file with a
 * shared classifier names the same matrix as the embedding.
 */
int orc_class_wtype(uint32_t file_wtype, uint32_t q8_mask, uint32_t class_bit,
                    uint32_t shared_classifier, uint32_t *out) {
    if (file_wtype != ORC_Q8_0 && file_wtype != ORC_Q4_0) return ORC_FORMAT;
    switch (class_bit) {
        case 1: case 2: case 4: case 8: case 16: case 32: case 64: break;
        default: return ORC_ARG;
    }
    if (file_wtype == ORC_Q8_0) {
        *out = ORC_Q8_0;
        return ORC_OK;
    }
    uint32_t bits = class_bit;
    if (shared_classifier && (class_bit == 1 || class_bit == 2)) bits = 1u | 2u;
    *out = (q8_mask & bits) ? ORC_Q8_0 : ORC_Q4_0;
    return ORC_OK;
}

/*
 * Checks the loader applies to one matrix's bytes: a buffer shorter than the
 * arrays the shape implies, or a Q8_0 quant equal to -128, is a format
 * error.  Padding bytes are not inspected (the page writes them as zero but
 * does not list them among the checks).
 */
int orc_check_image(uint32_t wtype, uint32_t scale_f16, uint64_t rows,
                    uint64_t cols, const uint8_t *img, uint64_t nbytes) {
    uint64_t span[5];
    int st = orc_span(wtype, scale_f16, rows, cols, span);
    if (st != ORC_OK) return st;
    if (img == NULL) return ORC_ARG;
    if (nbytes < span[3]) return ORC_FORMAT;
    if (wtype == ORC_Q8_0) {
        for (uint64_t i = 0; i < span[0]; ++i)
            if (img[i] == 0x80) return ORC_FORMAT;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * GGUF block data (minfer, "GGUF load" page, section "Quantized sizing: 32
 * values in 18 bytes"): a Q4_0 or Q8_0 tensor is a run of blocks, each an
 * f16 scale d followed by the block's quants - BlockQ4_0 { d: f16,
 * qs: 16 bytes } (18 bytes), BlockQ8_0 { d: f16, qs: 32 int8 } (34 bytes);
 * the tensor's size is its element count / 32 x the block size.
 * Readings (the page names the blocks but not these points): the blocks are
 * in the same row-major order as the .mlb arrays (a tensor's first dimension
 * is the row length, so block k covers row k / (C/32)); the scale is
 * little-endian; and the 16 Q4_0 bytes hold their 32 elements in the .mlb
 * page's nibble order (byte j: element j low, element j + 16 high).
 * ---------------------------------------------------------------------- */

/* bytes[0] = rows * cols / 32 * (18 | 34), overflow-checked. */
int orc_gguf_span(uint32_t wtype, uint64_t rows, uint64_t cols, uint64_t *bytes) {
    if (wtype != ORC_Q8_0 && wtype != ORC_Q4_0) return ORC_FORMAT;
    if (rows == 0 || cols == 0 || cols % 32 != 0) return ORC_SHAPE;
    if (rows > ORC_DIM_LIMIT || cols > ORC_DIM_LIMIT) return ORC_SHAPE;
    uint64_t blocks = rows * (cols / 32); /* <= 2^43: no overflow */
    uint64_t bsize = (wtype == ORC_Q8_0) ? 34 : 18;
    if (blocks > UINT64_MAX / bsize) return ORC_SHAPE;
    *bytes = blocks * bsize;
    return ORC_OK;
}

/* The loader's checks on GGUF block data: long enough, no Q8_0 quant byte
 * of -128 (the .mlb rule, applied to the matrix whatever file holds it). */
int orc_check_gguf(uint32_t wtype, uint64_t rows, uint64_t cols,
                   const uint8_t *src, uint64_t nbytes) {
    uint64_t need;
    int st = orc_gguf_span(wtype, rows, cols, &need);
    if (st != ORC_OK) return st;
    if (src == NULL) return ORC_ARG;
    if (nbytes < need) return ORC_FORMAT;
    if (wtype == ORC_Q8_0) {
        uint64_t blocks = need / 34;
        for (uint64_t k = 0; k < blocks; ++k)
            for (int j = 0; j < 32; ++j)
                if (src[34 * k + 2 + j] == 0x80) return ORC_FORMAT;
    }
    return ORC_OK;
}

/* The .mlb image (q array, zero pad, f16 d array, zero pad; full_span
 * bytes, scale_f16 = 1) holding the same weights as the GGUF blocks. */
int orc_gguf_to_image(uint32_t wtype, uint64_t rows, uint64_t cols,
                      const uint8_t *src, uint8_t *img) {
    uint64_t span[5], need;
    int st = orc_span(wtype, 1, rows, cols, span);
    if (st != ORC_OK) return st;
    st = orc_gguf_span(wtype, rows, cols, &need);
    if (st != ORC_OK) return st;
    memset(img, 0, span[4]);
    uint64_t qb = (wtype == ORC_Q8_0) ? 32 : 16, bsize = 2 + qb;
    uint64_t blocks = rows * (cols / 32);
    for (uint64_t k = 0; k < blocks; ++k) {
        const uint8_t *b = src + k * bsize;
        memcpy(img + k * qb, b + 2, qb);            /* quants of block k */
        memcpy(img + span[1] + 2 * k, b, 2);        /* its f16 scale */
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Weight writer (the .mlb page, "Quantization rule" and the two paragraphs
 * after it), per block of 32 consecutive weights of a row, in float32
 * operations rounded one at a time:
 *   - Q8_0, f32 scales: the quantization rule itself (orc_quantize_q8);
 *   - Q8_0, f16 scales: d = amax / 127 rounded to the nearest f16, then
 *     q = trunc(x * (1 / d) + copysign(0.5, x)) with d as rounded,
 *     clamped to [-127, 127]; a d above 65504 cannot be stored and is
 *     refused;
 *   - Q4_0, "round" rule (the rounding the page attributes to llama.cpp):
 *     d = (the element of largest magnitude) / -8, level =
 *     trunc(x * (1 / d) + 8.5), at most 15, stored as the nibble; with f16
 *     scales d is stored rounded to f16.
 * Readings (the page leaves these open): the element of largest magnitude
 * is the first one reaching it; a Q4_0 block with d = 0 uses 1 / d = 0
 * (every nibble 8, every weight 0), as llama.cpp does, and so does one whose
 * 1 / d overflows (|d| < 2^-128, weights below 2^-125); the Q4_0 levels use
 * the float32 d also when the stored scale is its f16 rounding (only the
 * Q8_0 rule names the rounded d for the codes); an f16 Q8_0 scale that
 * rounds to 0 from amax >= 1e-30 gives q = 0 (every weight is 0 either
 * way); the f16 rounding is the oracle's own round-to-nearest-even of the
 * float32 value; a Q4_0 f16 scale above 65504 is refused like a Q8_0 one.
 * The least-squares Q4_0 search is orc_quantize_q4_search below.
 * Returns ORC_OK, ORC_SHAPE / ORC_FORMAT as orc_span, or ORC_FORMAT for a
 * scale that does not fit f16 (then img is unspecified).  img receives
 * full_span bytes (both pads zero).
 * ---------------------------------------------------------------------- */

/* float32 -> IEEE binary16 bits, round to nearest even (finite inputs and
 * infinities; NaN becomes a quiet NaN). */
uint16_t orc_f16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t ex = (u >> 23) & 0xFFu, man = u & 0x7FFFFFu;
    if (ex == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    /* value = 1.man x 2^(ex - 127) for normal f32; f16 normal exponent range
     * is [-14, 15], subnormals step 2^-24 */
    int e = (int)ex - 127;
    if (ex == 0) return sign; /* f32 subnormals are far below f16's range */
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    /* integer significand with the implicit bit: m24 = 1.man x 2^23 */
    uint32_t m24 = man | 0x800000u;
    /* the f16 result, in units of its last place: shift right by s bits */
    int s = (e >= -14) ? 13 : 13 + (-14 - e); /* normals keep 10 bits */
    if (s > 24) return sign;                   /* below half the smallest subnormal */
    uint32_t q = m24 >> s, rem = m24 & ((1u << s) - 1u), half = 1u << (s - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    if (e >= -14) {
        /* q in [2^10, 2^11]; 2^11 carries into the exponent */
        int E = e + 15;
        if (q == 0x800u) { q = 0x400u; ++E; }
        if (E > 30) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)(q & 0x3FFu));
    }
    /* subnormal (q may round up to 0x400, the smallest normal: same bits) */
    return (uint16_t)(sign | (uint16_t)q);
}

static float orc_trunc_clamp(float u, float lo, float hi) {
    float t = truncf(u);
    if (t > hi) return hi;
    if (t < lo) return lo;
    return t;
}

int orc_quantize_weights(uint32_t wtype, uint32_t scale_f16, uint64_t rows,
                         uint64_t cols, const float *w, uint8_t *img) {
    uint64_t span[5];
    int st = orc_span(wtype, scale_f16, rows, cols, span);
    if (st != ORC_OK) return st;
    memset(img, 0, span[4]);
    uint64_t nblk = rows * (cols / 32);
    uint8_t *dptr = img + span[1];
    for (uint64_t k = 0; k < nblk; ++k) {
        const float *x = w + 32 * k;
        float dstore; /* the scale as stored (f32 path), or its f16 value */
        uint16_t dbits16 = 0;
        if (wtype == ORC_Q8_0) {
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(x[j]);
                if (a > amax) amax = a;
            }
            int8_t *q = (int8_t *)img + 32 * k;
            if (amax < 1e-30f) {
                dstore = 0.0f;
                for (int j = 0; j < 32; ++j) q[j] = 0;
            } else if (!scale_f16) {
                dstore = amax / 127.0f;
                float id = 127.0f / amax;
                for (int j = 0; j < 32; ++j) {
                    volatile float t = x[j] * id;
                    float u = t + copysignf(0.5f, x[j]);
                    q[j] = (int8_t)(int)orc_trunc_clamp(u, -127.0f, 127.0f);
                }
            } else {
                float d32 = amax / 127.0f;
                dbits16 = orc_f16_bits(d32);
                if ((dbits16 & 0x7FFFu) >= 0x7C00u) return ORC_FORMAT; /* > 65504 */
                float d16 = (float)orc_f16_value(dbits16);
                if (d16 == 0.0f) {
                    for (int j = 0; j < 32; ++j) q[j] = 0;
                } else {
                    float id = 1.0f / d16;
                    for (int j = 0; j < 32; ++j) {
                        volatile float t = x[j] * id;
                        float u = t + copysignf(0.5f, x[j]);
                        q[j] = (int8_t)(int)orc_trunc_clamp(u, -127.0f, 127.0f);
                    }
                }
                dstore = d16;
            }
        } else {
            float amax = 0.0f, mx = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(x[j]);
                if (a > amax) { amax = a; mx = x[j]; }
            }
            float d = mx / -8.0f;
            float id = (d != 0.0f) ? 1.0f / d : 0.0f;
            if (isinf(id)) id = 0.0f; /* |d| < 2^-128: the block writes as zeros */
            uint8_t *qb = img + 16 * k;
            for (int j = 0; j < 16; ++j) {
                volatile float t0 = x[j] * id, t1 = x[j + 16] * id;
                float l0 = truncf(t0 + 8.5f), l1 = truncf(t1 + 8.5f);
                if (l0 > 15.0f) l0 = 15.0f;
                if (l1 > 15.0f) l1 = 15.0f;
                qb[j] = (uint8_t)((unsigned)l0 | ((unsigned)l1 << 4));
            }
            if (scale_f16) {
                dbits16 = orc_f16_bits(d);
                if ((dbits16 & 0x7FFFu) >= 0x7C00u) return ORC_FORMAT;
            }
            dstore = d;
        }
        if (scale_f16) {
            dptr[2 * k] = (uint8_t)(dbits16 & 0xFFu);
            dptr[2 * k + 1] = (uint8_t)(dbits16 >> 8);
        } else {
            memcpy(dptr + 4 * k, &dstore, 4);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Q4_0 least-squares search (the .mlb page's paragraph on the Q4_0 writer
 * that fits each block, the page's default), per block of 32 weights x:
 *   1. the element of largest magnitude mx (the first to reach amax);
 *      amax = 0 writes d = 0 and nibbles 8;
 *   2. a block with amax < 1e-6 is divided by amax (its largest magnitude
 *      becomes exactly 1) and its fitted d multiplied back by amax;
 *   3. for each candidate level L = -6.0, -6.2, ..., -8.4 (13 values, the
 *      float32 nearest each decimal): iscale = L / mx, level
 *      l = rint(x * iscale) clamped to [-8, 7], then the weighted
 *      least-squares scale with weights w = x^2,
 *        d = sum w x l / sum w l^2,
 *      and its weighted error  E = sum w (x - d l)^2;
 *   4. the candidate with the smallest E wins (the first on ties; a NaN E
 *      never replaces an earlier candidate);
 *   5. nibbles = l + 8 of the winner; with f16 scales d is rounded to the
 *      nearest f16 (the nibbles stay those of the fit).
 * Readings (the page leaves these open): float32 throughout, each
 * operation rounded on its own (no fused multiply-add), the sums taken in
 * element order j = 0..31 with terms (w x) l, w (l l) and w (r r),
 * r = x - d l; rint rounds half to even (the usual numpy rounding); a fit
 * that is not finite (cubes overflow float32 once amax is above about 2^42)
 * and an f16 scale above 65504 are refused.
 * Returns ORC_OK, ORC_SHAPE / ORC_FORMAT as orc_span, or ORC_FORMAT for a
 * refused block (img then unspecified).  img receives full_span bytes.
 * ---------------------------------------------------------------------- */
static const float ORC_LSQ_LEVEL[13] = {-6.0f, -6.2f, -6.4f, -6.6f, -6.8f, -7.0f, -7.2f,
                                        -7.4f, -7.6f, -7.8f, -8.0f, -8.2f, -8.4f};

/* levels of candidate L for the (scaled) block v with largest element mx */
static void orc_lsq_levels(const float *v, float mx, float L, float *l) {
    float iscale = L / mx;
    for (int j = 0; j < 32; ++j) {
        float t = rintf(v[j] * iscale);
        if (t < -8.0f) t = -8.0f;
        if (t > 7.0f) t = 7.0f;
        l[j] = t;
    }
}

int orc_quantize_q4_search(uint32_t scale_f16, uint64_t rows, uint64_t cols,
                           const float *w, uint8_t *img) {
    uint64_t span[5];
    int st = orc_span(ORC_Q4_0, scale_f16, rows, cols, span);
    if (st != ORC_OK) return st;
    memset(img, 0, span[4]);
    uint64_t nblk = rows * (cols / 32);
    uint8_t *dptr = img + span[1];
    for (uint64_t k = 0; k < nblk; ++k) {
        const float *x = w + 32 * k;
        float amax = 0.0f, mx = 0.0f;
        for (int j = 0; j < 32; ++j) {
            float a = fabsf(x[j]);
            if (a > amax) { amax = a; mx = x[j]; }
        }
        float d = 0.0f, best_l[32];
        for (int j = 0; j < 32; ++j) best_l[j] = 0.0f;
        if (amax != 0.0f) {
            float v[32], wt[32], cube[32], l[32];
            const int tiny = amax < 1e-6f;
            for (int j = 0; j < 32; ++j) v[j] = tiny ? x[j] / amax : x[j];
            float m = tiny ? mx / amax : mx;
            for (int j = 0; j < 32; ++j) {
                wt[j] = v[j] * v[j];
                cube[j] = wt[j] * v[j];
            }
            float best_e = 0.0f;
            for (int i = 0; i < 13; ++i) {
                orc_lsq_levels(v, m, ORC_LSQ_LEVEL[i], l);
                float sxl = 0.0f, sll = 0.0f;
                for (int j = 0; j < 32; ++j) {
                    sxl += cube[j] * l[j];
                    sll += wt[j] * (l[j] * l[j]);
                }
                float dc = sxl / sll;
                float e = 0.0f;
                for (int j = 0; j < 32; ++j) {
                    float r = v[j] - dc * l[j];
                    e += wt[j] * (r * r);
                }
                if (i == 0 || e < best_e) {
                    best_e = e;
                    d = dc;
                    memcpy(best_l, l, sizeof best_l);
                }
            }
            if (tiny) d = d * amax;
            if (!isfinite(d)) return ORC_FORMAT;
        }
        uint8_t *qb = img + 16 * k;
        for (int j = 0; j < 16; ++j)
            qb[j] = (uint8_t)((unsigned)(best_l[j] + 8.0f) | ((unsigned)(best_l[j + 16] + 8.0f) << 4));
        if (scale_f16) {
            uint16_t b = orc_f16_bits(d);
            if ((b & 0x7FFFu) >= 0x7C00u) return ORC_FORMAT; /* > 65504 */
            dptr[2 * k] = (uint8_t)(b & 0xFFu);
            dptr[2 * k + 1] = (uint8_t)(b >> 8);
        } else {
            memcpy(dptr + 4 * k, &d, 4);
        }
    }
    return ORC_OK;
}
