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
 *   - "Q4_0" (byte j of a block holds element j in the low nibble and
 *     element j+16 in the high nibble, w = (nibble - 8) x d);
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
 * Activation quantizer ("Quantization rule"), per block of 32, in float32
 * operations in the page's order:
 *   amax = max |x|;  amax < 1e-30 -> d = 0, q = 0;
 *   else d = amax / 127, q = trunc(x * (127 / amax) + copysign(0.5, x)),
 *   clamped to [-127, 127].
 * Each operation is rounded on its own (no fused multiply-add).  n must be a
 * multiple of 32.
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
