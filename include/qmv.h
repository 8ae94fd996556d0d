/*
 * qmv.h - block-quantized weight matrix x activation products on one
 * MI355X (gfx950) GPU.  Plain C ABI: no HIP, PyTorch or C++ types.
 *
 * A matrix is stored the way Krafla's ".mlb model, version 1" format page
 * describes a quantized matrix ("Body", and the sections "Q8_0" and "Q4_0"):
 *   - rows are outputs: y[r] = sum_c W[r][c] * x[c];
 *   - two arrays, one after the other: q, the quants (Q8_0: rows*cols int8
 *     bytes; Q4_0: rows*cols/2 bytes), then d, one scale per block of 32
 *     consecutive weights of a row (f32, or IEEE f16 when scale_f16 = 1);
 *   - both arrays are padded with zeros up to a 64-byte boundary, so d
 *     starts at pad64(q bytes); the padding after d may be absent;
 *   - Q8_0: w = q * d, and a quant byte of -128 is not allowed;
 *   - Q4_0: the 16 bytes of a block carry elements 0..15 in their low four
 *     bits and elements 16..31 in their high four bits, in order;
 *     w = (nibble - 8) * d;
 *   - everything little-endian.
 * Conventions this library fixes where the page is silent: row r's blocks
 * (and scales) are consecutive, block k = r * (cols / 32) + c / 32; a
 * dequantized weight is the single float32 product fl32(v * d) with IEEE
 * signed zeros and subnormals; rows and cols are each at most 2^24 (the one
 * limit the page's limits sentence keeps) and cols is a multiple of 32.
 *
 * Status: every function returns QMV_OK (0) or a negative QMV_E_* code.
 * Errors are detected on the host before anything is launched; the classes
 * follow the page's "Validation done by the loader" table (ML_E_FORMAT,
 * ML_E_SHAPE), plus argument, device and memory errors.
 *
 * Streams: `stream` is a hipStream_t passed as a pointer; NULL is the null
 * stream.  Compute calls only enqueue work on it and return; they never
 * synchronize.  The one exception to "no allocation": the matrix-core
 * products (qmv_gemm, qmv_gemm_q8 when it splits K, and qmv_gemv on batches
 * above 8 that the f16 LM-head kernel does not take) keep staged
 * activations and partial sums in a workspace owned by the library, one per
 * (device, stream), allocated on first need and grown (never freed) for a
 * larger call; such a first call on a stream must not be made while the
 * stream is being captured into a graph (QMV_E_ARG).
 *
 * Pointers: `x`, `y`, `ids`, `out`, `q`, `d`, `s` of the compute calls are
 * device pointers owned by the caller, each 16-byte aligned (QMV_E_ARG
 * otherwise).  The caller keeps them alive until the work on `stream` is
 * done and must not let an output overlap an input.
 */
#ifndef QMV_H
#define QMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qmv_mat *qmv_handle;

/* Storage types: the values of the .mlb header field "wtype". */
enum { QMV_Q8_0 = 1, QMV_Q4_0 = 2 };

enum {
    QMV_OK = 0,
    QMV_E_ARG = -1,    /* null pointer, misaligned pointer, zero batch/count,
                          upload twice, compute before upload, wrong device */
    QMV_E_FORMAT = -2, /* unknown wtype, scale_f16 not 0/1, buffer shorter
                          than the arrays, a Q8_0 quant equal to -128 */
    QMV_E_SHAPE = -3,  /* zero dimension, cols not a multiple of 32, a
                          dimension above 2^24, size overflow */
    QMV_E_DEVICE = -4, /* a HIP runtime error (launch or copy) */
    QMV_E_NOMEM = -5   /* device or host allocation failed */
};

/*
 * Sizes of a matrix's arrays, from the page's quantized-matrix paragraph:
 * q_bytes = rows*cols (Q8_0) or rows*cols/2 (Q4_0); d_offset =
 * pad64(q_bytes); d_bytes = rows*cols/32 * (scale_f16 ? 2 : 4); min_span =
 * d_offset + d_bytes (the smallest buffer qmv_upload accepts).  Pure host
 * arithmetic in uint64_t; every sum and product is checked for overflow, as
 * the page's "Validation done by the loader" section requires of a loader.
 * Any output pointer may be NULL.
 * Errors: QMV_E_FORMAT (wtype, scale_f16), QMV_E_SHAPE (dimensions).
 */
int qmv_span(uint32_t wtype, uint32_t scale_f16, uint32_t rows, uint32_t cols,
             uint64_t *q_bytes, uint64_t *d_offset, uint64_t *d_bytes,
             uint64_t *min_span);

/*
 * Storage type of one matrix class, from the page's q8_mask paragraph.
 * class_bit is one of 1 tok_emb, 2 wcls, 4 wq/wk (wg, lqkv), 8 wv (lz),
 * 16 wo (lout), 32 w1/w3, 64 w2.  A Q8_0 file (file_wtype 1) stores all
 * classes as Q8_0.  In a Q4_0 file a set bit of q8_mask stores that class
 * as Q8_0; with shared_classifier != 0 the embedding (also the classifier)
 * is Q8_0 if bit 1 or bit 2 is set, and asking for class 2 names that same
 * matrix.  Pure host arithmetic.
 * Errors: QMV_E_FORMAT (file_wtype), QMV_E_ARG (class_bit not one of the
 * seven bits, wtype_out NULL).
 */
int qmv_class_wtype(uint32_t file_wtype, uint32_t q8_mask, uint32_t class_bit,
                    uint32_t shared_classifier, uint32_t *wtype_out);

/*
 * Creates an empty matrix handle of the given storage type and shape (no
 * device memory yet).  *out receives the handle, owned by the caller until
 * qmv_destroy.  Errors: QMV_E_ARG (out NULL), QMV_E_FORMAT, QMV_E_SHAPE
 * (as qmv_span), QMV_E_NOMEM.
 */
int qmv_create(qmv_handle *out, uint32_t wtype, uint32_t scale_f16,
               uint32_t rows, uint32_t cols);

/*
 * Copies one matrix's bytes, exactly as the file holds them starting at its
 * q array (q, zero padding, d, optional trailing padding), from host memory
 * `src` into one device allocation on the current device, keeping the
 * file's offsets (d at d_offset) and the scales in their stored type.  The
 * bytes are checked first: nbytes < min_span or a Q8_0 quant byte equal to
 * 0x80 is QMV_E_FORMAT (padding bytes are not inspected).  Only the first
 * min_span bytes are read.  The call waits for the copy on `stream`, so src
 * may be released when it returns.  A handle is uploaded once and is then
 * read-only; compute calls on several streams may share it.
 * Errors: QMV_E_ARG (null, second upload), QMV_E_FORMAT, QMV_E_NOMEM,
 * QMV_E_DEVICE.
 */
int qmv_upload(qmv_handle h, const void *src, uint64_t nbytes, void *stream);

/*
 * Size of a Q4_0 / Q8_0 tensor's data in a GGUF file, from the minfer page's
 * "Quantized sizing: 32 values in 18 bytes": rows * cols / 32 blocks of 18
 * bytes (BlockQ4_0: an f16 scale d, then 16 bytes of nibbles) or 34 bytes
 * (BlockQ8_0: d, then 32 int8 quants).  Pure host arithmetic.
 * Errors: QMV_E_ARG (bytes NULL), QMV_E_FORMAT (wtype), QMV_E_SHAPE (as
 * qmv_span).
 */
int qmv_gguf_span(uint32_t wtype, uint32_t rows, uint32_t cols, uint64_t *bytes);

/*
 * Upload from GGUF block data instead of the two arrays: src holds the
 * matrix's rows * cols / 32 blocks in row-major order (row r's blocks
 * consecutive; a GGUF tensor's first dimension is the row length), each an
 * f16 little-endian scale followed by the quants, the 16 Q4_0 bytes in the
 * .mlb nibble order (byte j: element j low, element j + 16 high).  The
 * blocks are copied to the device and repacked there, once, into the same
 * image qmv_upload builds (q array, zero padding, f16 d array), so every
 * compute call sees identical bytes.  The handle must have been created
 * with scale_f16 = 1 (GGUF blocks carry f16 scales) and not yet uploaded.
 * Checks, on the host: nbytes >= qmv_gguf_span and no Q8_0 quant byte equal
 * to 0x80 (QMV_E_FORMAT).  Waits for `stream`; src may be released on
 * return.  Allocates the image and a temporary device copy of src.
 * Errors: QMV_E_ARG (null, second upload), QMV_E_FORMAT (f32-scale handle,
 * short data, -128), QMV_E_NOMEM, QMV_E_DEVICE.
 */
int qmv_upload_gguf(qmv_handle h, const void *src, uint64_t nbytes, void *stream);

/* Releases the handle and its device memory.  The caller makes sure no work
 * that reads it is still pending.  NULL is accepted.  Returns QMV_OK. */
int qmv_destroy(qmv_handle h);

/*
 * Decode product (GEMV), y[t][r] = sum_c W[r][c] * x[t][c], for t < batch.
 * x: float32 [batch][cols], y: float32 [batch][rows], row-major, device
 * memory.  The weights stay quantized in device memory and are decoded in
 * registers.  Every output is within 2e-3 * sum_c |W[r][c]| |x[t][c]| of
 * the exact product (the .mlb page's "Body" defines the product; the bound
 * is the parity bar), by these means:
 * Batches up to 8 run the bandwidth-bound vector kernels: every activation is
 * represented, per block of 32 (the span of one weight scale), in 24-bit
 * fixed point relative to the block's largest magnitude amax, the block sums
 * of weight codes times activation digits are exact integer dot products
 * (the Q8_0 activation quantization of the .mlb page's "Quantization rule",
 * with three int8 digits instead of one), and blocks are accumulated in
 * float32.  A nonzero activation that the fixed point would keep to fewer
 * than 10 significant bits (more than about 2^13 below its block's amax) is
 * left out of the digits and its products are added in float32 from the
 * activation itself, so every activation counts to within 2^-10 of itself.
 * A non-finite activation makes the outputs of its batch row NaN.
 * Larger batches (an LM head over a batch of hidden states, say) run on the
 * matrix cores with f16 operands and float32 accumulation: each token's
 * activations scaled by a power of two from its largest magnitude and
 * rounded to f16; each weight fl16(q * d * 2^k), k one per matrix (the f16
 * LM-head kernel: Q8_0 with f16 scales and 512 or 1024 columns) or one per
 * row (every other matrix), from the largest finite scale, found at upload.
 * This is within about 2^-10 * sum_c |W[r][c]| |x[t][c]| for activations
 * within 2^28 of their token's largest and scales within 2^20 of the
 * largest of their row (matrix, for the LM-head kernel); a non-finite
 * activation makes its token's outputs NaN.
 * Errors: QMV_E_ARG (null or misaligned pointer, batch 0, no upload, a first
 * matrix-core call on a stream under graph capture), QMV_E_NOMEM
 * (workspace), QMV_E_DEVICE (launch failure).
 */
int qmv_gemv(qmv_handle h, const float *x, float *y, uint32_t batch,
             void *stream);

/*
 * Grouped decode product: n (1..8) matrices with the same cols, multiplying
 * the same activations, in one launch: ys[i][t][r] = sum_c W_i[r][c] x[t][c].
 * This is how a decode layer's matrices that share an input run (wq, wk, wv;
 * w1, w3 — the .mlb page's body order), and it saves the fixed start-up and
 * drain of every launch after the first.  hs: n handles (any mix of Q4_0 /
 * Q8_0 and scale types); x: float32 [batch][cols]; ys: a host array of n
 * device pointers, float32 [batch][rows_i].  Each output is bit for bit
 * what qmv_gemv computes for that matrix (the same per-row arithmetic).
 * Errors: QMV_E_ARG (n not in 1..8, null or misaligned pointer, batch 0, a
 * handle not uploaded), QMV_E_SHAPE (cols differ), QMV_E_DEVICE.
 */
int qmv_gemv_group(const qmv_handle *hs, uint32_t n, const float *x,
                   float *const *ys, uint32_t batch, void *stream);

/*
 * Gated feed-forward pair of a decode layer in one launch:
 *   h[t][r] = act(sum_c W1[r][c] x[t][c]) * sum_c W3[r][c] x[t][c],
 * w1 the gate and w3 the up projection (the .mlb page's body table), act
 * the header field of that name: 0 = SiLU, a / (1 + e^-a); 1 = GELU with
 * the tanh approximation, a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))).
 * Both sums are the products qmv_gemv computes (the same per-row
 * arithmetic); the activation is the device's float32 expf / tanhf, and
 * the row pair is multiplied once, so h is within the propagated bound
 * (|act'| <= 1.13) of the exact result plus a few float32 rounding steps.
 * x: float32 [batch][cols], h: float32 [batch][rows], device memory,
 * 16-byte aligned; batch passes of up to 4 vectors.
 * Errors: QMV_E_ARG (null or misaligned pointer, batch 0, act > 1, a handle
 * not uploaded), QMV_E_SHAPE (rows or cols differ, or rows longer than four
 * steps: cols > 8192 for Q4_0, > 4096 for Q8_0 — such a pair runs as
 * qmv_gemv_group and the caller's activation), QMV_E_FORMAT (the two differ
 * in storage or scale type), QMV_E_DEVICE.
 */
int qmv_gemv_gated(qmv_handle w1, qmv_handle w3, uint32_t act, const float *x,
                   float *h, uint32_t batch, void *stream);

/*
 * Prefill product (GEMM), y[t][r] = sum_c W[r][c] * x[t][c], with x given
 * as bfloat16 bit patterns: x_bf16 uint16 [batch][cols], y float32
 * [batch][rows], device memory.  On the matrix cores with f16 operands and
 * float32 accumulation: a first kernel stages each token's activations in
 * f16, scaled by a power of two from the token's largest magnitude (exact for
 * values within 2^31 of it); each weight enters as fl16(v * d * 2^(8 - E_r)),
 * E_r the exponent of row r's largest finite scale (found at upload), so a
 * weight keeps 2^-11 relative precision when its scale is within 2^20 of
 * the row's largest; the outputs are scaled back exactly.  Every output is
 * within 2e-3 * sum_c |W[r][c]| |x[t][c]| of the exact product over that
 * range (2^-11 for the weights plus the float32 accumulation); a token
 * holding inf or NaN gets NaN outputs.  When the matrix has too few tiles to
 * fill the GPU the K dimension is split and the slices' partial sums are
 * added in slice order by a third kernel (deterministic).  Errors: as
 * qmv_gemv, plus QMV_E_ARG for a first call on a stream under graph
 * capture and QMV_E_NOMEM if its workspace cannot be allocated.
 */
int qmv_gemm(qmv_handle h, const uint16_t *x_bf16, float *y, uint32_t batch,
             void *stream);

/*
 * qmv_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results, with the staged activations and split-K
 * partial sums in a fixed 64 MiB array of the library's own on each GPU
 * (held until the process ends) instead of an allocated workspace.  No
 * allocation happens in this call.  A batch whose workspace would exceed the
 * array is taken in passes of fewer tokens (a multiple of 32); QMV_E_SHAPE
 * if even a pass of 32 tokens does not fit (rows or cols very large).  All
 * calls on one GPU share the array: calls that overlap in time on one GPU
 * (different streams, or host threads) race and must be serialised by the
 * caller.  Arguments and other errors as qmv_gemm.
 */
int qmv_gemm_noalloc(qmv_handle h, const uint16_t *x_bf16, float *y, uint32_t batch,
                     void *stream);

/*
 * Prefill product on Q8_0-quantized activations (the page's CPU path: the
 * activations quantized per block of 32 by the "Quantization rule", e.g.
 * with qmv_quantize_q8, then per-block integer dot products):
 *   y[t][r] = sum_b fl(dw[r,b] * dx[t,b]) * s[t,r,b],
 *   s[t,r,b] = sum_j v[r,32b+j] * xq[t,32b+j]   (exact 32-bit integers),
 * dw the matrix's block scales, v its codes (Q8_0 quants, Q4_0 nibble - 8).
 * The block sums run on the int8 matrix cores (one 32x32x32 product per
 * block), the combine is float32: within (cols/32 + 1) * 2^-24 *
 * sum_b |dw dx s| of the exact sum.  xq: int8 [batch][cols], dx: float32
 * [batch][cols/32], y: float32 [batch][rows], device memory, 16-byte
 * aligned.  When the output tiles are too few to fill the GPU, K is split
 * and the slices' partial sums are added in slice order by a second kernel
 * (deterministic), in a per-stream workspace as for qmv_gemm.  Errors:
 * QMV_E_ARG (null or misaligned pointer, batch 0, no upload, a first
 * split-K call on a stream under graph capture), QMV_E_SHAPE (an operand
 * of 4 GiB or more), QMV_E_NOMEM (workspace), QMV_E_DEVICE.
 */
int qmv_gemm_q8(qmv_handle h, const int8_t *xq, const float *dx, float *y, uint32_t batch,
                void *stream);

/*
 * Embedding-row gather: out[i][c] = fl32(v * d) of row ids[i], bit for bit
 * the dequantized weight (scaling such as an embedding factor is the
 * caller's).  ids: int32 [n], out: float32 [n][cols], device memory.  An id
 * outside [0, rows) yields a row of zeros (memory stays safe; the host does
 * not read ids).  Errors: QMV_E_ARG (null or misaligned pointer, n 0, no
 * upload), QMV_E_DEVICE.
 */
int qmv_embed_rows(qmv_handle h, const int32_t *ids, uint32_t n, float *out,
                   void *stream);

/*
 * Activation quantizer of the page's "Quantization rule", per block of 32
 * consecutive values, in separate float32 operations (no fused
 * multiply-add, correctly rounded divisions): amax = max |x|; amax < 1e-30
 * gives d = 0 and q = 0; else d = amax / 127 and q = trunc(x * (127 / amax)
 * + copysign(0.5, x)) clamped to [-127, 127].  x: float32 [n], q: int8 [n],
 * d: float32 [n / 32], device memory; n a multiple of 32.
 * Errors: QMV_E_ARG (null or misaligned pointer, n 0), QMV_E_SHAPE
 * (n % 32 != 0), QMV_E_DEVICE.
 */
int qmv_quantize_q8(const float *x, uint64_t n, int8_t *q, float *d,
                    void *stream);

/*
 * Weight writer: the .mlb image (q array, its zero padding, d array:
 * min_span bytes as qmv_span gives them) of float32 weights w [rows][cols]
 * (device memory), quantized per block of 32 by the rules of the .mlb
 * page's "Quantization rule" section, in separate float32 operations:
 *   - Q8_0, f32 scales: exactly qmv_quantize_q8 (the page uses one rule
 *     for the writer and the activation quantizer);
 *   - Q8_0, f16 scales: d = amax / 127 rounded to the nearest f16, then
 *     q = trunc(x * (1 / d) + copysign(0.5, x)) with d as rounded,
 *     clamped to [-127, 127] (q = 0 when d rounds to 0);
 *   - Q4_0, rule QMV_Q4_ROUND, the page's "round" rule: d = (the first
 *     element of largest magnitude) / -8, nibble = min(15, trunc(x * (1 /
 *     d) + 8.5)) with 1 / d taken as 0 when d = 0 or when it overflows
 *     (|d| < 2^-128); with f16 scales d is stored rounded to f16 while the
 *     nibbles use the float32 d;
 *   - Q4_0, rule QMV_Q4_SEARCH, the page's least-squares writer: the first
 *     element of largest magnitude mx is mapped to each of the 13 levels
 *     L = -6.0, -6.2, ..., -8.4; levels rint(x * (L / mx)) (half to even)
 *     clamped to [-8, 7]; d = sum w x l / sum w l^2 with w = x^2, summed in
 *     element order; the candidate of smallest sum w (x - d l)^2 wins, the
 *     first on ties; the values of a block whose largest magnitude is
 *     under 1e-6 are divided by that magnitude before the fit and d is
 *     multiplied by it after; nibble = level + 8; an f16 d is the fitted d
 *     rounded to f16.
 * rule: QMV_Q4_ROUND (0) for every storage type, QMV_Q4_SEARCH (1) for
 * Q4_0 only.
 * image (device, 16-byte aligned, at least min_span bytes) receives the
 * bytes; they can be written to a file or uploaded with qmv_upload.
 * status (a device uint32, 4-byte aligned) is set to 0, and to 1 if some
 * scale cannot be stored: an f16 scale above 65504, or a least-squares fit
 * that is not finite (weights above about 2^42, whose float32 cubes
 * overflow); the image is then not a valid file's.  Read it once the work
 * on `stream` is done.  Like the compute calls it only enqueues kernels (no
 * allocation, no memset), so it can be captured in a graph.
 * Errors: QMV_E_FORMAT (wtype, scale_f16), QMV_E_SHAPE, QMV_E_ARG (null or
 * misaligned pointer, image too small, rule > 1 or QMV_Q4_SEARCH with
 * Q8_0), QMV_E_DEVICE.
 */
enum { QMV_Q4_ROUND = 0, QMV_Q4_SEARCH = 1 };
int qmv_quantize_weights(uint32_t wtype, uint32_t scale_f16, uint32_t rule, uint32_t rows,
                         uint32_t cols, const float *w, void *image, uint64_t image_bytes,
                         uint32_t *status, void *stream);

/*
 * Per-block integer dot products of the weight quants with quantized
 * activations: s[r][b] = sum_{j<32} v[r][32b + j] * xq[32b + j] in int32,
 * exact (v the Q8_0 quant or Q4_0 nibble - 8).  xq: int8 [cols],
 * s: int32 [rows][cols / 32], device memory.
 * Errors: QMV_E_ARG (null or misaligned pointer, no upload), QMV_E_DEVICE.
 */
int qmv_block_dots(qmv_handle h, const int8_t *xq, int32_t *s, void *stream);

/*
 * Measurement aid, not part of the product: reads nbytes of device memory
 * at src with 16-byte loads (1 KiB per wavefront load, 32 KiB per
 * workgroup, all requested at once), the read ceiling against which the
 * decode kernels' rates are set.  src 16-byte aligned, nbytes a nonzero multiple of 16;
 * sink: 64 uint32 of device memory the kernel may write (it keeps the loads
 * alive; practically never written).  Errors: QMV_E_ARG, QMV_E_DEVICE.
 */
int qmv_read_probe(const void *src, uint64_t nbytes, uint32_t *sink, void *stream);

/*
 * Measurement aid, not part of the product: the rate of the prefill
 * product's matrix-core instruction (v_mfma_f32_32x32x16_f16) back to
 * back, the ceiling against which the product's rate is set.  256
 * workgroups of 4 * waves_per_simd waves (waves_per_simd 1 or 2); every
 * wave runs 8 independent chains of iters products (iters 1 .. 2^20) on
 * constant operands (random_operands 0: 1 and 0) or on two alternating sets
 * of pseudo-random values in [-0.5, 0.5) (1), and writes clocks[2 w] =
 * shader-clock cycles and clocks[2 w + 1] = 100 MHz wall-clock ticks of its
 * chains (w = wave index over the grid).  clocks: 2 * 1024 * waves_per_simd
 * uint64 of device memory, 8-byte aligned; sink: 64 * 1024 * waves_per_simd
 * floats of device memory (the lanes' sums, which keep the products).
 * Errors: QMV_E_ARG, QMV_E_DEVICE.
 */
int qmv_mfma_probe(uint32_t random_operands, uint32_t waves_per_simd, uint32_t iters,
                   uint64_t *clocks, float *sink, void *stream);

/* Static text for a status code (never NULL). */
const char *qmv_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
