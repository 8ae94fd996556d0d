// Launchers of the gfx950 kernels (internal to libqmv).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qmv {

// A device-resident matrix: q array at `q`, scales at `d` (f16 or f32).
struct MatView {
    const uint8_t* q;
    const void* d;
    const int32_t* rexp;  // per row: largest finite |d| of the row in [2^(e-1), 2^e); 0 if none
    uint32_t wtype, scale_f16, rows, cols;
    int32_t dexp;         // the same over the whole matrix
};

// y[t][r] = sum_c W[r][c] x[t][c]; x f32 [batch][cols], y f32 [batch][rows].
// Batches above 8 that the f16 LM-head kernel does not take run on the
// GEMM, which stages the activations in `workspace` (gemv_workspace_bytes
// of them; none needed when that is 0).
size_t gemv_workspace_bytes(const MatView& m, uint32_t batch);
hipError_t launch_gemv(const MatView& m, const float* x, float* y,
                       uint32_t batch, void* workspace, hipStream_t stream);

// One launch for n <= 8 matrices with the same cols multiplying the same x:
// ys[i] = W_i x (falls back to one launch per matrix when they do not fit).
// (batches above 8 run matrix by matrix, with a workspace of the largest
// gemv_workspace_bytes of the matrices).
hipError_t launch_gemv_group(const MatView* ms, uint32_t n, const float* x, float* const* ys,
                             uint32_t batch, void* workspace, hipStream_t stream);

// Gated pair of a feed-forward layer: h[t][r] = act(sum_c W1[r][c] x[t][c]) *
// sum_c W3[r][c] x[t][c], act 0 = SiLU, 1 = GELU (tanh form), in one launch
// per pass of up to 4 vectors.  gemv_gated_fits tells whether a pair can
// (the same storage type, scale type and shape, rows of <= 4 steps of 64
// chunks: cols <= 8192 for Q4_0, <= 4096 for Q8_0); otherwise
// launch_gemv_gated returns hipErrorNotSupported.
bool gemv_gated_fits(const MatView& w1, const MatView& w3);
hipError_t launch_gemv_gated(const MatView& w1, const MatView& w3, uint32_t act, const float* x,
                             float* h, uint32_t batch, hipStream_t stream);

// Same product on the matrix cores with f16 operands: x is bf16 bits, or
// f32 (x_f32 = true).  The activations are first staged as scaled f16 in
// `workspace`, which also holds the partial sums when K is split
// (gemm_workspace_bytes of it, 256-byte aligned).
size_t gemm_workspace_bytes(const MatView& m, uint32_t batch, bool x_f32);
hipError_t launch_gemm(const MatView& m, const void* x, bool x_f32, float* y,
                       uint32_t batch, void* workspace, hipStream_t stream);

// The library's fixed GEMM scratch on the current device (its address, found
// once per device, and its size).
hipError_t gemm_scratch(void** ptr, size_t* bytes);
// launch_gemm over a workspace of ws_bytes: the batch is taken in passes of
// at most that workspace (hipErrorNotSupported if a pass of 32 tokens needs
// more).
hipError_t launch_gemm_within(const MatView& m, const void* x, bool x_f32, float* y,
                              uint32_t batch, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

// y[i] = sum over z < splits of part[z * total + i], added in z order.
hipError_t launch_splitk_sum(const float* part, float* y, uint64_t total, uint32_t splits,
                             hipStream_t stream);

// Product on Q8_0-quantized activations on the int8 matrix cores:
// y[t][r] = sum_b fl(dw[r,b] dx[t,b]) * s[t,r,b] with exact int32 block
// sums s of the weight codes and xq (int8 [batch][cols]), dx float32
// [batch][cols/32].  K may be split as in launch_gemm (workspace of
// gemm_q8act_workspace_bytes).  hipErrorNotSupported when an offset would
// pass 32 bits.
size_t gemm_q8act_workspace_bytes(const MatView& m, uint32_t batch);
hipError_t launch_gemm_q8act(const MatView& m, const int8_t* xq, const float* dx, float* y,
                             uint32_t batch, float* workspace, hipStream_t stream);

// Batched product on the matrix cores with f16 operands (Q8_0 with f16
// scales, cols 512 or 1024, any batch): returns hipErrorNotSupported for
// other matrices (gemv_mfma_fits false), which then take launch_gemm.
bool gemv_mfma_fits(const MatView& m);
hipError_t launch_gemv_mfma(const MatView& m, const float* x, float* y, uint32_t batch,
                            hipStream_t stream);

// out[i][c] = fl32(v * d) of row ids[i] (zeros for an id out of range).
hipError_t launch_embed(const MatView& m, const int32_t* ids, uint32_t n,
                        float* out, hipStream_t stream);

// GGUF Q4_0 / Q8_0 blocks (f16 scale, then quants; 2-byte aligned at src)
// repacked: block k's quants to q + k * (16 | 32), its scale to d[k].
hipError_t launch_gguf_repack(uint32_t wtype, const void* src, uint64_t nblocks, uint8_t* q,
                              uint16_t* d, hipStream_t stream);

// Writer rules over nblocks blocks of float32 weights w: quants to q, then
// q_pad (< 64) zero bytes, scales to d (float or f16 bits); *bad cleared,
// then set to 1 when a scale cannot be stored.  rule 0: Q8_0 or the Q4_0
// round rule; 1: the Q4_0 least-squares search.  Kernels only (no memset).
hipError_t launch_quantize_weights(uint32_t wtype, uint32_t scale_f16, uint32_t rule,
                                   const float* w, uint64_t nblocks, uint8_t* q, uint32_t q_pad,
                                   void* d, uint32_t* bad, hipStream_t stream);

// Activation Q8_0 quantizer over n floats (n % 32 == 0).
hipError_t launch_quantize_q8(const float* x, uint64_t n, int8_t* q, float* d,
                              hipStream_t stream);

// s[r][b] = sum_j v[r][32b+j] * xq[32b+j] (int32).
hipError_t launch_block_dots(const MatView& m, const int8_t* xq, int32_t* s,
                             hipStream_t stream);

// Reads n16 16-byte words from src (measurement aid: the read ceiling).
hipError_t launch_read_probe(const void* src, uint64_t n16, uint32_t* sink, hipStream_t stream);
// One workgroup per compute unit (256), 4 or 8 waves (1 or 2 per SIMD).
constexpr uint32_t kProbeWorkgroups = 256;
hipError_t launch_mfma_probe(bool random, uint32_t waves_per_simd, uint32_t iters, uint64_t* clocks,
                             float* sink, hipStream_t stream);

}  // namespace qmv
