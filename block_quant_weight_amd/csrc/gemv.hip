// Decode product (GEMV) for Q4_0 / Q8_0 matrices on gfx950.
//
// y[t][r] = sum_c W[r][c] * x[t][c] (Krafla ".mlb model, version 1" page,
// "Body": rows are outputs).  The weights stay quantized in HBM and are
// decoded in registers: Q4_0 byte j of a block holds element j in its low
// nibble and element j + 16 in its high nibble, w = (nibble - 8) * d
// (section "Q4_0"); Q8_0 w = q * d (section "Q8_0").
//
// Work split: one wavefront owns NR consecutive rows.  Lane l reads the
// 16-byte chunks l, l + 64, ... of each of its rows, so every load
// instruction of the wave covers 1 KiB of contiguous quants; a Q4_0 chunk
// is one whole block (32 weights), a Q8_0 chunk half a block (16 weights).
// The activations of a chunk are loaded once and reused by the NR rows.
//
// Arithmetic per chunk: raw = sum_j u_j * x_j in float32 with u_j the
// unsigned code (Q4_0 nibble, or Q8_0 byte XOR 0x80 = q + 128), then
// acc += d * (raw - OFF * sum_j x_j) with OFF = 8 or 128.  The code -> float
// conversion is one v_cvt_f32_ubyteN per weight.  sum_j x_j is accumulated
// in the same element order as raw, so a block of all-zero weights gives
// raw == OFF * sum exactly (OFF is a power of two) and contributes exactly 0.
#include "device_common.h"
#include "kernels.h"

namespace qmv {
namespace {

constexpr int kWaves = 4;  // wavefronts per workgroup

// Q4_0 block: sum of nibble_j * x_j.  Byte 4i+k gives element 4i+k (low
// nibble) and element 16+4i+k (high nibble).
__device__ __forceinline__ float q4_raw_dot(const uint4 qv, const float (&xs)[32]) {
    const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x0F0F0F0Fu;
        const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;
        acc = fmaf(ubyte_f32<0>(lo), xs[4 * i + 0], acc);
        acc = fmaf(ubyte_f32<1>(lo), xs[4 * i + 1], acc);
        acc = fmaf(ubyte_f32<2>(lo), xs[4 * i + 2], acc);
        acc = fmaf(ubyte_f32<3>(lo), xs[4 * i + 3], acc);
        acc = fmaf(ubyte_f32<0>(hi), xs[16 + 4 * i + 0], acc);
        acc = fmaf(ubyte_f32<1>(hi), xs[16 + 4 * i + 1], acc);
        acc = fmaf(ubyte_f32<2>(hi), xs[16 + 4 * i + 2], acc);
        acc = fmaf(ubyte_f32<3>(hi), xs[16 + 4 * i + 3], acc);
    }
    return acc;
}

// sum of x over a Q4_0 block, in the element order of q4_raw_dot
__device__ __forceinline__ float q4_xsum(const float (&xs)[32]) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) s += xs[4 * i + k];
#pragma unroll
        for (int k = 0; k < 4; ++k) s += xs[16 + 4 * i + k];
    }
    return s;
}

// Q8_0 half block (16 int8): sum of (q_j + 128) * x_j.
__device__ __forceinline__ float q8_raw_dot(const uint4 qv, const float (&xs)[16]) {
    const uint32_t w[4] = {qv.x ^ 0x80808080u, qv.y ^ 0x80808080u,
                           qv.z ^ 0x80808080u, qv.w ^ 0x80808080u};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = fmaf(ubyte_f32<0>(w[i]), xs[4 * i + 0], acc);
        acc = fmaf(ubyte_f32<1>(w[i]), xs[4 * i + 1], acc);
        acc = fmaf(ubyte_f32<2>(w[i]), xs[4 * i + 2], acc);
        acc = fmaf(ubyte_f32<3>(w[i]), xs[4 * i + 3], acc);
    }
    return acc;
}

__device__ __forceinline__ float q8_xsum(const float (&xs)[16]) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += xs[j];
    return s;
}

template <uint32_t WT, bool SF16, int NR, int NB>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const float* __restrict__ x, float* __restrict__ y, uint32_t rows,
    uint32_t cols) {
    constexpr int CW = (WT == kQ4) ? 32 : 16;  // weights per 16-byte chunk
    constexpr float OFF = (WT == kQ4) ? 8.f : 128.f;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const uint32_t r0 = wave * NR;
    if (r0 >= rows) return;  // uniform per wave
    const uint32_t nchunks = cols / CW;
    const uint64_t row_bytes = (WT == kQ4) ? (cols >> 1) : cols;
    const uint32_t nblk = cols >> 5;

    const uint8_t* qr[NR];
    uint64_t dr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        // rows past the end re-read the last row; their sums are dropped
        const uint32_t rr = min(r0 + r, rows - 1);
        qr[r] = q + static_cast<uint64_t>(rr) * row_bytes;
        dr[r] = static_cast<uint64_t>(rr) * nblk;
    }
    float acc[NR][NB];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

    for (uint32_t ch = lane; ch < nchunks; ch += 64) {
        uint4 qv[NR];
        float dv[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            qv[r] = *reinterpret_cast<const uint4*>(qr[r] + 16ull * ch);
            dv[r] = load_scale<SF16>(d, dr[r] + (WT == kQ4 ? ch : (ch >> 1)));
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float xs[CW];
            const float4* xp = reinterpret_cast<const float4*>(
                x + static_cast<uint64_t>(b) * cols + static_cast<uint64_t>(ch) * CW);
#pragma unroll
            for (int i = 0; i < CW / 4; ++i) {
                const float4 t = xp[i];
                xs[4 * i + 0] = t.x;
                xs[4 * i + 1] = t.y;
                xs[4 * i + 2] = t.z;
                xs[4 * i + 3] = t.w;
            }
            float sx;
            if constexpr (WT == kQ4) sx = q4_xsum(xs); else sx = q8_xsum(xs);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float raw;
                if constexpr (WT == kQ4) raw = q4_raw_dot(qv[r], xs);
                else raw = q8_raw_dot(qv[r], xs);
                acc[r][b] = fmaf(dv[r], raw - OFF * sx, acc[r][b]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float s = wave_sum(acc[r][b]);
            if (lane == 0 && r0 + r < rows)
                y[static_cast<uint64_t>(b) * rows + r0 + r] = s;
        }
    }
}

template <uint32_t WT, bool SF16, int NB>
hipError_t gemv_pass(const MatView& m, const float* x, float* y, hipStream_t s) {
    constexpr int NR = 4;
    const uint32_t waves = (m.rows + NR - 1) / NR;
    const uint32_t blocks = (waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((gemv_kernel<WT, SF16, NR, NB>), dim3(blocks), dim3(256), 0, s,
                       m.q, m.d, x, y, m.rows, m.cols);
    return hipGetLastError();
}

template <uint32_t WT, bool SF16>
hipError_t gemv_batched(const MatView& m, const float* x, float* y,
                        uint32_t batch, hipStream_t s) {
    uint32_t done = 0;
    while (done < batch) {
        const uint32_t left = batch - done;
        const float* xp = x + static_cast<uint64_t>(done) * m.cols;
        float* yp = y + static_cast<uint64_t>(done) * m.rows;
        hipError_t e;
        uint32_t nb;
        if (left >= 8) { nb = 8; e = gemv_pass<WT, SF16, 8>(m, xp, yp, s); }
        else if (left >= 4) { nb = 4; e = gemv_pass<WT, SF16, 4>(m, xp, yp, s); }
        else if (left >= 2) { nb = 2; e = gemv_pass<WT, SF16, 2>(m, xp, yp, s); }
        else { nb = 1; e = gemv_pass<WT, SF16, 1>(m, xp, yp, s); }
        if (e != hipSuccess) return e;
        done += nb;
    }
    return hipSuccess;
}

}  // namespace

// Batches up to this size run the vector kernel; larger ones the matrix
// cores (each vector pass re-reads the whole matrix).
constexpr uint32_t kGemvMaxBatch = 8;

hipError_t launch_gemv(const MatView& m, const float* x, float* y,
                       uint32_t batch, hipStream_t s) {
    if (batch > kGemvMaxBatch) return launch_gemm(m, x, true, y, batch, s);
    if (m.wtype == kQ4) {
        return m.scale_f16 ? gemv_batched<kQ4, true>(m, x, y, batch, s)
                           : gemv_batched<kQ4, false>(m, x, y, batch, s);
    }
    return m.scale_f16 ? gemv_batched<kQ8, true>(m, x, y, batch, s)
                       : gemv_batched<kQ8, false>(m, x, y, batch, s);
}

}  // namespace qmv
