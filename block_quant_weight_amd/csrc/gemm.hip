// Prefill product (GEMM) on the gfx950 matrix cores.
//
// Y[t][r] = sum_c W[r][c] * X[t][c] (Krafla ".mlb model, version 1" page,
// "Body"), t over the batch of activation rows.  This is the one place the
// product is a dense contraction, so it runs on MFMA:
//   - a workgroup owns a BM x BN tile of Y (tokens x matrix rows) and walks
//     K in steps of BK = 64 (two quant blocks);
//   - each step stages the activations into LDS as bfloat16 and decodes the
//     quantized weights of the tile (Q4_0: nibble j / j + 16 of byte j,
//     w = (nibble - 8) * d; Q8_0: w = q * d) to w32 = fl32(v * d) and then
//     to bfloat16 (round to nearest even, v_cvt_pk_bf16_f32) in LDS;
//   - four wavefronts (2 x 2) each multiply a (BM/2) x 64 sub-tile with
//     v_mfma_f32_32x32x16_bf16, accumulating in float32.
// Float32 activations (an LM head fed hidden states) are split into
// hi = bf16(x) and lo = bf16(x - hi), and both terms are multiplied: the
// activation error drops from 2^-9 to about 2^-17 relative.
#include "device_common.h"
#include "kernels.h"

namespace qmv {
namespace {

constexpr int kBN = 128;  // matrix rows per tile
constexpr int kBK = 64;   // K per step
constexpr int kLDK = kBK + 8;  // LDS row pitch in bf16 (144 B: spreads banks)

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3,
                                        float a4, float a5, float a6, float a7) {
    bf16x8 v;
    v[0] = static_cast<__bf16>(a0);
    v[1] = static_cast<__bf16>(a1);
    v[2] = static_cast<__bf16>(a2);
    v[3] = static_cast<__bf16>(a3);
    v[4] = static_cast<__bf16>(a4);
    v[5] = static_cast<__bf16>(a5);
    v[6] = static_cast<__bf16>(a6);
    v[7] = static_cast<__bf16>(a7);
    return v;
}

// Decode one block (32 weights) of row n starting at column k into four
// bf16x8 vectors, elements 0..31 in order.
template <uint32_t WT, bool SF16>
__device__ __forceinline__ void decode_block(const uint8_t* __restrict__ q,
                                             const void* __restrict__ d,
                                             uint32_t K, uint32_t n, uint32_t k,
                                             bf16x8 (&out)[4]) {
    const uint32_t nblk = K >> 5;
    const uint64_t blk = static_cast<uint64_t>(n) * nblk + (k >> 5);
    const float dv = load_scale<SF16>(d, blk);
    if constexpr (WT == kQ4) {
        const uint4 qv = *reinterpret_cast<const uint4*>(q + 16ull * blk);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
        float lo[16], hi[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t byte = (w[i] >> (8 * b)) & 0xFFu;
                lo[4 * i + b] = static_cast<float>(static_cast<int>(byte & 15u) - 8) * dv;
                hi[4 * i + b] = static_cast<float>(static_cast<int>(byte >> 4) - 8) * dv;
            }
        }
        out[0] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
        out[1] = pack8(lo[8], lo[9], lo[10], lo[11], lo[12], lo[13], lo[14], lo[15]);
        out[2] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
        out[3] = pack8(hi[8], hi[9], hi[10], hi[11], hi[12], hi[13], hi[14], hi[15]);
    } else {
        const uint8_t* p = q + static_cast<uint64_t>(n) * K + k;
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float v[32];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                v[4 * i + c] = static_cast<float>(static_cast<int8_t>((w[i] >> (8 * c)) & 0xFFu)) * dv;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            out[g] = pack8(v[8 * g], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3],
                           v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7]);
    }
}

template <uint32_t WT, bool SF16, bool XF32, int BM>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const void* __restrict__ xv, float* __restrict__ y, uint32_t M, uint32_t N,
    uint32_t K) {
    constexpr int TM = BM / 64;  // 32x32 MFMA tiles per wave along M
    constexpr int TN = 2;        // and along N (wave covers 64 rows)
    __shared__ __attribute__((aligned(16))) __bf16 As[BM * kLDK];
    __shared__ __attribute__((aligned(16))) __bf16 Al[XF32 ? BM * kLDK : 8];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[kBN * kLDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const uint32_t m0 = blockIdx.y * BM;
    const uint32_t n0 = blockIdx.x * kBN;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    for (uint32_t k0 = 0; k0 < K; k0 += kBK) {
        // ---- activations -> LDS (BM x 64) ----
        constexpr int SEGS = BM * kBK / 8;  // 8-element segments
#pragma unroll
        for (int it = 0; it < SEGS / 256; ++it) {
            const int s = tid + 256 * it;
            const int r = s >> 3, c8 = (s & 7) * 8;
            const uint32_t m = m0 + r, k = k0 + c8;
            bf16x8 hi, lo;
            if (m < M && k < K) {
                if constexpr (XF32) {
                    const float* xp = static_cast<const float*>(xv) +
                                      static_cast<uint64_t>(m) * K + k;
                    const float4 a = *reinterpret_cast<const float4*>(xp);
                    const float4 b = *reinterpret_cast<const float4*>(xp + 4);
                    const float xs[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const __bf16 h = static_cast<__bf16>(xs[e]);
                        hi[e] = h;
                        lo[e] = static_cast<__bf16>(xs[e] - static_cast<float>(h));
                    }
                } else {
                    hi = *reinterpret_cast<const bf16x8*>(
                        static_cast<const uint16_t*>(xv) + static_cast<uint64_t>(m) * K + k);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    hi[e] = static_cast<__bf16>(0.f);
                    lo[e] = static_cast<__bf16>(0.f);
                }
            }
            *reinterpret_cast<bf16x8*>(&As[r * kLDK + c8]) = hi;
            if constexpr (XF32) *reinterpret_cast<bf16x8*>(&Al[r * kLDK + c8]) = lo;
        }
        // ---- weights -> LDS (128 rows x 2 blocks, one block per thread) ----
        {
            const int r = tid >> 1, blk = tid & 1;
            const uint32_t n = n0 + r, k = k0 + 32 * blk;
            bf16x8 w[4];
            if (n < N && k < K) {
                decode_block<WT, SF16>(q, d, K, n, k, w);
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[g][e] = static_cast<__bf16>(0.f);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<bf16x8*>(&Bs[r * kLDK + 32 * blk + 8 * g]) = w[g];
        }
        __syncthreads();
        // ---- MFMA over the step ----
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            const int kcol = kk + 8 * (lane >> 5);
            bf16x8 a[TM], al[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * (BM / 2) + i * 32 + (lane & 31);
                a[i] = *reinterpret_cast<const bf16x8*>(&As[row * kLDK + kcol]);
                if constexpr (XF32)
                    al[i] = *reinterpret_cast<const bf16x8*>(&Al[row * kLDK + kcol]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * 64 + j * 32 + (lane & 31);
                b[j] = *reinterpret_cast<const bf16x8*>(&Bs[row * kLDK + kcol]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
                    if constexpr (XF32)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], b[j], acc[i][j], 0, 0, 0);
                }
        }
        __syncthreads();
    }
    // ---- epilogue: lane holds column n = lane % 32 of each 32x32 tile and
    // rows 8*(v/4) + 4*(lane/32) + v%4 ----
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t m = m0 + wm * (BM / 2) + i * 32 + 8 * (v >> 2) +
                                   4 * (lane >> 5) + (v & 3);
                const uint32_t n = n0 + wn * 64 + j * 32 + (lane & 31);
                if (m < M && n < N) y[static_cast<uint64_t>(m) * N + n] = acc[i][j][v];
            }
}

template <uint32_t WT, bool SF16, bool XF32>
hipError_t gemm_dispatch(const MatView& m, const void* x, float* y,
                         uint32_t batch, hipStream_t s) {
    const dim3 block(256);
    if (batch <= 64) {
        const dim3 grid((m.rows + kBN - 1) / kBN, (batch + 63) / 64);
        hipLaunchKernelGGL((gemm_kernel<WT, SF16, XF32, 64>), grid, block, 0, s,
                           m.q, m.d, x, y, batch, m.rows, m.cols);
    } else {
        const dim3 grid((m.rows + kBN - 1) / kBN, (batch + 127) / 128);
        hipLaunchKernelGGL((gemm_kernel<WT, SF16, XF32, 128>), grid, block, 0, s,
                           m.q, m.d, x, y, batch, m.rows, m.cols);
    }
    return hipGetLastError();
}

template <bool XF32>
hipError_t gemm_by_type(const MatView& m, const void* x, float* y,
                        uint32_t batch, hipStream_t s) {
    if (m.wtype == kQ4)
        return m.scale_f16 ? gemm_dispatch<kQ4, true, XF32>(m, x, y, batch, s)
                           : gemm_dispatch<kQ4, false, XF32>(m, x, y, batch, s);
    return m.scale_f16 ? gemm_dispatch<kQ8, true, XF32>(m, x, y, batch, s)
                       : gemm_dispatch<kQ8, false, XF32>(m, x, y, batch, s);
}

}  // namespace

hipError_t launch_gemm(const MatView& m, const void* x, bool x_f32, float* y,
                       uint32_t batch, hipStream_t s) {
    // grid.y carries the token tiles: at most 65535 of them
    if ((batch + 63) / 64 > 65535u) return hipErrorInvalidValue;
    return x_f32 ? gemm_by_type<true>(m, x, y, batch, s)
                 : gemm_by_type<false>(m, x, y, batch, s);
}

}  // namespace qmv
