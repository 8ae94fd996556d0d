// Embedding-row gather, activation Q8_0 quantizer and per-block integer dot
// products on gfx950.
//
// Gather: out[i][c] = fl32(v * d) for row ids[i], bit for bit the
// dequantized weight (Krafla ".mlb model, version 1" page: the embedding
// table tok_emb is a quantized matrix of vocab rows, "Body"; sections "Q8_0"
// and "Q4_0" give v and w = v * d).  One wavefront per id; lane l decodes
// the 16-byte quant chunks l, l + 64, ... of the row.
//
// Read probe (a measurement aid, no part of the product): each workgroup
// reads its own 32 KiB with 1 KiB-per-wave loads, all requested at once; the
// words are folded by XOR and stored only in the (practically never met)
// case that the fold equals a fixed constant, which keeps the loads without
// a store stream.
//
// Matrix-core rate probe (a measurement aid, no part of the product): every
// wave runs eight independent chains of v_mfma_f32_32x32x16_f16, the
// prefill product's instruction, and records the shader-clock cycles and
// the 100 MHz wall-clock ticks its chains took; operands are either
// constant (1 and 0) or two sets of hashed values in [-0.5, 0.5) that
// alternate from one product to the next, as the operands of a real
// product change, since the clock the power limit allows depends on how
// many bits the matrix cores' inputs toggle.
//
// Quantizer: the page's "Quantization rule" in separate float32 operations
// (__fmul_rn / __fadd_rn cannot be fused; float division is correctly
// rounded on this target).
#include "device_common.h"
#include "kernels.h"

namespace qmv {
namespace {

template <uint32_t WT, bool SF16>
__global__ __launch_bounds__(256) void embed_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const int32_t* __restrict__ ids, float* __restrict__ out, uint32_t n,
    uint32_t rows, uint32_t cols) {
    constexpr int CW = (WT == kQ4) ? 32 : 16;
    const int lane = threadIdx.x & 63;
    const uint32_t i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const int32_t id = ids[i];
    const bool valid = id >= 0 && static_cast<uint32_t>(id) < rows;
    const uint32_t nchunks = cols / CW;
    const uint64_t row_bytes = (WT == kQ4) ? (cols >> 1) : cols;
    const uint32_t nblk = cols >> 5;
    float* orow = out + static_cast<uint64_t>(i) * cols;
    for (uint32_t ch = lane; ch < nchunks; ch += 64) {
        float w[CW];
        if (valid) {
            const uint64_t r = static_cast<uint64_t>(id);
            const uint4 qv = *reinterpret_cast<const uint4*>(q + r * row_bytes + 16ull * ch);
            const float dv = load_scale<SF16>(d, r * nblk + (WT == kQ4 ? ch : (ch >> 1)));
            const uint32_t ws[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t byte = (ws[k] >> (8 * b)) & 0xFFu;
                    if constexpr (WT == kQ4) {
                        w[4 * k + b] = static_cast<float>(static_cast<int>(byte & 15u) - 8) * dv;
                        w[16 + 4 * k + b] = static_cast<float>(static_cast<int>(byte >> 4) - 8) * dv;
                    } else {
                        w[4 * k + b] = static_cast<float>(static_cast<int8_t>(byte)) * dv;
                    }
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < CW; ++e) w[e] = 0.f;
        }
        float4* op = reinterpret_cast<float4*>(orow + static_cast<uint64_t>(ch) * CW);
#pragma unroll
        for (int e = 0; e < CW / 4; ++e)
            op[e] = make_float4(w[4 * e], w[4 * e + 1], w[4 * e + 2], w[4 * e + 3]);
    }
}

// One thread per block of 32 activations.
__global__ __launch_bounds__(256) void quantize_q8_kernel(
    const float* __restrict__ x, uint64_t nblocks, int8_t* __restrict__ q,
    float* __restrict__ d) {
    const uint64_t b = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
    const float4* xp = reinterpret_cast<const float4*>(x + 32 * b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = xp[i];
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float a = fabsf(v[j]);
        if (a > amax) amax = a;
    }
    uint32_t packed[8];
    if (amax < 1e-30f) {
        d[b] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) packed[i] = 0;
    } else {
        d[b] = amax / 127.0f;
        const float id = 127.0f / amax;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float xj = v[4 * i + c];
                const float t = __fmul_rn(xj, id);
                const float u = __fadd_rn(t, copysignf(0.5f, xj));
                float tr = truncf(u);
                tr = fminf(fmaxf(tr, -127.f), 127.f);
                const int qi = static_cast<int>(tr);
                word |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * c);
            }
            packed[i] = word;
        }
    }
    uint4* qp = reinterpret_cast<uint4*>(q + 32 * b);
    qp[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    qp[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

// One thread per (row, block): s = sum_j v_j * xq_j with v_dot4_i32_i8.
template <uint32_t WT>
__global__ __launch_bounds__(256) void block_dots_kernel(
    const uint8_t* __restrict__ q, const int8_t* __restrict__ xq,
    int32_t* __restrict__ s, uint32_t rows, uint32_t cols) {
    const uint32_t nblk = cols >> 5;
    const uint64_t idx = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<uint64_t>(rows) * nblk) return;
    const uint32_t b = static_cast<uint32_t>(idx % nblk);
    const uint4 x0 = *reinterpret_cast<const uint4*>(xq + 32ull * b);
    const uint4 x1 = *reinterpret_cast<const uint4*>(xq + 32ull * b + 16);
    const int xw[8] = {static_cast<int>(x0.x), static_cast<int>(x0.y),
                       static_cast<int>(x0.z), static_cast<int>(x0.w),
                       static_cast<int>(x1.x), static_cast<int>(x1.y),
                       static_cast<int>(x1.z), static_cast<int>(x1.w)};
    int acc = 0;
    if constexpr (WT == kQ4) {
        // nibbles 0..15 as int8 lanes; v = nibble - 8 is folded in as
        // -8 * sum(xq) over the block.
        const uint4 qv = *reinterpret_cast<const uint4*>(q + 16ull * idx);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
        int xsum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lo = static_cast<int>(w[i] & 0x0F0F0F0Fu);
            const int hi = static_cast<int>((w[i] >> 4) & 0x0F0F0F0Fu);
            acc = __builtin_amdgcn_sdot4(lo, xw[i], acc, false);
            acc = __builtin_amdgcn_sdot4(hi, xw[4 + i], acc, false);
            xsum = __builtin_amdgcn_sdot4(0x01010101, xw[i], xsum, false);
            xsum = __builtin_amdgcn_sdot4(0x01010101, xw[4 + i], xsum, false);
        }
        acc -= 8 * xsum;
    } else {
        const uint8_t* p = q + 32ull * idx;  // row r, block b: byte r*cols + 32b
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint4 c = *reinterpret_cast<const uint4*>(p + 16);
        const int w[8] = {static_cast<int>(a.x), static_cast<int>(a.y),
                          static_cast<int>(a.z), static_cast<int>(a.w),
                          static_cast<int>(c.x), static_cast<int>(c.y),
                          static_cast<int>(c.z), static_cast<int>(c.w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_sdot4(w[i], xw[i], acc, false);
    }
    s[idx] = acc;
}

constexpr uint32_t kProbeMagic = 0x9E3779B9u;
constexpr uint32_t kProbeLoads = 8;                          // 16-byte loads per thread
constexpr uint32_t kProbeBytes = 256 * kProbeLoads * 16;     // bytes per workgroup

// Workgroup g reads bytes [g * 32 KiB, (g + 1) * 32 KiB) of src: every load
// requested before any is used (one round trip, like the one-shot product
// kernels), raw buffer loads with the streaming cache policy of the weight
// streams, zeros past the end.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ src, uint64_t nbytes,
                                                         uint32_t* __restrict__ sink) {
    const uint64_t base = static_cast<uint64_t>(blockIdx.x) * kProbeBytes;
    const uint64_t left = nbytes - base;
    const uint32_t range = left < kProbeBytes ? static_cast<uint32_t>(left) : kProbeBytes;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src + base), static_cast<short>(0), static_cast<int>(range), 0x00020000);
    uint32_t v[kProbeLoads][4];
#pragma unroll
    for (uint32_t u = 0; u < kProbeLoads; ++u) {
        typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));
        const probe_u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, (u * 256 + threadIdx.x) * 16, 0, 2);
        v[u][0] = t[0]; v[u][1] = t[1]; v[u][2] = t[2]; v[u][3] = t[3];
    }
    uint32_t acc = 0;
#pragma unroll
    for (uint32_t u = 0; u < kProbeLoads; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    if (acc == kProbeMagic) sink[blockIdx.x & 63] = acc;
}

constexpr uint32_t kMfmaChains = 8;

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    return x ^ (x >> 16);
}

// Wave w of the grid writes clocks[2 w] (shader-clock cycles) and
// clocks[2 w + 1] (100 MHz ticks) over its iters x kMfmaChains products,
// and its lanes' sums to sink[64 w + lane] (which keeps the products).
template <bool RANDOM>
__global__ __launch_bounds__(512) void mfma_probe_kernel(uint64_t* __restrict__ clocks, uint32_t iters,
                                                         float* __restrict__ sink) {
    typedef _Float16 probe_f16x8 __attribute__((ext_vector_type(8)));
    typedef float probe_f32x16 __attribute__((ext_vector_type(16)));
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t gw = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    probe_f16x8 a[2], b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (RANDOM) {
                a[j][i] = static_cast<_Float16>(
                    static_cast<float>(probe_hash(lane * 131u + i + gw * 7u + j * 5003u) & 0xFFFFu) / 65536.0f - 0.5f);
                b[j][i] = static_cast<_Float16>(
                    static_cast<float>(probe_hash(lane * 977u + i * 13u + gw + j * 7919u) & 0xFFFFu) / 65536.0f - 0.5f);
            } else {
                a[j][i] = static_cast<_Float16>(1.0f);
                b[j][i] = static_cast<_Float16>(0.0f);
            }
        }
    probe_f32x16 acc[kMfmaChains];
#pragma unroll
    for (uint32_t k = 0; k < kMfmaChains; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (uint32_t k = 0; k < kMfmaChains; ++k)
            acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[k & 1], b[k & 1], acc[k], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (uint32_t k = 0; k < kMfmaChains; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += acc[k][v];
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
        clocks[2 * gw] = t1 - t0;
        clocks[2 * gw + 1] = w1 - w0;
    }
    sink[gw * 64 + lane] = sum;
}

}  // namespace

hipError_t launch_embed(const MatView& m, const int32_t* ids, uint32_t n,
                        float* out, hipStream_t s) {
    const dim3 grid((n + 3) / 4), block(256);
    if (m.wtype == kQ4) {
        if (m.scale_f16)
            hipLaunchKernelGGL((embed_kernel<kQ4, true>), grid, block, 0, s, m.q, m.d, ids, out, n, m.rows, m.cols);
        else
            hipLaunchKernelGGL((embed_kernel<kQ4, false>), grid, block, 0, s, m.q, m.d, ids, out, n, m.rows, m.cols);
    } else {
        if (m.scale_f16)
            hipLaunchKernelGGL((embed_kernel<kQ8, true>), grid, block, 0, s, m.q, m.d, ids, out, n, m.rows, m.cols);
        else
            hipLaunchKernelGGL((embed_kernel<kQ8, false>), grid, block, 0, s, m.q, m.d, ids, out, n, m.rows, m.cols);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_q8(const float* x, uint64_t n, int8_t* q, float* d,
                              hipStream_t s) {
    const uint64_t nblocks = n / 32;
    const uint64_t grid = (nblocks + 255) / 256;
    if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_q8_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                       x, nblocks, q, d);
    return hipGetLastError();
}

hipError_t launch_block_dots(const MatView& m, const int8_t* xq, int32_t* out,
                             hipStream_t s) {
    const uint64_t total = static_cast<uint64_t>(m.rows) * (m.cols >> 5);
    const uint64_t grid = (total + 255) / 256;
    if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (m.wtype == kQ4)
        hipLaunchKernelGGL((block_dots_kernel<kQ4>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                           m.q, xq, out, m.rows, m.cols);
    else
        hipLaunchKernelGGL((block_dots_kernel<kQ8>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                           m.q, xq, out, m.rows, m.cols);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, uint64_t n16, uint32_t* sink, hipStream_t s) {
    const uint64_t nbytes = n16 * 16;
    const uint64_t grid = (nbytes + kProbeBytes - 1) / kProbeBytes;
    if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(src), nbytes, sink);
    return hipGetLastError();
}

hipError_t launch_mfma_probe(bool random, uint32_t waves_per_simd, uint32_t iters, uint64_t* clocks,
                             float* sink, hipStream_t s) {
    const dim3 grid(kProbeWorkgroups), block(256 * waves_per_simd);
    if (random)
        hipLaunchKernelGGL(mfma_probe_kernel<true>, grid, block, 0, s, clocks, iters, sink);
    else
        hipLaunchKernelGGL(mfma_probe_kernel<false>, grid, block, 0, s, clocks, iters, sink);
    return hipGetLastError();
}

}  // namespace qmv
