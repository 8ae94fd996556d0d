// Matrix images built on the GPU: GGUF block data repacked into the
// two-array layout, and float32 weights quantized by the .mlb writer's rules.
//
// GGUF (minfer, "GGUF load" page, "Quantized sizing: 32 values in 18
// bytes"): a Q4_0 / Q8_0 tensor is a run of blocks, each an f16 scale and
// then the block's quants (BlockQ4_0: 2 + 16 bytes, BlockQ8_0: 2 + 32
// bytes).  The repack moves block k's quants to q + k * (16 | 32) and its
// scale to d + 2k: the same weights, in the layout every compute kernel
// reads (the .mlb page, "Body").
//
// Writer (the .mlb page, "Quantization rule" and the paragraphs after it),
// per block of 32 weights, each float32 operation rounded on its own
// (nothing is contracted into a fused multiply-add; divisions are correctly rounded
// on this target):
//   - Q8_0 with f32 scales: the quantization rule, the same kernel as the
//     activation quantizer (the page uses one rule for both);
//   - Q8_0 with f16 scales: d = fl16(amax / 127), q = trunc(x * (1 / d) +
//     copysign(0.5, x)) with d as rounded, clamped to [-127, 127]; a d
//     above 65504 cannot be stored;
//   - Q4_0 "round" rule: d = (first element of largest magnitude) / -8,
//     nibble = min(15, trunc(x * (1 / d) + 8.5)), 1 / d taken as 0 when
//     d = 0 or when 1 / d overflows (|d| < 2^-128); with f16 scales d is
//     stored as fl16(d), the nibbles use the float32 d.
//   - Q4_0 least-squares search: the largest element mx mapped to each
//     candidate level L = -6.0, -6.2, ..., -8.4; levels rint(x * (L / mx))
//     clamped to [-8, 7]; d = sum w x l / sum w l^2 with w = x^2; the
//     candidate of smallest weighted error sum w (x - d l)^2 wins (the first
//     on ties); a block below 1e-6 is divided by its largest magnitude
//     first and d multiplied back; the sums run in element order; a fit
//     that is not finite, or with f16 scales above 65504, is refused.
// An f16 Q8_0 scale that rounds to 0 gives q = 0 (the weights are 0 either
// way).
#include "device_common.h"
#include "kernels.h"

// No contraction: x * (1 / d) and the following add round separately.
#pragma clang fp contract(off)

namespace qmv {
namespace {

// One thread per block.  The source blocks sit at 2-byte alignment, so
// they are read as 16-bit words.
template <uint32_t WT>
__global__ __launch_bounds__(256) void gguf_repack_kernel(const uint16_t* __restrict__ src,
                                                          uint64_t nblocks, uint8_t* __restrict__ q,
                                                          uint16_t* __restrict__ d) {
    constexpr int QW = (WT == kQ4) ? 8 : 16;  // 16-bit words of quants per block
    const uint64_t k = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (k >= nblocks) return;
    const uint16_t* b = src + k * (1 + QW);
    uint32_t w[QW / 2];
#pragma unroll
    for (int i = 0; i < QW / 2; ++i)
        w[i] = static_cast<uint32_t>(b[1 + 2 * i]) | (static_cast<uint32_t>(b[2 + 2 * i]) << 16);
    uint4* qp = reinterpret_cast<uint4*>(q + k * (2 * QW));
#pragma unroll
    for (int i = 0; i < QW / 8; ++i)
        qp[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    d[k] = b[0];
}

// float32 -> f16 bits, round to nearest even.  The register barrier keeps the
// compiler from folding a multiply that produced f into a mixed-precision
// multiply-add with a +0 addend, which turns a -0 result into +0.
__device__ __forceinline__ uint16_t f16_bits(float f) {
    asm("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Q8_0 with f16 scales.  *bad is set when a scale does not fit f16.
__global__ __launch_bounds__(256) void quantize_q8_f16_kernel(const float* __restrict__ w,
                                                              uint64_t nblocks, int8_t* __restrict__ q,
                                                              uint16_t* __restrict__ d,
                                                              uint32_t* __restrict__ bad) {
    const uint64_t k = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (k >= nblocks) return;
    float v[32];
    const float4* xp = reinterpret_cast<const float4*>(w + 32 * k);
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
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    uint32_t packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint16_t db = 0;
    if (!(amax < 1e-30f)) {
        db = f16_bits(amax / 127.0f);
        if ((db & 0x7FFFu) >= 0x7C00u) *bad = 1u;  // above 65504
        const float d16 = static_cast<float>(__builtin_bit_cast(_Float16, db));
        if (d16 != 0.f) {
            const float id = 1.0f / d16;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t word = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float xj = v[4 * i + c];
                    const float u = xj * id + copysignf(0.5f, xj);
                    const float tr = fminf(fmaxf(truncf(u), -127.f), 127.f);
                    word |= (static_cast<uint32_t>(static_cast<int>(tr)) & 0xFFu) << (8 * c);
                }
                packed[i] = word;
            }
        }
    }
    uint4* qp = reinterpret_cast<uint4*>(q + 32 * k);
    qp[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    qp[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    d[k] = db;
}

// Q4_0, round rule.  d_out is float [nblocks] or uint16_t (f16) [nblocks].
template <bool SF16>
__global__ __launch_bounds__(256) void quantize_q4_round_kernel(const float* __restrict__ w,
                                                                uint64_t nblocks, uint8_t* __restrict__ q,
                                                                void* __restrict__ d_out,
                                                                uint32_t* __restrict__ bad) {
    const uint64_t k = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (k >= nblocks) return;
    float v[32];
    const float4* xp = reinterpret_cast<const float4*>(w + 32 * k);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = xp[i];
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
    // the first element of largest magnitude, with its sign
    float amax = 0.f, mx = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float a = fabsf(v[j]);
        if (a > amax) {
            amax = a;
            mx = v[j];
        }
    }
    const float d = mx / -8.0f;
    float id = d != 0.f ? 1.0f / d : 0.f;
    if (__builtin_isinf(id)) id = 0.f;  // |d| < 2^-128: the block writes as zeros
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = 4 * i + c;
            const float l0 = fminf(truncf(v[j] * id + 8.5f), 15.f);
            const float l1 = fminf(truncf(v[j + 16] * id + 8.5f), 15.f);
            const uint32_t byte = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 4);
            word |= byte << (8 * c);
        }
        packed[i] = word;
    }
    *reinterpret_cast<uint4*>(q + 16 * k) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if constexpr (SF16) {
        const uint16_t db = f16_bits(d);
        if ((db & 0x7FFFu) >= 0x7C00u) *bad = 1u;
        static_cast<uint16_t*>(d_out)[k] = db;
    } else {
        static_cast<float*>(d_out)[k] = d;
    }
}

// The 13 candidate levels of the least-squares search (the float32 nearest
// each decimal value).
__constant__ float kSearchLevel[13] = {-6.0f, -6.2f, -6.4f, -6.6f, -6.8f, -7.0f, -7.2f,
                                       -7.4f, -7.6f, -7.8f, -8.0f, -8.2f, -8.4f};

__device__ __forceinline__ float search_level(float v, float iscale) {
    return fminf(fmaxf(rintf(v * iscale), -8.f), 7.f);
}

// Q4_0 least-squares search, one thread per block: 13 candidates of 32
// levels, each scored by its weighted error (about 400 float32 operations
// per candidate); the winner's levels are computed again for the store.
template <bool SF16>
__global__ __launch_bounds__(256) void quantize_q4_search_kernel(const float* __restrict__ w,
                                                                 uint64_t nblocks, uint8_t* __restrict__ q,
                                                                 void* __restrict__ d_out,
                                                                 uint32_t* __restrict__ bad) {
    const uint64_t k = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (k >= nblocks) return;
    float v[32];
    const float4* xp = reinterpret_cast<const float4*>(w + 32 * k);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = xp[i];
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
    float amax = 0.f, mx = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float a = fabsf(v[j]);
        if (a > amax) {
            amax = a;
            mx = v[j];
        }
    }
    float d = 0.f, iscale = 0.f;  // iscale 0: every level 0 (nibble 8)
    if (amax != 0.f) {
        const bool tiny = amax < 1e-6f;
        if (tiny) {
#pragma unroll
            for (int j = 0; j < 32; ++j) v[j] = v[j] / amax;
            mx = mx / amax;
        }
        float wt[32], cube[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            wt[j] = v[j] * v[j];
            cube[j] = wt[j] * v[j];
        }
        float best_e = 0.f;
#pragma unroll 1
        for (int i = 0; i < 13; ++i) {
            const float is = kSearchLevel[i] / mx;
            float l[32];
            float sxl = 0.f, sll = 0.f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                l[j] = search_level(v[j], is);
                sxl = sxl + cube[j] * l[j];
                sll = sll + wt[j] * (l[j] * l[j]);
            }
            const float dc = sxl / sll;
            float e = 0.f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float r = v[j] - dc * l[j];
                e = e + wt[j] * (r * r);
            }
            if (i == 0 || e < best_e) {
                best_e = e;
                d = dc;
                iscale = is;
            }
        }
        if (tiny) d = d * amax;
        if (!__builtin_isfinite(d)) *bad = 1u;
    }
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = 4 * i + c;
            const uint32_t n0 = static_cast<uint32_t>(search_level(v[j], iscale) + 8.f);
            const uint32_t n1 = static_cast<uint32_t>(search_level(v[j + 16], iscale) + 8.f);
            word |= (n0 | (n1 << 4)) << (8 * c);
        }
        packed[i] = word;
    }
    *reinterpret_cast<uint4*>(q + 16 * k) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if constexpr (SF16) {
        const uint16_t db = f16_bits(d);
        if ((db & 0x7FFFu) >= 0x7C00u) *bad = 1u;
        static_cast<uint16_t*>(d_out)[k] = db;
    } else {
        static_cast<float*>(d_out)[k] = d;
    }
}

// Clears the status word and the zero padding between the q and d arrays
// (a kernel rather than memsets, so the call can be captured in a graph).
__global__ void writer_prepare_kernel(uint32_t* __restrict__ bad, uint8_t* __restrict__ pad,
                                      uint32_t pad_bytes) {
    const uint32_t t = threadIdx.x;
    if (t == 0) *bad = 0u;
    if (t < pad_bytes) pad[t] = 0;
}

}  // namespace

hipError_t launch_gguf_repack(uint32_t wtype, const void* src, uint64_t nblocks, uint8_t* q,
                              uint16_t* d, hipStream_t s) {
    const uint64_t grid = (nblocks + 255) / 256;
    if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const uint16_t* p = static_cast<const uint16_t*>(src);
    if (wtype == kQ4)
        hipLaunchKernelGGL(gguf_repack_kernel<kQ4>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                           p, nblocks, q, d);
    else
        hipLaunchKernelGGL(gguf_repack_kernel<kQ8>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                           p, nblocks, q, d);
    return hipGetLastError();
}

hipError_t launch_quantize_weights(uint32_t wtype, uint32_t scale_f16, uint32_t rule,
                                   const float* w, uint64_t nblocks, uint8_t* q, uint32_t q_pad,
                                   void* d, uint32_t* bad, hipStream_t s) {
    if (q_pad >= 64 || (rule != 0 && wtype != kQ4)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(writer_prepare_kernel, dim3(1), dim3(64), 0, s, bad,
                       q + nblocks * (wtype == kQ4 ? 16 : 32), q_pad);
    if (wtype == kQ8 && !scale_f16)
        return launch_quantize_q8(w, nblocks * 32, reinterpret_cast<int8_t*>(q), static_cast<float*>(d), s);
    const uint64_t grid = (nblocks + 255) / 256;
    if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const dim3 g(static_cast<uint32_t>(grid)), b(256);
    if (rule != 0) {
        if (scale_f16)
            hipLaunchKernelGGL(quantize_q4_search_kernel<true>, g, b, 0, s, w, nblocks, q, d, bad);
        else
            hipLaunchKernelGGL(quantize_q4_search_kernel<false>, g, b, 0, s, w, nblocks, q, d, bad);
    } else if (wtype == kQ8)
        hipLaunchKernelGGL(quantize_q8_f16_kernel, g, b, 0, s, w, nblocks, reinterpret_cast<int8_t*>(q),
                           static_cast<uint16_t*>(d), bad);
    else if (scale_f16)
        hipLaunchKernelGGL(quantize_q4_round_kernel<true>, g, b, 0, s, w, nblocks, q, d, bad);
    else
        hipLaunchKernelGGL(quantize_q4_round_kernel<false>, g, b, 0, s, w, nblocks, q, d, bad);
    return hipGetLastError();
}

}  // namespace qmv
