// Small device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qmv {

constexpr uint32_t kQ8 = 1;  // .mlb wtype code of Q8_0
constexpr uint32_t kQ4 = 2;  // .mlb wtype code of Q4_0

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Scale k as float32.  An IEEE binary16 scale widens exactly
// (v_cvt_f32_f16 keeps f16 subnormals).
template <bool SF16>
__device__ __forceinline__ float load_scale(const void* __restrict__ d, uint64_t k) {
    if constexpr (SF16) {
        const uint16_t h = static_cast<const uint16_t*>(d)[k];
        return static_cast<float>(__builtin_bit_cast(_Float16, h));
    } else {
        return static_cast<const float*>(d)[k];
    }
}

// Byte i (0..3) of a 32-bit word converted to float (v_cvt_f32_ubyteN).
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
    return static_cast<float>((w >> (8 * I)) & 0xFFu);
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace qmv
