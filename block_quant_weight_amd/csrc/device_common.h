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

// Raw bits of scale k (f16 in the low half, or f32), and their value.
template <bool SF16>
__device__ __forceinline__ uint32_t load_scale_bits(const void* __restrict__ d, uint64_t k) {
    if constexpr (SF16) return static_cast<const uint16_t*>(d)[k];
    else return static_cast<const uint32_t*>(d)[k];
}
template <bool SF16>
__device__ __forceinline__ float scale_from_bits(uint32_t b) {
    if constexpr (SF16)
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
    else return __builtin_bit_cast(float, b);
}

// Byte i (0..3) of a 32-bit word converted to float (v_cvt_f32_ubyteN).
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
    return static_cast<float>((w >> (8 * I)) & 0xFFu);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float read_lane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes of a wavefront, returned in every lane.  DPP moves
// reduce each row of 16 lanes (swap neighbours, swap pairs, rotate by 4 and
// by 8), then the four row sums are read out and added in a fixed order.
__device__ __forceinline__ float wave_reduce(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x124>(v);  // row_ror:4
    v += dpp_mov<0x128>(v);  // row_ror:8
    return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

}  // namespace qmv
