// Batched decode product on the matrix cores, f16 operands: Y[t][r] =
// sum_c W[r][c] x[t][c] for a Q8_0 matrix with f16 scales and up to 1024
// columns over batches above 8 — the shared classifier (LM head) applied to a
// batch of hidden states (Krafla ".mlb model, version 1" page, header field
// `shared_classifier`; "Body" for the product, "Q8_0" for w = q * d).
//
// Operands.  Each workgroup converts the batch's activations once: token t is
// scaled by 2^(14 - E_t), E_t the exponent of its largest magnitude, and
// rounded to f16 (relative error <= 2^-11 for every value within 2^28 of the
// largest; a non-finite activation makes the token's outputs NaN).  A weight
// enters as fl16(q * d * 2^(8 - E_d)), E_d the exponent of the matrix's
// largest scale: d * 2^(8 - E_d) is exact in f16 (at most 256) and the
// product q * d' of two exact f16 values is rounded once (relative error
// <= 2^-11), built from the quant byte with a byte permute (f16 1024 + u, u =
// q + 128), an exact f16 subtraction of 1152 and one f16 multiply.  The
// matrix cores multiply the f16 values exactly and accumulate in float32;
// the outputs are scaled back by powers of two.  Each output is thus within
// about 2^-10 * sum_c |W[r][c]| |x[t][c]| (+ float32 rounding) of the exact
// product, half the 2e-3 tolerance.
//
// Work split.  One workgroup of 8 waves per compute unit keeps up to 64
// tokens of f16 activations in LDS (one row of 2*cols + 16 bytes per token,
// the 16-byte pad spreading a wave's fragment reads over all banks).  Each
// wave walks tiles of 32 weight rows; tokens are the A operand (two 32-token
// tiles) and weight rows the B operand of v_mfma_f32_32x32x16_f16, so a
// lane's output column is a weight row and stores of 32 consecutive rows per
// token coalesce.  Lane (r, h) = (lane % 32, lane / 32) loads 16 quant bytes
// of row r at 32j + 16h per block j (one 16-byte load per lane and block, the
// two halves of a lane pair covering the 32-byte block), which feed two
// matrix-core steps; the activations are read with the same split of k, so
// A and B agree on which k each step sums.  The loads run kRing blocks ahead
// through a ring of registers (raw buffer loads: past the last tile they get
// an out-of-range offset and return zeros, so the ring needs no branches).
#include "device_common.h"
#include "kernels.h"

namespace qmv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kTokens = 64;     // tokens per pass (two 32-token tiles)
constexpr int kMaxCols = 1024;  // activations of one pass must fit LDS
constexpr int kRing = 8;        // blocks of quants in flight per wave
constexpr uint32_t kOob = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// Largest value over the wave (each lane's v an unsigned magnitude).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x124, 0xF, 0xF, true)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, true)));
    const uint32_t a = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16)));
    const uint32_t b = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48)));
    return max(a, b);
}

// 16 Q8_0 quants (one lane's half block) -> 16 f16 weights q * d'.
__device__ __forceinline__ void dequant16(const u32x4 w, f16x2 dd, f16x8 (&out)[2]) {
    const f16x2 bias = {static_cast<_Float16>(1152.f), static_cast<_Float16>(1152.f)};
    f16x2 h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = w[i] ^ 0x80808080u;  // q + 128 in each byte
        // [u0, 0x64, u1, 0x64] and [u2, 0x64, u3, 0x64]: f16 values 1024 + u
        const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
        const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
        h[2 * i] = (__builtin_bit_cast(f16x2, lo) - bias) * dd;      // exact q, one rounding
        h[2 * i + 1] = (__builtin_bit_cast(f16x2, hi) - bias) * dd;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[k][2 * i] = h[4 * k + i][0];
            out[k][2 * i + 1] = h[4 * k + i][1];
        }
}

__global__ __launch_bounds__(kWaves * 64) void gemv_mfma_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ d, const float* __restrict__ x,
    float* __restrict__ y, uint32_t rows, uint32_t cols, uint32_t ntok, float wscale,
    float inv_wscale) {
    __shared__ __align__(16) uint8_t xs[kTokens * (2 * kMaxCols + 16)];
    __shared__ float tinv[kTokens];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t P = 2 * cols + 16;  // LDS bytes per token
    const uint32_t nj = cols / 32;     // blocks per row = steps per tile
    const uint32_t r = lane & 31, h = lane >> 5;

    // ---- ring prologue: the first kRing blocks of this wave's tiles ----
    const uint32_t tiles = (rows + 31) / 32;
    const uint32_t first = blockIdx.x * kWaves + wid;
    const uint32_t stride = gridDim.x * kWaves;
    const uint32_t my_tiles = first < tiles ? (tiles - first + stride - 1) / stride : 0;
    const uint32_t nsteps = my_tiles * nj;
    const __amdgpu_buffer_rsrc_t qrs = rsrc(q, rows * cols);
    const __amdgpu_buffer_rsrc_t drs = rsrc(d, rows * nj * 2);
    u32x4 rq[kRing];
    uint32_t rd[kRing];
    uint32_t lt = 0, lj = 0;  // tile (of this wave) and block of the next load
    auto load = [&](int slot) {
        const uint32_t row = (first + lt * stride) * 32 + r;
        const bool ok = lt < my_tiles && row < rows;
        const uint32_t qo = ok ? row * cols + 32 * lj + 16 * h : kOob;
        const uint32_t dof = ok ? (row * nj + lj) * 2 : kOob;
        rd[slot] = __builtin_amdgcn_raw_buffer_load_b16(drs, dof, 0, 0);
        rq[slot] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qo, 0, 0);
        if (++lj == nj) { lj = 0; ++lt; }
    };
#pragma unroll
    for (int u = 0; u < kRing; ++u) load(u);

    // ---- activations -> f16 in LDS: wave w converts tokens w, w + 8, ...,
    // with all of its loads requested first (one round trip, not eight) ----
    constexpr int TPW = kTokens / kWaves;  // tokens per wave
    float4 v[TPW][4];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const uint32_t t = wid + kWaves * k;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t c4 = lane + 64 * i;  // float4 index within the token
            v[k][i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t < ntok && 4 * c4 < cols)
                v[k][i] = reinterpret_cast<const float4*>(x + static_cast<uint64_t>(t) * cols)[c4];
        }
    }
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const uint32_t t = wid + kWaves * k;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m = max(m, __builtin_bit_cast(uint32_t, v[k][i].x) & 0x7FFFFFFFu);
            m = max(m, __builtin_bit_cast(uint32_t, v[k][i].y) & 0x7FFFFFFFu);
            m = max(m, __builtin_bit_cast(uint32_t, v[k][i].z) & 0x7FFFFFFFu);
            m = max(m, __builtin_bit_cast(uint32_t, v[k][i].w) & 0x7FFFFFFFu);
        }
        m = wave_max_u32(m);
        const bool finite = m < 0x7F800000u;
        const int E = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, m));
        const int sh = finite ? 14 - E : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t c4 = lane + 64 * i;
            if (4 * c4 < cols) {
                float4 a = v[k][i];
                if (!finite) a = make_float4(0.f, 0.f, 0.f, 0.f);
                const f16x2 p0 = {static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.x, sh)),
                                  static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.y, sh))};
                const f16x2 p1 = {static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.z, sh)),
                                  static_cast<_Float16>(__builtin_amdgcn_ldexpf(a.w, sh))};
                *reinterpret_cast<uint2*>(xs + t * P + 8 * c4) =
                    make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
            }
        }
        if (lane == 0)
            tinv[t] = t >= ntok ? 0.f
                    : finite ? __builtin_amdgcn_ldexpf(1.0f, -sh) * inv_wscale
                             : __builtin_bit_cast(float, 0x7FC00000u);
    }
    __syncthreads();

    // ---- tiles: kRing blocks per round; a tile's nj blocks are a whole
    // number of rounds (cols % (32 * kRing) == 0), so tiles end between
    // rounds.  Stores are raw buffer stores (a token or row past the end gets
    // an out-of-range offset and is dropped, no branch).
    const __amdgpu_buffer_rsrc_t yrs = rsrc(y, ntok * rows * 4);
    f32x16 acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;
    uint32_t ct = 0, cj = 0;  // tile and first block of the round being multiplied
    for (uint32_t s0 = 0; s0 < nsteps; s0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            // weights of block cj + u: d' = d * 2^(8 - E_d), exact in f16
            const _Float16 ds = static_cast<_Float16>(
                static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(rd[u]))) * wscale);
            const f16x2 dd = {ds, ds};
            f16x8 wf[2];
            dequant16(rq[u], dd, wf);
            load(u);  // the ring slot is free again: the block kRing ahead
            // activations of the same block, both token tiles, same split of k
            f16x8 xf[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint8_t* p = xs + (32 * mt + r) * P + 2 * (32 * (cj + u) + 16 * h);
                xf[mt][0] = *reinterpret_cast<const f16x8*>(p);
                xf[mt][1] = *reinterpret_cast<const f16x8*>(p + 16);
            }
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[mt][k], wf[k], acc[mt], 0, 0, 0);
        }
        cj += kRing;
        if (cj == nj) {
            const uint32_t row = (first + ct * stride) * 32 + r;
            const bool rok = row < rows;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const uint32_t t = 32 * mt + 8 * (v / 4) + 4 * h + (v % 4);
                    const uint32_t off = (rok && t < ntok) ? (t * rows + row) * 4 : kOob;
                    // the store takes the 32-bit pattern (an unsigned int)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __builtin_bit_cast(uint32_t, acc[mt][v] * tinv[t]), yrs, off, 0, 0);
                    acc[mt][v] = 0.f;
                }
            cj = 0;
            ++ct;
        }
    }
}

}  // namespace

hipError_t launch_gemv_mfma(const MatView& m, const float* x, float* y, uint32_t batch,
                            hipStream_t s) {
    // Q8_0 with f16 scales, cols a multiple of 256 fitting one pass of
    // activations in LDS, and weights and outputs within 32-bit buffer offsets
    if (m.wtype != kQ8 || !m.scale_f16 || m.cols > static_cast<uint32_t>(kMaxCols) ||
        m.cols % (32 * kRing) != 0 || static_cast<uint64_t>(m.rows) * m.cols >= 0xFFFFFFF0ull ||
        static_cast<uint64_t>(m.rows) * kTokens * 4 >= 0xFFFFFFF0ull)
        return hipErrorNotSupported;
    const float wscale = ldexpf(1.0f, 8 - m.dexp);
    const float inv = ldexpf(1.0f, m.dexp - 8);
    const uint32_t tiles = (m.rows + 31) / 32;
    const uint32_t want = (tiles + kWaves - 1) / kWaves;
    const uint32_t blocks = want < 256 ? want : 256;
    for (uint32_t done = 0; done < batch; done += kTokens) {
        const uint32_t nt = batch - done < static_cast<uint32_t>(kTokens) ? batch - done : kTokens;
        hipLaunchKernelGGL(gemv_mfma_kernel, dim3(blocks), dim3(kWaves * 64), 0, s, m.q,
                           static_cast<const uint16_t*>(m.d), x + static_cast<uint64_t>(done) * m.cols,
                           y + static_cast<uint64_t>(done) * m.rows, m.rows, m.cols, nt, wscale, inv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmv
