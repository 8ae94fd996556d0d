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

// ---------------------------------------------------------------------------
// Large-batch kernel: tile 256 tokens x 128 matrix rows, BK = 64.
//
// Eight waves in two groups of four.  Within a group the waves are 2 x 2,
// each multiplying 128 tokens x 64 rows (4 x 2 tiles of 32x32) per 16-wide
// k slice: 6 LDS fragment reads feed 8 MFMAs.  Group 0 takes k slices 0 and
// 2 of every step, group 1 slices 1 and 3, so each SIMD runs two waves (one
// stalls, the other issues) while the LDS traffic per MFMA stays that of a
// 128 x 64 wave tile; the groups' sums are added through LDS at the end.
// The weights of a tile are decoded once per workgroup: each thread decodes
// half a quant block per step with fma(code, d, -OFF*d) = fl32((code - OFF)
// * d), bit-identical to the single f32 product v * d, then
// v_cvt_pk_bf16_f32 (round to nearest even).
//
// Pipeline: LDS is double-buffered; global loads for step s + 2 are issued
// into a register set before step s is multiplied, and the set of step s + 1
// is written to the other LDS buffer in parts between the k slices.  All
// loads are raw buffer loads; rows, tokens and k past the end get an
// out-of-range offset (zeros, no traffic).  With split-K (grid.z) each slice
// writes its partial tile to a workspace that a second kernel sums in slice
// order.
// ---------------------------------------------------------------------------

namespace big {

constexpr int BM = 256, BN = 128, BK = 64, LDK = BK + 8;
constexpr int NT = 512;                   // threads per workgroup
constexpr int XSEG = BM * BK / 8 / NT;    // 16-byte activation segments per thread per step

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kOob = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(n), 0x00020000);
}

// One step's global data held by a thread: XSEG activation segments and half
// a quant block (Q4_0: 8 bytes, Q8_0: 16 bytes) with its scale.
template <uint32_t WT>
struct Stage {
    uint4 xs[XSEG];
    uint32_t q[WT == kQ4 ? 2 : 4];
    uint32_t d;
};

template <uint32_t WT, bool SF16>
struct Ctx {
    __amdgpu_buffer_rsrc_t xr, qr, dr;
    uint32_t M, N, K, m0, n0, ke;
    int tid;
    // fetch step k0 into st (k0 may be past ke: then everything is out of range)
    __device__ __forceinline__ void fetch(uint32_t k0, Stage<WT>& st) const {
#pragma unroll
        for (int i = 0; i < XSEG; ++i) {
            const int seg = tid + NT * i;
            const uint32_t r = seg >> 3, c8 = (seg & 7) * 8;
            const uint32_t m = m0 + r, k = k0 + c8;
            const uint32_t off = (m < M && k < ke) ? (m * K + k) * 2 : kOob;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            st.xs[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
        // thread -> (row r, block b, half h) of the 128 x 2 blocks
        const uint32_t r = tid >> 2, b = (tid >> 1) & 1, h = tid & 1;
        const uint32_t n = n0 + r, k = k0 + 32 * b;
        const bool ok = n < N && k < ke;
        const uint32_t blk = n * (K >> 5) + (k >> 5);
        if constexpr (WT == kQ4) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(qr, ok ? blk * 16 + 8 * h : kOob, 0, 0);
            st.q[0] = v[0];
            st.q[1] = v[1];
        } else {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qr, ok ? blk * 32 + 16 * h : kOob, 0, 0);
            st.q[0] = v[0];
            st.q[1] = v[1];
            st.q[2] = v[2];
            st.q[3] = v[3];
        }
        if constexpr (SF16) st.d = __builtin_amdgcn_raw_buffer_load_b16(dr, ok ? blk * 2 : kOob, 0, 0);
        else st.d = __builtin_amdgcn_raw_buffer_load_b32(dr, ok ? blk * 4 : kOob, 0, 0);
    }
};

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

// Write step data to LDS in two parts (placed between the k slices so the
// decode interleaves with the matrix cores): part 0 copies the activation
// segments, part 1 decodes the thread's half block to bf16.  Q4_0 half h
// holds bytes 8h .. 8h + 7: elements 8h .. 8h + 7 (low nibbles) and
// 16 + 8h .. 16 + 8h + 7 (high nibbles).  Q8_0 half h is elements 16h ..
// 16h + 15.
template <uint32_t WT, bool SF16, int PART>
__device__ __forceinline__ void store_part(const Stage<WT>& st, __bf16* __restrict__ xs,
                                           __bf16* __restrict__ ws, int tid) {
    if constexpr (PART == 0) {
#pragma unroll
        for (int i = 0; i < XSEG; ++i) {
            const int seg = tid + NT * i;
            const int r = seg >> 3, c8 = (seg & 7) * 8;
            *reinterpret_cast<uint4*>(&xs[r * LDK + c8]) = st.xs[i];
        }
    } else {
        const float dv = scale_from_bits<SF16>(st.d);
        const int r = tid >> 2, b = (tid >> 1) & 1, h = tid & 1;
        __bf16* row = &ws[r * LDK + 32 * b];
        if constexpr (WT == kQ4) {
            // w = (n - 8) d = fma(n, d, -8d): n d and 8 d are exact, one rounding
            const float m8d = -8.f * dv;
            uint32_t mask = 0x0F0F0F0Fu;
            asm("" : "+v"(mask));
            float lo[8], hi[8];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t l = st.q[i] & mask, hh = (st.q[i] >> 4) & mask;
                lo[4 * i + 0] = fmaf(ubyte_f32<0>(l), dv, m8d);
                lo[4 * i + 1] = fmaf(ubyte_f32<1>(l), dv, m8d);
                lo[4 * i + 2] = fmaf(ubyte_f32<2>(l), dv, m8d);
                lo[4 * i + 3] = fmaf(ubyte_f32<3>(l), dv, m8d);
                hi[4 * i + 0] = fmaf(ubyte_f32<0>(hh), dv, m8d);
                hi[4 * i + 1] = fmaf(ubyte_f32<1>(hh), dv, m8d);
                hi[4 * i + 2] = fmaf(ubyte_f32<2>(hh), dv, m8d);
                hi[4 * i + 3] = fmaf(ubyte_f32<3>(hh), dv, m8d);
            }
            *reinterpret_cast<uint4*>(row + 8 * h) =
                make_uint4(pk_bf16(lo[0], lo[1]), pk_bf16(lo[2], lo[3]), pk_bf16(lo[4], lo[5]),
                           pk_bf16(lo[6], lo[7]));
            *reinterpret_cast<uint4*>(row + 16 + 8 * h) =
                make_uint4(pk_bf16(hi[0], hi[1]), pk_bf16(hi[2], hi[3]), pk_bf16(hi[4], hi[5]),
                           pk_bf16(hi[6], hi[7]));
        } else {
            // w = q d = fma(q + 128, d, -128 d): one rounding of the exact q d
            const float m128d = -128.f * dv;
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = st.q[i] ^ 0x80808080u;
                o[2 * i] = pk_bf16(fmaf(ubyte_f32<0>(w), dv, m128d), fmaf(ubyte_f32<1>(w), dv, m128d));
                o[2 * i + 1] = pk_bf16(fmaf(ubyte_f32<2>(w), dv, m128d), fmaf(ubyte_f32<3>(w), dv, m128d));
            }
            *reinterpret_cast<uint4*>(row + 16 * h) = make_uint4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<uint4*>(row + 16 * h + 8) = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
}

template <uint32_t WT, bool SF16>
__global__ __launch_bounds__(NT) void gemm_big_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d, const uint16_t* __restrict__ x,
    float* __restrict__ y, float* __restrict__ ws_partial, uint32_t M, uint32_t N, uint32_t K,
    uint32_t k_per_split) {
    constexpr int TM = 4, TN = 2;
    __shared__ __attribute__((aligned(16))) __bf16 Xs[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 Ws[2][BN * LDK];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int grp = wid >> 2;                    // which k slices: 2 grp, 2 grp + 1 ... (see below)
    const int wm = (wid >> 1) & 1, wn = wid & 1;
    Ctx<WT, SF16> c;
    c.M = M; c.N = N; c.K = K; c.tid = tid;
    c.m0 = blockIdx.y * BM;
    c.n0 = blockIdx.x * BN;
    const uint32_t kb = blockIdx.z * k_per_split;
    c.ke = min(K, kb + k_per_split);
    c.xr = rsrc(x, static_cast<uint64_t>(M) * K * 2);
    const uint64_t qbytes = (WT == kQ4) ? static_cast<uint64_t>(N) * K / 2 : static_cast<uint64_t>(N) * K;
    c.qr = rsrc(q, qbytes);
    c.dr = rsrc(d, static_cast<uint64_t>(N) * (K / 32) * (SF16 ? 2 : 4));

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    Stage<WT> sa, sb;
    c.fetch(kb, sa);
    c.fetch(kb + BK, sb);
    store_part<WT, SF16, 0>(sa, Xs[0], Ws[0], tid);
    store_part<WT, SF16, 1>(sa, Xs[0], Ws[0], tid);
    __syncthreads();

    // One step: this group's two k slices (16 grp and 32 + 16 grp) of MFMAs
    // on LDS buffer `cur`, with the two store parts of the next step's data
    // (register set nx) into the other buffer between them.
    auto step = [&](int cur, const Stage<WT>& nx) {
        const __bf16* __restrict__ xs = Xs[cur];
        const __bf16* __restrict__ wsb = Ws[cur];
        bf16x8 a[2][TM], b[2][TN];
        auto frags = [&](int kk, int set) {
            const int kc = kk + 8 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[set][i] = *reinterpret_cast<const bf16x8*>(&xs[(wm * 128 + i * 32 + (lane & 31)) * LDK + kc]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[set][j] = *reinterpret_cast<const bf16x8*>(&wsb[(wn * 64 + j * 32 + (lane & 31)) * LDK + kc]);
        };
        auto mm = [&](int set) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[set][i], b[set][j], acc[i][j], 0, 0, 0);
        };
        frags(16 * grp, 0);
        frags(32 + 16 * grp, 1);
        mm(0);
        store_part<WT, SF16, 0>(nx, Xs[cur ^ 1], Ws[cur ^ 1], tid);
        mm(1);
        store_part<WT, SF16, 1>(nx, Xs[cur ^ 1], Ws[cur ^ 1], tid);
    };

    // Step s reads LDS[s & 1]; sa/sb alternate as the register set of step
    // s + 1.  The loop exit sits after the barrier so that each step's MFMAs
    // and the next step's stores form one block the scheduler can
    // interleave; the last step stores (zeros) into the unused buffer.
    uint32_t k0 = kb;
    for (;;) {
        c.fetch(k0 + 2 * BK, sa);          // step s + 2
        step(0, sb);
        __syncthreads();
        if (k0 + BK >= c.ke) break;
        c.fetch(k0 + 3 * BK, sb);
        step(1, sa);
        __syncthreads();
        k0 += 2 * BK;
        if (k0 >= c.ke) break;
    }

    // ---- add group 1's sums into group 0's through LDS (the stage buffers
    // are free now), two tile columns at a time ----
    float* red = reinterpret_cast<float*>(&Xs[0][0]);  // 4 waves x 4 tiles x 16 x 64 floats
    const int wq = wid & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (grp == 1) {
#pragma unroll
            for (int i = 2 * half; i < 2 * half + 2; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        red[(((wq * 4 + (i - 2 * half) * TN + j) * 16 + v) << 6) + lane] = acc[i][j][v];
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int i = 2 * half; i < 2 * half + 2; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[i][j][v] += red[(((wq * 4 + (i - 2 * half) * TN + j) * 16 + v) << 6) + lane];
        }
        __syncthreads();
    }
    if (grp == 1) return;

    // epilogue: lane holds column n = lane % 32, rows 8 (v / 4) + 4 (lane / 32) + v % 4
    float* out = ws_partial ? ws_partial + static_cast<uint64_t>(blockIdx.z) * M * N : y;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t m = c.m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const uint32_t n = c.n0 + wn * 64 + j * 32 + (lane & 31);
                if (m < M && n < N) out[static_cast<uint64_t>(m) * N + n] = acc[i][j][v];
            }
}

// y = sum of the split-K partials, in slice order (deterministic).  Slice z
// starts at part + z * total; with total % 4 == 0 every slice is 16-byte
// aligned and each thread adds float4s, else single floats.
template <bool VEC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            float* __restrict__ y, uint64_t total,
                                                            uint32_t splits) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if constexpr (VEC) {
        if (4 * i >= total) return;
        const float4* p = reinterpret_cast<const float4*>(part);
        const uint64_t t4 = total / 4;
        float4 s = p[i];
        for (uint32_t z = 1; z < splits; ++z) {
            const float4 t = p[z * t4 + i];
            s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
        }
        reinterpret_cast<float4*>(y)[i] = s;
    } else {
        if (i >= total) return;
        float s = part[i];
        for (uint32_t z = 1; z < splits; ++z) s += part[z * total + i];
        y[i] = s;
    }
}

}  // namespace big

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

namespace {

// Shape of the large-batch launch: tiles and split-K slices.
struct BigPlan {
    bool use = false;
    uint32_t tiles_n = 0, tiles_m = 0, splits = 1, k_per_split = 0;
};

BigPlan big_plan(const MatView& m, uint32_t batch, bool x_f32) {
    BigPlan p;
    if (x_f32 || batch < 128) return p;
    // 32-bit buffer offsets over the activations, quants and scales
    const uint64_t qbytes = (m.wtype == kQ4) ? uint64_t{m.rows} * m.cols / 2
                                             : uint64_t{m.rows} * m.cols;
    if (uint64_t{batch} * m.cols * 2 >= 0xFFFFFFF0ull || qbytes >= 0xFFFFFFF0ull ||
        uint64_t{m.rows} * (m.cols / 32) * 4 >= 0xFFFFFFF0ull)
        return p;
    p.use = true;
    p.tiles_n = (m.rows + big::BN - 1) / big::BN;
    p.tiles_m = (batch + big::BM - 1) / big::BM;
    const uint32_t tiles = p.tiles_n * p.tiles_m;
    const uint32_t steps = (m.cols + big::BK - 1) / big::BK;
    // too few tiles for 256 compute units: split K, keeping >= 8 steps a slice
    uint32_t splits = 1;
    while (tiles * splits * 2 <= 320 && steps / (splits * 2) >= 8) splits *= 2;
    const uint32_t per = (steps + splits - 1) / splits;
    p.k_per_split = per * big::BK;
    p.splits = (m.cols + p.k_per_split - 1) / p.k_per_split;
    return p;
}

}  // namespace

hipError_t launch_splitk_sum(const float* part, float* y, uint64_t total, uint32_t splits,
                             hipStream_t s) {
    const bool vec = total % 4 == 0;
    const uint64_t blocks = ((vec ? total / 4 : total) + 255) / 256;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (vec)
        hipLaunchKernelGGL(big::splitk_reduce_kernel<true>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(256), 0, s, part, y, total, splits);
    else
        hipLaunchKernelGGL(big::splitk_reduce_kernel<false>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(256), 0, s, part, y, total, splits);
    return hipGetLastError();
}

size_t gemm_workspace_bytes(const MatView& m, uint32_t batch, bool x_f32) {
    const BigPlan p = big_plan(m, batch, x_f32);
    if (!p.use || p.splits == 1) return 0;
    return static_cast<size_t>(p.splits) * batch * m.rows * sizeof(float);
}

hipError_t launch_gemm(const MatView& m, const void* x, bool x_f32, float* y,
                       uint32_t batch, float* workspace, hipStream_t s) {
    const BigPlan p = big_plan(m, batch, x_f32);
    if (p.use) {
        if (p.tiles_m > 65535u || p.splits > 65535u) return hipErrorInvalidValue;
        float* part = p.splits > 1 ? workspace : nullptr;
        if (p.splits > 1 && part == nullptr) return hipErrorInvalidValue;
        const dim3 grid(p.tiles_n, p.tiles_m, p.splits);
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        if (m.wtype == kQ4) {
            if (m.scale_f16)
                hipLaunchKernelGGL((big::gemm_big_kernel<kQ4, true>), grid, dim3(big::NT), 0, s,
                                   m.q, m.d, xb, y, part, batch, m.rows, m.cols, p.k_per_split);
            else
                hipLaunchKernelGGL((big::gemm_big_kernel<kQ4, false>), grid, dim3(big::NT), 0, s,
                                   m.q, m.d, xb, y, part, batch, m.rows, m.cols, p.k_per_split);
        } else {
            if (m.scale_f16)
                hipLaunchKernelGGL((big::gemm_big_kernel<kQ8, true>), grid, dim3(big::NT), 0, s,
                                   m.q, m.d, xb, y, part, batch, m.rows, m.cols, p.k_per_split);
            else
                hipLaunchKernelGGL((big::gemm_big_kernel<kQ8, false>), grid, dim3(big::NT), 0, s,
                                   m.q, m.d, xb, y, part, batch, m.rows, m.cols, p.k_per_split);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.splits == 1) return e;
        return launch_splitk_sum(part, y, static_cast<uint64_t>(batch) * m.rows, p.splits, s);
    }
    // grid.y carries the token tiles: at most 65535 of them
    if ((batch + 63) / 64 > 65535u) return hipErrorInvalidValue;
    return x_f32 ? gemm_by_type<true>(m, x, y, batch, s)
                 : gemm_by_type<false>(m, x, y, batch, s);
}

}  // namespace qmv
