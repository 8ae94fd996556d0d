// Decode product (GEMV) for Q4_0 / Q8_0 matrices on gfx950.
//
// y[t][r] = sum_c W[r][c] * x[t][c] (Krafla ".mlb model, version 1" page,
// "Body": rows are outputs).  The weights stay quantized in HBM and are
// decoded in registers: a Q4_0 block keeps elements 0..15 in the low four
// bits of its 16 bytes and elements 16..31 in the high four bits, w =
// (nibble - 8) * d (section "Q4_0"); Q8_0 w = q * d (section "Q8_0").
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
//
// The mask is passed through an empty asm so the optimizer cannot see its
// value: otherwise it rewrites mask + v_cvt_f32_ubyteN (1.25 instructions
// per weight) as v_bfe_u32 + v_cvt_f32_ubyte0 (2 per weight).
__device__ __forceinline__ float q4_raw_dot(const uint4 qv, const float (&xs)[32]) {
    uint32_t mask = 0x0F0F0F0Fu;
    asm("" : "+v"(mask));
    const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & mask;
        const uint32_t hi = (w[i] >> 4) & mask;
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

// Loads the quants and the raw scale bits of chunk ch of each of the NR
// rows.  The scales are widened only where they are used, so that nothing
// waits for a prefetch before its step.
template <uint32_t WT, bool SF16, int NR>
__device__ __forceinline__ void load_chunk(const uint8_t* const (&qr)[NR],
                                           const uint64_t (&dr)[NR],
                                           const void* __restrict__ d, uint32_t ch,
                                           uint4 (&qv)[NR], uint32_t (&dv)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
        qv[r] = *reinterpret_cast<const uint4*>(qr[r] + 16ull * ch);
#pragma unroll
    for (int r = 0; r < NR; ++r)
        dv[r] = load_scale_bits<SF16>(d, dr[r] + (WT == kQ4 ? ch : (ch >> 1)));
}

template <int CW>
__device__ __forceinline__ void load_x(const float* __restrict__ xp, float (&xs)[CW]) {
    const float4* p = reinterpret_cast<const float4*>(xp);
#pragma unroll
    for (int i = 0; i < CW / 4; ++i) {
        const float4 t = p[i];
        xs[4 * i + 0] = t.x;
        xs[4 * i + 1] = t.y;
        xs[4 * i + 2] = t.z;
        xs[4 * i + 3] = t.w;
    }
}

// acc += d * (raw - OFF * sum x) for each row, kept only where `valid`
// (a select, not a branch: a branch would let the compiler sink the
// prefetch loads into it).
template <uint32_t WT, bool SF16, int NR, int CW>
__device__ __forceinline__ void accumulate(const uint4 (&qv)[NR], const uint32_t (&dbits)[NR],
                                           const float (&xs)[CW], bool valid,
                                           float (&acc)[NR]) {
    constexpr float OFF = (WT == kQ4) ? 8.f : 128.f;
    float sx;
    if constexpr (WT == kQ4) sx = q4_xsum(xs); else sx = q8_xsum(xs);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float raw;
        if constexpr (WT == kQ4) raw = q4_raw_dot(qv[r], xs);
        else raw = q8_raw_dot(qv[r], xs);
        const float t = fmaf(scale_from_bits<SF16>(dbits[r]), raw - OFF * sx, acc[r]);
        acc[r] = valid ? t : acc[r];
    }
}

// One step of the chunk loop: multiply chunk `ch` (quants already in cq)
// and, if PREFETCH, request the quants of chunk `nxt` into nq.  The
// activations of `ch` are requested before that prefetch: loads complete in
// issue order, so waiting for the activations must not wait for the
// prefetch.  Whether to prefetch is a template parameter, never a branch, so
// the wait-count placement sees one path.
template <uint32_t WT, bool SF16, int NR, int NB, int CW, bool PREFETCH>
__device__ __forceinline__ void gemv_step(
    const uint8_t* const (&qr)[NR], const uint64_t (&dr)[NR], const void* __restrict__ d,
    const float* __restrict__ x, uint32_t cols, uint32_t ch, bool valid, uint32_t nxt,
    const uint4 (&cq)[NR], const uint32_t (&cd)[NR], uint4 (&nq)[NR], uint32_t (&nd)[NR],
    float (&acc)[NB][NR]) {
    if constexpr (NB * CW <= 64) {
        float xs[NB][CW];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            load_x<CW>(x + static_cast<uint64_t>(b) * cols + static_cast<uint64_t>(ch) * CW, xs[b]);
        // keep the issue order: activations, then the prefetch, then math
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PREFETCH) load_chunk<WT, SF16, NR>(qr, dr, d, nxt, nq, nd);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b) accumulate<WT, SF16, NR, CW>(cq, cd, xs[b], valid, acc[b]);
    } else {
        if constexpr (PREFETCH) load_chunk<WT, SF16, NR>(qr, dr, d, nxt, nq, nd);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float xs[CW];
            load_x<CW>(x + static_cast<uint64_t>(b) * cols + static_cast<uint64_t>(ch) * CW, xs);
            accumulate<WT, SF16, NR, CW>(cq, cd, xs, valid, acc[b]);
        }
    }
}

// One wavefront per NR consecutive rows; NB activation vectors at once.
// Every lane runs the same number of chunk steps S (a chunk index past the
// end of the row is clamped to the last chunk and not accumulated).  Steps
// alternate between two register sets, so a prefetch is never copied; the
// loop runs pairs of prefetching steps and the last one or two steps are
// peeled.
template <uint32_t WT, bool SF16, int NR, int NB>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const float* __restrict__ x, float* __restrict__ y, uint32_t rows,
    uint32_t cols) {
    constexpr int CW = (WT == kQ4) ? 32 : 16;  // weights per 16-byte chunk
    const int lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const uint32_t r0 = wave * NR;
    if (r0 >= rows) return;  // uniform per wave
    const uint32_t nchunks = cols / CW;
    const uint32_t last = nchunks - 1;
    const uint32_t S = (nchunks + 63) / 64;  // steps, the same for every lane
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
    float acc[NB][NR];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[b][r] = 0.f;

    uint4 qa[NR], qb[NR];
    uint32_t da[NR], db[NR];
    const uint32_t c = lane;
    load_chunk<WT, SF16, NR>(qr, dr, d, min(c, last), qa, da);
    uint32_t k = 0;
    for (; k + 2 < S; k += 2) {  // steps k, k+1; both prefetch
        const uint32_t c0 = c + 64 * k, c1 = c0 + 64, c2 = c1 + 64;
        gemv_step<WT, SF16, NR, NB, CW, true>(qr, dr, d, x, cols, c0, true, c1,
                                              qa, da, qb, db, acc);
        gemv_step<WT, SF16, NR, NB, CW, true>(qr, dr, d, x, cols, c1, true, min(c2, last),
                                              qb, db, qa, da, acc);
    }
    const uint32_t c0 = c + 64 * k, c1 = c0 + 64;
    if (k + 1 < S) {  // two steps left: the last chunk index may be past the end
        gemv_step<WT, SF16, NR, NB, CW, true>(qr, dr, d, x, cols, c0, true, min(c1, last),
                                              qa, da, qb, db, acc);
        gemv_step<WT, SF16, NR, NB, CW, false>(qr, dr, d, x, cols, min(c1, last), c1 < nchunks,
                                               0, qb, db, qa, da, acc);
    } else {          // one step left
        gemv_step<WT, SF16, NR, NB, CW, false>(qr, dr, d, x, cols, min(c0, last), c0 < nchunks,
                                               0, qa, da, qb, db, acc);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float s = wave_reduce(acc[b][r]);
            if (lane == 0 && r0 + r < rows)
                y[static_cast<uint64_t>(b) * rows + r0 + r] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// One-shot kernel with integer block dot products.
//
// Activations as digits.  A workgroup first converts the activations, per
// block of 32 consecutive values (the span of one weight scale): with E the
// binary exponent of the block's largest magnitude (amax in [2^(E-1), 2^E)),
// each value becomes the integer X = rne(x * 2^(30-E)), |X| <= 2^30, so x is
// kept to within 2^(E-31) <= amax * 2^-30.  X is split into four signed
// base-256 digits, X = D0 + 256 D1 + 65536 (D2 + 256 D3) with Dk in
// [-128, 127], and each digit plane is stored as packed int8, so that
// v_dot4_i32_i8 multiplies four weight codes by four digits exactly.  A block
// then adds
//     d * 2^(E-30) * (L + 65536 H),   L = T0 + 256 T1,  H = T2 + 256 T3,
//     Tk = sum_j v_j Dk_j,
// to its row, where L and H are exact int32 sums and the blocks are
// accumulated in float32.  Q8_0 quants are used as they are (signed int8); a
// Q4_0 nibble n enters as the unsigned byte n and the -8 offset as the exact
// starting values -8 * sum_j (D0_j + 256 D1_j) and -8 * sum_j (D2_j + 256 D3_j).
// Zero weights give exactly zero; a non-finite activation makes its block's
// scale NaN.
//
// Small activations.  A nonzero value with |X| < 2^9 (below about 2^-21 of
// its block's largest) would keep fewer than 10 significant bits, so it is
// not put in the digits (X = 0 there); a 32-bit mask per chunk marks it, and
// after the digit sums of all its chunks each row adds d * (v_j * x_j) in
// float32 for every marked j, in ascending order, with x_j the activation
// itself.  Every other value keeps |X| >= 2^9, a relative error of at most
// 2^-10, so each output is within about 2^-10 of sum |w| |x| whatever the
// spread of a block's values.  For N(0,1) data about one value in 10^6 is
// small, so a launch almost never takes that pass.
//
// Work split: one wavefront owns NR consecutive rows; lane l reads the 16-byte
// chunks l, l + 64, ... of each row (a Q4_0 chunk is a whole block, a Q8_0
// chunk half a block).  Order of requests at entry:
//   1. the thread's share of the activations (a half or a quarter block),
//   2. every scale, then every quant chunk of the wave's rows (raw buffer
//      loads; a step past the row's end gets an out-of-range offset: zeros,
//      no traffic, and no branch around the load),
// then the digit conversion into LDS, one barrier, and the rows are multiplied
// as their quants arrive (loads complete in issue order).
//
// LDS layout per activation vector, for chunk c = l + 64k:
//   digit piece p (16 bytes = 16 digits of one plane) at ((k*P + p)*64 + l),
//     Q4_0: P = 8, piece 2*plane + half; Q8_0: P = 4, piece = plane;
//   then the block info at (k*64 + l): Q4_0 {-8*sum (D0 + 256 D1),
//   -8*sum (D2 + 256 D3), 2^(E-30), small-value mask} as 16 bytes, Q8_0
//   {2^(E-30), small-value mask} as 8 bytes.
// A wave reading step k touches 64 consecutive 16-byte slots.
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOob = 0xFFFFFFF0u;  // an offset past any buffer's end

// Cache policy of the weight streams (quants and scales): non-temporal.  The
// weights are read once per product, so they are kept from displacing the
// activations and other small data in the L2 and the MALL; measured 4-8%
// faster on every GEMV shape than the default policy.
constexpr int kStream = 2;

// A raw buffer descriptor over [base, base + bytes).  The launchers make
// sure a wave's range stays below 2^32 - 16 bytes (the out-of-range offset),
// so the size is computed in 32 bits: a 64-bit compare here would be done in
// vector registers and make the compiler wait for outstanding loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

template <uint32_t WT>
struct DigitLayout {
    static constexpr int CW = (WT == kQ4) ? 32 : 16;   // weights per 16-byte chunk
    static constexpr int P = (WT == kQ4) ? 8 : 4;      // digit pieces per chunk
    static constexpr int INFO = (WT == kQ4) ? 16 : 8;  // info bytes per chunk
    // bytes of one staged activation vector with S steps of 64 chunks:
    // digit pieces, then the block info per chunk
    static __host__ __device__ uint32_t vector_bytes(uint32_t S) { return S * 64 * (P * 16 + INFO); }
};

__device__ __forceinline__ int dpp_swap_pair_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
}

// Bytes [b0 b1 b2 b3] of four words -> the four planes {b_k of w0..w3}.
__device__ __forceinline__ void transpose4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                           uint32_t (&p)[4]) {
    // v_perm_b32: selector byte s picks byte s of the 64-bit {src0:src1}
    // (0..3 from src1, 4..7 from src0)
    const uint32_t a = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // w0.0 w1.0 w0.1 w1.1
    const uint32_t b = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // w0.2 w1.2 w0.3 w1.3
    const uint32_t c = __builtin_amdgcn_perm(w3, w2, 0x05010400u);  // w2.0 w3.0 w2.1 w3.1
    const uint32_t e = __builtin_amdgcn_perm(w3, w2, 0x07030602u);  // w2.2 w3.2 w2.3 w3.3
    p[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);                 // w0.0 w1.0 w2.0 w3.0
    p[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);                 // w0.1 w1.1 w2.1 w3.1
    p[2] = __builtin_amdgcn_perm(e, b, 0x05040100u);                 // w0.2 w1.2 w2.2 w3.2
    p[3] = __builtin_amdgcn_perm(e, b, 0x07060302u);                 // w0.3 w1.3 w2.3 w3.3
}

// Converts half block j (16 activations in xv; j even = first half) and
// stores its digit pieces and, from the even lane, its block info.  The two
// halves of a block sit in adjacent lanes of one wave, which exchange their
// largest magnitude and digit sums.  `dig` and `info` point at the vector's
// LDS area; h is the half block's index within its vector.  Returns true if
// the half block holds a small value (below).
template <uint32_t WT>
__device__ __forceinline__ bool stage_half(const float4 (&xv)[4], uint32_t h,
                                           int4* __restrict__ dig, void* __restrict__ info) {
    using L = DigitLayout<WT>;
    const float v[16] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w, xv[1].x, xv[1].y, xv[1].z, xv[1].w,
                         xv[2].x, xv[2].y, xv[2].z, xv[2].w, xv[3].x, xv[3].y, xv[3].z, xv[3].w};
    // largest magnitude as an integer maximum of the absolute bit patterns,
    // so that inf and NaN win over every finite value
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, __builtin_bit_cast(uint32_t, v[i]) & 0x7FFFFFFFu);
    m = max(m, static_cast<uint32_t>(dpp_swap_pair_i(static_cast<int>(m))));
    const int E = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, m));
    const float sx = m >= 0x7F800000u ? __builtin_bit_cast(float, 0x7FC00000u)
                                      : __builtin_amdgcn_ldexpf(1.0f, E - 30);
    // X = rne(x * 2^(30-E)) (exact scaling, then a round to integer), biased
    // by 128 in each of its four bytes.  A nonzero value whose X is below
    // 2^9 in magnitude would keep less than 10 significant bits: such a
    // ("small") value is left out of the digits (X = 0 there), marked in the
    // chunk's mask, and its product added in float32 from the activation
    // itself after the digit sums.
    uint32_t u[16];
    uint32_t small = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int X = static_cast<int>(__builtin_rintf(__builtin_amdgcn_ldexpf(v[i], 30 - E)));
        const bool sm = static_cast<uint32_t>(X + 511) < 1023u &&
                        (__builtin_bit_cast(uint32_t, v[i]) << 1) != 0u;
        small |= sm ? (1u << i) : 0u;
        u[i] = sm ? 0x80808080u : static_cast<uint32_t>(X) + 0x80808080u;
    }
    uint32_t pl[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t p[4];
        transpose4(u[4 * g], u[4 * g + 1], u[4 * g + 2], u[4 * g + 3], p);
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) pl[dd][g] = p[dd] ^ 0x80808080u;  // byte + 128 -> signed digit
    }
    if constexpr (WT == kQ4) {
        const uint32_t c = h >> 1, half = h & 1, k = c >> 6, l = c & 63;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
            dig[(k * L::P + 2 * dd + half) * 64 + l] =
                make_int4(pl[dd][0], pl[dd][1], pl[dd][2], pl[dd][3]);
        int sd[4];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
            int a = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) a = __builtin_amdgcn_sdot4(pl[dd][g], 0x01010101, a, false);
            sd[dd] = a + dpp_swap_pair_i(a);
        }
        // the block's mask: element 16 * half + i of the block is bit
        // 16 * half + i
        const uint32_t mine = small << (16 * half);
        const uint32_t both = mine | static_cast<uint32_t>(dpp_swap_pair_i(static_cast<int>(mine)));
        if (half == 0)
            static_cast<int4*>(info)[k * 64 + l] =
                make_int4(-8 * (sd[0] + 256 * sd[1]), -8 * (sd[2] + 256 * sd[3]),
                          __builtin_bit_cast(int, sx), static_cast<int>(both));
    } else {
        const uint32_t c = h, k = c >> 6, l = c & 63;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
            dig[(k * L::P + dd) * 64 + l] = make_int4(pl[dd][0], pl[dd][1], pl[dd][2], pl[dd][3]);
        static_cast<uint2*>(info)[k * 64 + l] = make_uint2(__builtin_bit_cast(uint32_t, sx), small);
    }
    return small != 0;
}

// Reductions over the 8 lanes of an aligned group (xor 1, xor 2 by quad
// permutes, then the other quad of the eight by row_half_mirror).
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true)));
    return max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, true)));
}
__device__ __forceinline__ uint32_t group8_or(uint32_t v) {
    v |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));
    v |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true));
    return v | static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, true));
}
__device__ __forceinline__ int group8_add(int v) {
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
    v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
    return v + __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);
}

// Converts quarter block q (4 activations xv) and stores its digits and,
// from the block's first lane (first two for Q8_0), the block info.  The
// eight quarters of a block sit in an aligned group of 8 lanes of one wave,
// which exchange the block's largest magnitude, digit sums and mask.  `dig`
// and `info` point at the vector's LDS area; q is the quarter's index
// within its vector.  Returns true if the quarter holds a small value
// (below).
template <uint32_t WT>
__device__ __forceinline__ bool stage_quarter(const float4 xv, uint32_t q, int4* __restrict__ dig,
                                              void* __restrict__ info) {
    using L = DigitLayout<WT>;
    const float v[4] = {xv.x, xv.y, xv.z, xv.w};
    // largest magnitude as an integer maximum of the absolute bit patterns,
    // so that inf and NaN win over every finite value
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, __builtin_bit_cast(uint32_t, v[i]) & 0x7FFFFFFFu);
    m = group8_max(m);
    const int E = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, m));
    const float sx = m >= 0x7F800000u ? __builtin_bit_cast(float, 0x7FC00000u)
                                      : __builtin_amdgcn_ldexpf(1.0f, E - 30);
    // X = rne(x * 2^(30-E)) (exact scaling, then a round to integer), biased
    // by 128 in each of its four bytes.  A nonzero value whose X is below
    // 2^9 in magnitude would keep less than 10 significant bits: such a
    // ("small") value is left out of the digits (X = 0 there), marked in the
    // chunk's mask, and its product added in float32 from the activation
    // itself after the digit sums.
    uint32_t u[4];
    uint32_t small = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int X = static_cast<int>(__builtin_rintf(__builtin_amdgcn_ldexpf(v[i], 30 - E)));
        const bool sm = static_cast<uint32_t>(X + 511) < 1023u &&
                        (__builtin_bit_cast(uint32_t, v[i]) << 1) != 0u;
        small |= sm ? (1u << i) : 0u;
        u[i] = sm ? 0x80808080u : static_cast<uint32_t>(X) + 0x80808080u;
    }
    uint32_t pl[4];
    transpose4(u[0], u[1], u[2], u[3], pl);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) pl[dd] ^= 0x80808080u;  // byte + 128 -> signed digit
    // quarter e of block blk: elements 4e .. 4e + 3 of the block, word e % 4
    // of half (Q4_0) or chunk (Q8_0) e / 4; the block's mask has element i
    // at bit i
    const uint32_t e = q & 7, blk = q >> 3;
    const uint32_t mask = group8_or(small << (4 * e));
    if constexpr (WT == kQ4) {
        const uint32_t k = blk >> 6, l = blk & 63, half = e >> 2;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
            reinterpret_cast<uint32_t*>(dig + (k * L::P + 2 * dd + half) * 64 + l)[e & 3] = pl[dd];
        int sd[4];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) sd[dd] = group8_add(__builtin_amdgcn_sdot4(pl[dd], 0x01010101, 0, false));
        // the -8 offset's exact starting values of planes 0 + 1 and 2 + 3
        if (e == 0)
            static_cast<int4*>(info)[k * 64 + l] =
                make_int4(-8 * (sd[0] + 256 * sd[1]), -8 * (sd[2] + 256 * sd[3]),
                          __builtin_bit_cast(int, sx), static_cast<int>(mask));
    } else {
        const uint32_t c = 2 * blk + (e >> 2), k = c >> 6, l = c & 63;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
            reinterpret_cast<uint32_t*>(dig + (k * L::P + dd) * 64 + l)[e & 3] = pl[dd];
        if ((e & 3) == 0)
            static_cast<uint2*>(info)[k * 64 + l] =
                make_uint2(__builtin_bit_cast(uint32_t, sx), (e >> 2) ? mask >> 16 : mask & 0xFFFFu);
    }
    return small != 0;
}

// The small-value mask of chunk slot `is` of a vector's block info.
template <uint32_t WT>
__device__ __forceinline__ uint32_t chunk_mask(const uint8_t* __restrict__ info, uint32_t is) {
    if constexpr (WT == kQ4) return static_cast<uint32_t>(reinterpret_cast<const int4*>(info)[is].w);
    else return reinterpret_cast<const uint2*>(info)[is].y;
}

// Adds the small activations of one step (mask bits, left out of the digit
// sums) to the wave-reduced row sums: sum[r] += d * (v_j * x_j) for each
// small element j of each chunk c of the step, in ascending c and j, with
// x_j read from xs (the activations of the step's first chunk).  mask_l is
// the lane's own chunk's mask (zero past the row).  The walk is
// wave-uniform: the quants and the scale of chunk c are read from lane c
// with readlane.
template <uint32_t WT, bool SF16, int NR, int SMAX>
__device__ __forceinline__ void small_sums(const uint4 (&qv)[NR][SMAX], const uint32_t (&dv)[NR][SMAX],
                                           int k, uint32_t mask_l, const float* __restrict__ xs,
                                           float (&sum)[NR]) {
    constexpr uint32_t CW = DigitLayout<WT>::CW;
    uint64_t chunks = __ballot(mask_l != 0u);
    while (chunks != 0) {
        const uint32_t c = static_cast<uint32_t>(__builtin_ctzll(chunks));
        chunks &= chunks - 1;
        uint32_t mask = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mask_l), c));
        uint32_t qw[NR][4], db[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            qw[r][0] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(qv[r][k].x), c));
            qw[r][1] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(qv[r][k].y), c));
            qw[r][2] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(qv[r][k].z), c));
            qw[r][3] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(qv[r][k].w), c));
            db[r] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dv[r][k]), c));
        }
        while (mask != 0) {
            const uint32_t j = __builtin_ctz(mask);
            mask &= mask - 1;
            const float xj = xs[c * CW + j];
            // element j: Q4_0 nibble of byte j % 16 (high half for j >= 16),
            // Q8_0 byte j
            const uint32_t byte = WT == kQ4 ? (j & 15u) : j;
            const uint32_t sh = 8 * (byte & 3u) + (WT == kQ4 ? 4 * (j >> 4) : 0);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint32_t w = qw[r][byte >> 2];
                const float code = WT == kQ4
                    ? static_cast<float>(static_cast<int>((w >> sh) & 15u) - 8)
                    : static_cast<float>(static_cast<int8_t>((w >> sh) & 0xFFu));
                sum[r] = fmaf(scale_from_bits<SF16>(db[r]), code * xj, sum[r]);
            }
        }
    }
}

// Workgroup-uniform OR of each thread's `mine` (every wave writes its own
// slot of `slots`, read after the barrier that this call performs).
__device__ __forceinline__ bool barrier_any(bool mine, uint32_t* slots, uint32_t waves) {
    const uint32_t wid = threadIdx.x >> 6;
    const bool w = __ballot(mine) != 0;
    if ((threadIdx.x & 63) == 0) slots[wid] = w ? 1u : 0u;
    __syncthreads();
    uint32_t any = 0;
    for (uint32_t i = 0; i < waves; ++i) any |= slots[i];
    return any != 0;
}

// T0 + 256 T1 + 65536 (T2 + 256 T3) in float32, from lo = T0 + 256 T1 and
// hi = T2 + 256 T3 (each exact in int32).
__device__ __forceinline__ float combine_digits(int lo, int hi) {
    return fmaf(static_cast<float>(hi), 65536.f, static_cast<float>(lo));
}

// Digit sums of one Q4_0 chunk (a whole block) with quants w; the -8 offset
// enters as the starting values info.x (planes 0 and 1) and info.y (planes
// 2 and 3).
__device__ __forceinline__ float q4_digit_dot(const uint4 w, const int4 (&pc)[8], const int4 info) {
    uint32_t mask = 0x0F0F0F0Fu;
    asm("" : "+v"(mask));
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
    int t[4] = {info.x, 0, info.y, 0};
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
        const int lo_d[4] = {pc[2 * dd].x, pc[2 * dd].y, pc[2 * dd].z, pc[2 * dd].w};
        const int hi_d[4] = {pc[2 * dd + 1].x, pc[2 * dd + 1].y, pc[2 * dd + 1].z, pc[2 * dd + 1].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t[dd] = __builtin_amdgcn_sdot4(static_cast<int>(q[i] & mask), lo_d[i], t[dd], false);
            t[dd] = __builtin_amdgcn_sdot4(static_cast<int>((q[i] >> 4) & mask), hi_d[i], t[dd], false);
        }
    }
    return combine_digits(t[0] + 256 * t[1], t[2] + 256 * t[3]);
}

// Digit sums of one Q8_0 chunk (half a block) with quants w.
__device__ __forceinline__ float q8_digit_dot(const uint4 w, const int4 (&pc)[4]) {
    const int q[4] = {static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                      static_cast<int>(w.w)};
    int t[4];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
        const int dg[4] = {pc[dd].x, pc[dd].y, pc[dd].z, pc[dd].w};
        int a = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) a = __builtin_amdgcn_sdot4(q[i], dg[i], a, false);
        t[dd] = a;
    }
    return combine_digits(t[0] + 256 * t[1], t[2] + 256 * t[3]);
}

// Adds one chunk of every row (quants qv[r][k], scale bits dv[r][k]) times
// the staged activations of one vector (digit pieces pc, block info at
// slot `is` of `info`) to acc[r], where `valid`.
template <uint32_t WT, bool SF16, int NR, int SMAX>
__device__ __forceinline__ void chunk_rows(const uint4 (&qv)[NR][SMAX], const uint32_t (&dv)[NR][SMAX],
                                           int k, const int4 (&pc)[DigitLayout<WT>::P],
                                           const uint8_t* __restrict__ info, uint32_t is, bool valid,
                                           float (&acc)[NR]) {
    float t[NR];
    float sx;
    if constexpr (WT == kQ4) {
        const int4 in = reinterpret_cast<const int4*>(info)[is];
        sx = __builtin_bit_cast(float, in.z);
#pragma unroll
        for (int r = 0; r < NR; ++r) t[r] = q4_digit_dot(qv[r][k], pc, in);
    } else {
        sx = __builtin_bit_cast(float, reinterpret_cast<const uint2*>(info)[is].x);
#pragma unroll
        for (int r = 0; r < NR; ++r) t[r] = q8_digit_dot(qv[r][k], pc);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float a = fmaf(scale_from_bits<SF16>(dv[r][k]) * sx, t[r], acc[r]);
        acc[r] = valid ? a : acc[r];
    }
}

// Activations per staging thread: a half block (16) when the vectors have
// at least 256 half blocks (a wave's worth for each SIMD), else a quarter
// block (4), so that short vectors are converted by all four SIMDs (the
// quarter form takes more instructions per value).
template <uint32_t WT, int NB, int SMAX>
constexpr int stage_values() {
    return NB * SMAX * 64 * DigitLayout<WT>::CW / 16 >= 256 ? 16 : 4;
}

// Staging parts each thread loads before the quants: enough for
// NB vectors of up to SMAX steps (at most 2; any rest is loaded afterwards).
template <uint32_t WT, int NB, int SMAX, int WAVES>
constexpr int stage_rounds() {
    constexpr int parts = NB * SMAX * 64 * DigitLayout<WT>::CW / stage_values<WT, NB, SMAX>();
    constexpr int r = (parts + WAVES * 64 - 1) / (WAVES * 64);
    constexpr int rmax = stage_values<WT, NB, SMAX>() == 4 ? 4 : 2;
    return r < 1 ? 1 : (r > rmax ? rmax : r);
}

// The one-shot product of workgroup `block` (blockIdx.x of a plain launch,
// or the block's index within its matrix in a grouped launch).
template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, int WAVES>
__device__ __forceinline__ void oneshot_body(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const float* __restrict__ x, float* __restrict__ y, uint32_t rows, uint32_t cols,
    uint32_t block, float4* __restrict__ smem) {
    using L = DigitLayout<WT>;
    constexpr int CW = L::CW;
    constexpr int P = L::P;
    constexpr int THREADS = WAVES * 64;
    constexpr int XR = stage_rounds<WT, NB, SMAX, WAVES>();
    constexpr uint32_t SB = SF16 ? 2 : 4;       // bytes per scale
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index in a scalar register, so that everything derived from
    // it (row range, buffer descriptors) is known to be wave-uniform
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t nchunks = cols / CW;
    const uint32_t S = (nchunks + 63) / 64;     // <= SMAX (host-checked)
    constexpr int SV = stage_values<WT, NB, SMAX>();  // activations per staging part
    const uint32_t nparts = cols / SV;          // staging parts per vector
    const uint32_t nstage = NB * nparts;
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
    const uint32_t dig_bytes = S * P * 64 * 16;     // per vector
    const uint32_t vec_bytes = L::vector_bytes(S);  // digits + info, per vector

    // ---- 1. this thread's activations ----
    const float4* x4 = reinterpret_cast<const float4*>(x);
    float4 xr[XR][SV / 4];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const uint32_t j = tid + i * THREADS;
        if (j < nstage) {
#pragma unroll
            for (int g = 0; g < SV / 4; ++g) xr[i][g] = x4[(SV / 4) * j + g];
        }
    }

    // ---- 2. every scale and quant chunk of this wave's rows ----
    const uint64_t row_bytes = (WT == kQ4) ? (cols >> 1) : cols;
    const uint32_t nblk = cols >> 5;
    const uint32_t row0 = (block * WAVES + wid) * NR;
    const uint32_t wrows = row0 < rows ? min(static_cast<uint32_t>(NR), rows - row0) : 0;
    const uint32_t rb = min(row0, rows - 1);
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(q + static_cast<uint64_t>(rb) * row_bytes, wrows * static_cast<uint32_t>(row_bytes));
    const __amdgpu_buffer_rsrc_t drs =
        make_rsrc(static_cast<const uint8_t*>(d) + static_cast<uint64_t>(rb) * nblk * SB,
                  wrows * nblk * SB);
    uint4 qv[NR][SMAX];
    uint32_t dv[NR][SMAX];
    // the small scale loads first: loads complete in issue order, so each
    // step then waits for its own quants only
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t blk = (WT == kQ4) ? ch : (ch >> 1);
            const uint32_t dofs = ch < nchunks ? (r * nblk + blk) * SB : kOob;
            if constexpr (SF16) dv[r][k] = __builtin_amdgcn_raw_buffer_load_b16(drs, dofs, 0, kStream);
            else dv[r][k] = __builtin_amdgcn_raw_buffer_load_b32(drs, dofs, 0, kStream);
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t qo = ch < nchunks ? r * static_cast<uint32_t>(row_bytes) + 16 * ch : kOob;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qrs, qo, 0, kStream);
            qv[r][k] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }

    // ---- 3. activations -> digits in LDS ----
    bool mysmall = false;
    // (a block's two halves, or eight quarters, are aligned adjacent lanes:
    // THREADS and the parts per vector are multiples of 8, and all of a
    // block's parts are staged or none)
    auto stage = [&](uint32_t j, const float4 (&xv)[SV / 4]) {
        const uint32_t b = j / nparts, pi = j - b * nparts;
        uint8_t* base = lds + b * vec_bytes;
        if constexpr (SV == 16)
            mysmall |= stage_half<WT>(xv, pi, reinterpret_cast<int4*>(base), base + dig_bytes);
        else
            mysmall |= stage_quarter<WT>(xv[0], pi, reinterpret_cast<int4*>(base), base + dig_bytes);
    };
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const uint32_t j = tid + i * THREADS;
        if (j < nstage) stage(j, xr[i]);
    }
    for (uint32_t j = tid + XR * THREADS; j < nstage; j += THREADS) {
        float4 xv[SV / 4];
#pragma unroll
        for (int g = 0; g < SV / 4; ++g) xv[g] = x4[(SV / 4) * j + g];
        stage(j, xv);
    }
    __shared__ uint32_t small_slots[WAVES];
    const bool any_small = barrier_any(mysmall, small_slots, WAVES);
    if (wrows == 0) return;  // uniform per wave, after the barrier

    // ---- 4. multiply ----
    auto multiply = [&](auto small_t) {
        constexpr bool SMALL = decltype(small_t)::value;
        float acc[NB][NR];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[b][r] = 0.f;
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            if (k < static_cast<int>(S)) {
                const bool valid = lane + 64u * k < nchunks;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const uint8_t* base = lds + b * vec_bytes;
                    const int4* dg = reinterpret_cast<const int4*>(base) + k * P * 64 + lane;
                    int4 pc[P];
#pragma unroll
                    for (int p = 0; p < P; ++p) pc[p] = dg[p * 64];
                    chunk_rows<WT, SF16, NR>(qv, dv, k, pc, base + dig_bytes, k * 64 + lane, valid,
                                             acc[b]);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float sum[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) sum[r] = wave_reduce(acc[b][r]);
            // then the small activations, left out of the digits, in
            // ascending order (every quant has arrived: the reads of x here
            // wait for nothing else)
            if constexpr (SMALL) {
                const uint8_t* info = lds + b * vec_bytes + dig_bytes;
#pragma unroll
                for (int k = 0; k < SMAX; ++k) {
                    if (k < static_cast<int>(S)) {
                        const uint32_t mask =
                            lane + 64u * k < nchunks ? chunk_mask<WT>(info, k * 64 + lane) : 0u;
                        small_sums<WT, SF16, NR>(qv, dv, k, mask,
                                                 x + static_cast<uint64_t>(b) * cols + 64u * k * CW, sum);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (lane == 0 && static_cast<uint32_t>(r) < wrows)
                    y[static_cast<uint64_t>(b) * rows + row0 + r] = sum[r];
        }
    };
    if (any_small) multiply(std::true_type{});
    else multiply(std::false_type{});
}

template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_oneshot_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const float* __restrict__ x, float* __restrict__ y, uint32_t rows, uint32_t cols) {
    extern __shared__ float4 smem[];
    oneshot_body<WT, SF16, NR, NB, SMAX, WAVES>(q, d, x, y, rows, cols, blockIdx.x, smem);
}

// The same for one-step rows of a single vector (the shape of a large
// classifier at batch 1), held to six waves per SIMD (at most 80 vector
// registers): measured 1 us faster on the 248320 x 1024 Q8_0 head than the
// five the compiler chooses by itself (eight spill and run slower).
template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(6))) void
gemv_oneshot_kernel_occ6(const uint8_t* __restrict__ q, const void* __restrict__ d,
                         const float* __restrict__ x, float* __restrict__ y, uint32_t rows,
                         uint32_t cols) {
    extern __shared__ float4 smem[];
    oneshot_body<WT, SF16, NR, NB, SMAX, WAVES>(q, d, x, y, rows, cols, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// Streaming kernel for large matrices: one workgroup of 8 waves per compute
// unit (measured 10.4-10.7 us for w1 | w3, 2 x 11008 x 4096 Q4_0, against
// 11.0-11.6 us with 16 waves, 10.8 us with 12 and 12.1 us with 4) converts
// the activations once, then each wave walks over a contiguous range of row
// tiles (NR rows each) of a list of matrices of one storage type, with the
// loads of its next tile in flight while it multiplies the current one (a
// three-deep ring measured slower).  The tile loop is branch-free around the
// loads: a tile past the end gets an empty buffer range, so its loads return
// zeros without memory traffic and the two register sets alternate in
// straight-line code (loads complete in issue order, so each wait covers one
// tile only).
// ---------------------------------------------------------------------------

constexpr int kMaxGroup = 8;
constexpr int kStreamWaves = 8;

struct TileArgs {
    const uint8_t* q[kMaxGroup];
    const void* d[kMaxGroup];
    float* y[kMaxGroup];
    uint32_t rows[kMaxGroup];
    uint32_t first[kMaxGroup + 1];   // first tile of each matrix; first[n] = all tiles
    uint32_t n;
};

template <int NR, int SMAX>
struct TileRegs {
    uint4 q[NR][SMAX];
    uint32_t d[NR][SMAX];
    uint32_t mat, row0, wrows;      // wave-uniform
};

// Requests the scales, then the quants, of tile t (which may be past the end).
template <uint32_t WT, bool SF16, int NR, int SMAX>
__device__ __forceinline__ void load_tile(const TileArgs& g, uint32_t t, uint32_t cols,
                                          uint32_t lane, uint32_t& mat, TileRegs<NR, SMAX>& b) {
    constexpr uint32_t CW = DigitLayout<WT>::CW;
    constexpr uint32_t SB = SF16 ? 2 : 4;
    // matrix of tile t: the number of later matrices that start at or before
    // t, in plain integer arithmetic (first[i] = 2^31 - 1 past the list), so
    // that it stays in scalar registers: neither a loop nor a lane mask here,
    // either of which makes the compiler wait for every outstanding load
    uint32_t m = 0;
#pragma unroll
    for (int i = 1; i <= kMaxGroup; ++i)
        m += 1u + static_cast<uint32_t>(static_cast<int32_t>(t - g.first[i]) >> 31);
    mat = min(m, g.n - 1);
    const bool live = t < g.first[g.n];
    const uint32_t row0 = live ? (t - g.first[mat]) * NR : 0;
    const uint32_t rows = g.rows[mat];
    const uint32_t wrows = live ? min(static_cast<uint32_t>(NR), rows - row0) : 0;
    const uint32_t nchunks = cols / CW;
    const uint64_t row_bytes = (WT == kQ4) ? (cols >> 1) : cols;
    const uint32_t nblk = cols >> 5;
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(g.q[mat] + static_cast<uint64_t>(row0) * row_bytes,
                  wrows * static_cast<uint32_t>(row_bytes));
    const __amdgpu_buffer_rsrc_t drs =
        make_rsrc(static_cast<const uint8_t*>(g.d[mat]) + static_cast<uint64_t>(row0) * nblk * SB,
                  wrows * nblk * SB);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t blk = (WT == kQ4) ? ch : (ch >> 1);
            const uint32_t dofs = ch < nchunks ? (r * nblk + blk) * SB : kOob;
            if constexpr (SF16) b.d[r][k] = __builtin_amdgcn_raw_buffer_load_b16(drs, dofs, 0, kStream);
            else b.d[r][k] = __builtin_amdgcn_raw_buffer_load_b32(drs, dofs, 0, kStream);
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t qo = ch < nchunks ? r * static_cast<uint32_t>(row_bytes) + 16 * ch : kOob;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qrs, qo, 0, kStream);
            b.q[r][k] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
    b.mat = mat;
    b.row0 = row0;
    b.wrows = wrows;
}

// Gated tile t: rows [t * NR/2, t * NR/2 + NR/2) of w1 (g.q[0], g.d[0]) in
// register rows 0 .. NR/2 - 1 and the same rows of w3 (g.q[1], g.d[1]) in
// rows NR/2 .. NR - 1; b.wrows counts the rows of one matrix.
template <uint32_t WT, bool SF16, int NR, int SMAX>
__device__ __forceinline__ void load_tile_gated(const TileArgs& g, uint32_t t, uint32_t cols,
                                                uint32_t lane, TileRegs<NR, SMAX>& b) {
    constexpr int NH = NR / 2;
    constexpr uint32_t CW = DigitLayout<WT>::CW;
    constexpr uint32_t SB = SF16 ? 2 : 4;
    const bool live = t < g.first[1];
    const uint32_t rows = g.rows[0];
    const uint32_t row0 = live ? t * NH : 0;
    const uint32_t wrows = live ? min(static_cast<uint32_t>(NH), rows - row0) : 0;
    const uint32_t nchunks = cols / CW;
    const uint64_t row_bytes = (WT == kQ4) ? (cols >> 1) : cols;
    const uint32_t nblk = cols >> 5;
    __amdgpu_buffer_rsrc_t qrs[2], drs[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        qrs[m] = make_rsrc(g.q[m] + static_cast<uint64_t>(row0) * row_bytes,
                           wrows * static_cast<uint32_t>(row_bytes));
        drs[m] = make_rsrc(static_cast<const uint8_t*>(g.d[m]) + static_cast<uint64_t>(row0) * nblk * SB,
                           wrows * nblk * SB);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t blk = (WT == kQ4) ? ch : (ch >> 1);
            const uint32_t dofs = ch < nchunks ? ((r % NH) * nblk + blk) * SB : kOob;
            if constexpr (SF16) b.d[r][k] = __builtin_amdgcn_raw_buffer_load_b16(drs[r / NH], dofs, 0, kStream);
            else b.d[r][k] = __builtin_amdgcn_raw_buffer_load_b32(drs[r / NH], dofs, 0, kStream);
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t qo = ch < nchunks ? (r % NH) * static_cast<uint32_t>(row_bytes) + 16 * ch : kOob;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qrs[r / NH], qo, 0, kStream);
            b.q[r][k] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
    b.mat = 0;
    b.row0 = row0;
    b.wrows = wrows;
}

// The FFN activations of the .mlb header field `act`: 0 SiLU, a * sigmoid(a);
// 1 GELU with the tanh approximation, a/2 * (1 + tanh(u)) with u =
// sqrt(2/pi) * (a + 0.044715 a^3), evaluated as a / (1 + e^(-2u)) (the same
// function, since 1 + tanh(u) = 2 / (1 + e^(-2u))): 1 + tanh(u) would lose
// all relative precision to cancellation for negative a.
__device__ __forceinline__ float ffn_act(float a, uint32_t act) {
    if (act == 0) return a / (1.0f + expf(-a));
    const float u = 0.7978845608028654f * (a + 0.044715f * a * a * a);
    return a / (1.0f + expf(-2.0f * u));
}

// Multiplies a loaded tile by the NB staged vectors and stores its rows.
// Gated (GATED = true): stores act(w1 row) * (w3 row) for each row pair.
template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, bool GATED, bool SMALL>
__device__ __forceinline__ void compute_tile(const TileArgs& g, const TileRegs<NR, SMAX>& b,
                                             const uint8_t* __restrict__ lds,
                                             const float* __restrict__ x, uint32_t cols,
                                             uint32_t S, uint32_t lane, uint32_t act,
                                             uint32_t steps_small) {
    using L = DigitLayout<WT>;
    constexpr int P = L::P;
    const uint32_t nchunks = cols / L::CW;
    const uint32_t dig_bytes = S * P * 64 * 16;
    const uint32_t vec_bytes = L::vector_bytes(S);
    float acc[NB][NR];
#pragma unroll
    for (int v = 0; v < NB; ++v)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[v][r] = 0.f;
#pragma unroll
    for (int k = 0; k < SMAX; ++k) {
        if (k < static_cast<int>(S)) {
            const bool valid = lane + 64u * k < nchunks;
#pragma unroll
            for (int v = 0; v < NB; ++v) {
                const uint8_t* base = lds + v * vec_bytes;
                const int4* dg = reinterpret_cast<const int4*>(base) + k * P * 64 + lane;
                int4 pc[P];
#pragma unroll
                for (int p = 0; p < P; ++p) pc[p] = dg[p * 64];
                chunk_rows<WT, SF16, NR>(b.q, b.d, k, pc, base + dig_bytes, k * 64 + lane, valid,
                                         acc[v]);
            }
        }
    }
    // the wave-reduced row sums, then the small activations (the one-shot
    // kernel's order, so that both give the same sums) on the steps that
    // hold any (bit v * SMAX + k of steps_small), then the stores
    const uint32_t rows = g.rows[b.mat];
    float* y = g.y[b.mat];
#pragma unroll
    for (int v = 0; v < NB; ++v) {
        float sum[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) sum[r] = wave_reduce(acc[v][r]);
        if constexpr (SMALL) {
            const uint8_t* info = lds + v * vec_bytes + dig_bytes;
#pragma unroll
            for (int k = 0; k < SMAX; ++k) {
                if ((steps_small >> (v * SMAX + k)) & 1u) {
                    const uint32_t mask =
                        lane + 64u * k < nchunks ? chunk_mask<WT>(info, k * 64 + lane) : 0u;
                    small_sums<WT, SF16, NR>(b.q, b.d, k, mask,
                                             x + static_cast<uint64_t>(v) * cols + 64u * k * L::CW, sum);
                }
            }
        }
        if constexpr (GATED) {
            constexpr int NH = NR / 2;
#pragma unroll
            for (int r = 0; r < NH; ++r)
                if (lane == 0 && static_cast<uint32_t>(r) < b.wrows)
                    y[static_cast<uint64_t>(v) * rows + b.row0 + r] = ffn_act(sum[r], act) * sum[r + NH];
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (lane == 0 && static_cast<uint32_t>(r) < b.wrows)
                    y[static_cast<uint64_t>(v) * rows + b.row0 + r] = sum[r];
        }
    }
}

template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, bool GATED = false>
__global__ __launch_bounds__(kStreamWaves * 64) void gemv_stream_kernel(
    TileArgs g, const float* __restrict__ x, uint32_t cols, uint32_t per_wg, uint32_t act) {
    extern __shared__ float4 smem[];
    using L = DigitLayout<WT>;
    constexpr int THREADS = kStreamWaves * 64;
    constexpr int XR = stage_rounds<WT, NB, SMAX, kStreamWaves>();
    const int tid = threadIdx.x;
    const uint32_t lane = tid & 63;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t S = (cols / L::CW + 63) / 64;
    constexpr int SV = stage_values<WT, NB, SMAX>();
    const uint32_t nparts = cols / SV;
    const uint32_t nstage = NB * nparts;
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
    const uint32_t dig_bytes = S * L::P * 64 * 16;
    const uint32_t vec_bytes = L::vector_bytes(S);
    // tiles of this wave: t0, t0 + step, ... below `end`; per_wg = 0 spreads
    // the tiles over the whole grid (t0 = global wave, step = all waves),
    // otherwise workgroup b owns tiles [b * per_wg, (b + 1) * per_wg)
    const uint32_t total = g.first[g.n];
    uint32_t t, step, end;
    if (per_wg == 0) {
        t = blockIdx.x * kStreamWaves + wid;
        step = gridDim.x * kStreamWaves;
        end = total;
    } else {
        t = blockIdx.x * per_wg + wid;
        step = kStreamWaves;
        end = min(total, (blockIdx.x + 1) * per_wg);
    }

    // activations first, then the first tiles
    const float4* x4 = reinterpret_cast<const float4*>(x);
    float4 xr[XR][SV / 4];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const uint32_t j = tid + i * THREADS;
        if (j < nstage) {
#pragma unroll
            for (int g = 0; g < SV / 4; ++g) xr[i][g] = x4[(SV / 4) * j + g];
        }
    }
    uint32_t mat = 0;
    // tiles at or past `end` load nothing
    auto tile = [&](uint32_t u) { return u < end ? u : 0xFFFFFFFEu; };
    TileRegs<NR, SMAX> ra, rb;
    auto load_any = [&](uint32_t u, TileRegs<NR, SMAX>& regs) {
        if constexpr (GATED) load_tile_gated<WT, SF16, NR, SMAX>(g, u, cols, lane, regs);
        else load_tile<WT, SF16, NR, SMAX>(g, u, cols, lane, mat, regs);
    };
    load_any(tile(t), ra);

    bool mysmall = false;
    auto stage = [&](uint32_t j, const float4 (&xv)[SV / 4]) {
        const uint32_t v = j / nparts, pi = j - v * nparts;
        uint8_t* base = lds + v * vec_bytes;
        if constexpr (SV == 16)
            mysmall |= stage_half<WT>(xv, pi, reinterpret_cast<int4*>(base), base + dig_bytes);
        else
            mysmall |= stage_quarter<WT>(xv[0], pi, reinterpret_cast<int4*>(base), base + dig_bytes);
    };
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const uint32_t j = tid + i * THREADS;
        if (j < nstage) stage(j, xr[i]);
    }
    for (uint32_t j = tid + XR * THREADS; j < nstage; j += THREADS) {
        float4 xv[SV / 4];
#pragma unroll
        for (int g = 0; g < SV / 4; ++g) xv[g] = x4[(SV / 4) * j + g];
        stage(j, xv);
    }
    __shared__ uint32_t small_slots[kStreamWaves];
    const bool any_small = barrier_any(mysmall, small_slots, kStreamWaves);
    // bit v * SMAX + k: step k of vector v holds a small activation (the
    // same for every tile, so found once)
    static_assert(NB * SMAX <= 32, "one bit per vector and step");
    uint32_t steps_small = 0;
    if (any_small) {
#pragma unroll
        for (int v = 0; v < NB; ++v)
#pragma unroll
            for (int k = 0; k < SMAX; ++k) {
                const bool has = k < static_cast<int>(S) && lane + 64u * k < cols / L::CW &&
                                 chunk_mask<WT>(lds + v * vec_bytes + dig_bytes, k * 64 + lane) != 0u;
                steps_small |= __ballot(has) != 0 ? (1u << (v * SMAX + k)) : 0u;
            }
    }

    // two register sets: the next tile's loads are in flight (the loop
    // without the small-activation pass unless a staged value is small)
    auto run = [&](auto small_t) {
        constexpr bool W = decltype(small_t)::value;
        while (t < end) {
            load_any(tile(t + step), rb);
            compute_tile<WT, SF16, NR, NB, SMAX, GATED, W>(g, ra, lds, x, cols, S, lane, act, steps_small);
            t += step;
            if (t >= end) break;
            load_any(tile(t + step), ra);
            compute_tile<WT, SF16, NR, NB, SMAX, GATED, W>(g, rb, lds, x, cols, S, lane, act, steps_small);
            t += step;
        }
    };
    if (any_small) run(std::true_type{});
    else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// Grouped launch: several matrices with the same number of columns multiply
// the same activations in one launch (a decode layer's wq | wk | wv, or
// w1 | w3).  Workgroups [first[i], first[i+1]) serve matrix i with the
// one-shot body of its own storage type, NR rows per wave.  One launch
// instead of several saves each extra launch's fixed start-up and drain.
// ---------------------------------------------------------------------------

struct GroupArgs {
    const uint8_t* q[kMaxGroup];
    const void* d[kMaxGroup];
    float* y[kMaxGroup];
    uint32_t rows[kMaxGroup];
    uint32_t kind[kMaxGroup];        // 2 * (wtype == Q8_0) + scale_f16
    uint32_t first[kMaxGroup + 1];   // first workgroup of each matrix
    uint32_t n;
};

// Held to six waves per SIMD (at most 80 vector registers; the compiler
// would take more for the four bodies and fit five): a decode layer's
// wq | wk | wv group measured 6.3 -> 5.9 us.
template <int NR, int NB, int SMAX4, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(6))) void gemv_group_kernel(GroupArgs g,
                                                                 const float* __restrict__ x,
                                                                 uint32_t cols) {
    extern __shared__ float4 smem[];
    // the matrix of this workgroup (uniform; a short scalar search)
    uint32_t i = 0;
    while (i + 1 < g.n && blockIdx.x >= g.first[i + 1]) ++i;
    const uint32_t blk = blockIdx.x - g.first[i];
    switch (g.kind[i]) {
        case 0: oneshot_body<kQ4, false, NR, NB, SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
        case 1: oneshot_body<kQ4, true, NR, NB, SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
        case 2: oneshot_body<kQ8, false, NR, NB, 2 * SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
        default: oneshot_body<kQ8, true, NR, NB, 2 * SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
    }
}

template <uint32_t WT, bool SF16, int NR, int NB>
hipError_t gemv_launch(const MatView& m, const float* x, float* y, hipStream_t s) {
    const uint32_t waves = (m.rows + NR - 1) / NR;
    const uint32_t blocks = (waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((gemv_kernel<WT, SF16, NR, NB>), dim3(blocks), dim3(256), 0, s,
                       m.q, m.d, x, y, m.rows, m.cols);
    return hipGetLastError();
}

template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, int WAVES>
hipError_t gemv_oneshot_launch(const MatView& m, const float* x, float* y, size_t lds,
                               hipStream_t s) {
    const uint32_t waves = (m.rows + NR - 1) / NR;
    const uint32_t blocks = (waves + WAVES - 1) / WAVES;
    if constexpr (NR == 4 && SMAX == 1 && NB == 1)
        hipLaunchKernelGGL((gemv_oneshot_kernel_occ6<WT, SF16, NR, NB, SMAX, WAVES>), dim3(blocks),
                           dim3(WAVES * 64), lds, s, m.q, m.d, x, y, m.rows, m.cols);
    else
        hipLaunchKernelGGL((gemv_oneshot_kernel<WT, SF16, NR, NB, SMAX, WAVES>), dim3(blocks),
                           dim3(WAVES * 64), lds, s, m.q, m.d, x, y, m.rows, m.cols);
    return hipGetLastError();
}

// The one-shot kernel's limits: at most 16 steps of 64 chunks per row, the
// staged activations in at most this much LDS, and a wave's rows within a
// 32-bit buffer range.
constexpr uint64_t kOneshotLds = 72 * 1024;
constexpr uint32_t kOneshotSteps = 16;

template <uint32_t WT>
uint64_t gemv_lds_bytes(uint32_t cols, uint32_t nb) {
    const uint32_t S = (cols / DigitLayout<WT>::CW + 63) / 64;
    return static_cast<uint64_t>(nb) * DigitLayout<WT>::vector_bytes(S);
}

template <uint32_t WT>
bool oneshot_fits(uint32_t cols, uint32_t nb, uint32_t nr) {
    const uint32_t S = (cols / DigitLayout<WT>::CW + 63) / 64;
    const uint64_t row_bytes = (WT == kQ4) ? cols / 2 : cols;
    return S <= kOneshotSteps && gemv_lds_bytes<WT>(cols, nb) <= kOneshotLds &&
           nr * row_bytes < 0xFFFFFFF0ull;
}

// Vectors per pass: the largest of 8, 4, 2, 1 that is left and whose staged
// activations fit the one-shot kernel's LDS.
template <uint32_t WT>
uint32_t pass_vectors(uint32_t cols, uint32_t left) {
    uint32_t nb = left >= 8 ? 8 : left >= 4 ? 4 : left >= 2 ? 2 : 1;
    while (nb > 1 && gemv_lds_bytes<WT>(cols, nb) > kOneshotLds) nb /= 2;
    return nb;
}

// Streaming launch over the matrices ms[0..n) (one storage type, one scale
// type, the same cols), NR rows per tile, one workgroup per compute unit.
template <uint32_t WT, bool SF16, int NR, int NB, int SMAX>
hipError_t stream_launch(const MatView* ms, uint32_t n, const float* x, float* const* ys,
                         uint32_t done, hipStream_t s) {
    TileArgs g{};
    g.n = n;
    uint32_t tiles = 0;
    for (uint32_t i = 0; i < n; ++i) {
        g.q[i] = ms[i].q;
        g.d[i] = ms[i].d;
        g.y[i] = ys[i] + static_cast<uint64_t>(done) * ms[i].rows;
        g.rows[i] = ms[i].rows;
        g.first[i] = tiles;
        tiles += (ms[i].rows + NR - 1) / NR;
    }
    g.first[n] = tiles;
    for (uint32_t i = n + 1; i <= static_cast<uint32_t>(kMaxGroup); ++i) g.first[i] = 0x7FFFFFFFu;
    const uint32_t cols = ms[0].cols;
    const uint32_t want = (tiles + kStreamWaves - 1) / kStreamWaves;
    const uint32_t cap = 256;
    const uint32_t blocks = want < cap ? want : cap;
    // contiguous tile ranges per workgroup
    const uint32_t per_wg = (tiles + blocks - 1) / blocks;
    const size_t lds = static_cast<size_t>(gemv_lds_bytes<WT>(cols, NB));
    const float* xp = x + static_cast<uint64_t>(done) * cols;
    hipLaunchKernelGGL((gemv_stream_kernel<WT, SF16, NR, NB, SMAX>), dim3(blocks),
                       dim3(kStreamWaves * 64), lds, s, g, xp, cols, per_wg, 0u);
    return hipGetLastError();
}

// Rows per tile of the streaming kernel: 4, 2, 1 for 1, 2, 3..4 steps per
// row (two tiles of quants in flight stay at <= 8 loads per lane); 0 when
// the rows need more steps.
template <uint32_t WT>
uint32_t stream_rows(uint32_t cols) {
    const uint32_t S = (cols / DigitLayout<WT>::CW + 63) / 64;
    return S == 1 ? 4 : S == 2 ? 2 : S <= 4 ? 1 : 0;
}

// Streaming pays for rows of two steps (a Q4_0 row of 4096 weights, say)
// once the tiles outnumber the resident waves (4096) by a margin; with one
// step per row the one-shot kernel's many small workgroups read faster.
template <uint32_t WT>
bool use_stream(const MatView* ms, uint32_t n) {
    const uint32_t nr = stream_rows<WT>(ms[0].cols);
    if (nr != 2) return false;
    uint64_t tiles = 0;
    for (uint32_t i = 0; i < n; ++i) tiles += (ms[i].rows + nr - 1) / nr;
    return tiles >= 6144;
}

// One streaming launch for a single activation vector (the decode case).
template <uint32_t WT, bool SF16>
hipError_t stream_pass(const MatView* ms, uint32_t n, const float* x, float* const* ys,
                       hipStream_t s) {
    switch (stream_rows<WT>(ms[0].cols)) {
        case 4: return stream_launch<WT, SF16, 4, 1, 1>(ms, n, x, ys, 0, s);
        case 2: return stream_launch<WT, SF16, 2, 1, 2>(ms, n, x, ys, 0, s);
        default: return stream_launch<WT, SF16, 1, 1, 4>(ms, n, x, ys, 0, s);
    }
}

// Launch shape: S = steps per row (64 chunks each).  Rows per wave NR: up to
// 4 for S = 1 and 2 for S = 2 (a wave's quant loads stay <= 4 per lane), 1
// beyond, and never so many that fewer than 2048 waves (8 per compute unit)
// remain.  Four waves per workgroup share one LDS copy of the activations
// for one-step rows (the LM head 248320 x 1024 Q8_0: 40.2 -> 39.0 us against
// eight) and for fewer than 4096 rows of two to four steps (1024 x 4096:
// 2.49 -> 2.39 us), eight for other rows of up to four steps, sixteen for
// rows of more than four steps (fewer copies of a wide vector) and for 4096
// to 8192 rows of two to four steps, which then take one row per wave.
// Measured: Q4_0 4096 x 4096 3.77 -> 3.62 us, Q4_0 4096 x 8192 6.1 -> 5.6
// us, Q8_0 4096 x 4096 4.77 -> 4.69 us; but 11008 x 4096 Q4_0 7.0 us against
// 6.6 us with two rows per wave in eight-wave groups, 1024 x 4096 slower too,
// and one-step rows slower in sixteen-wave groups.  For Q8_0 4096 x 11008
// (eleven steps), eight-wave groups (12.2 against 11.3 us) and two rows per
// wave (11.8 us) were slower.
template <uint32_t WT, bool SF16, int NB>
hipError_t gemv_pass(const MatView& m, const float* x, float* y, hipStream_t s) {
    constexpr uint32_t CW = DigitLayout<WT>::CW;
    const uint32_t S = (m.cols / CW + 63) / 64;
    uint32_t nr = S == 1 ? 4 : S == 2 ? 2 : 1;
    while (nr > 1 && m.rows / nr < 2048) nr /= 2;
    // rows of two to four steps, 4096 to 8192 of them: one row per wave in
    // sixteen-wave groups (one or two groups per compute unit)
    const bool wide = S >= 2 && S <= 4 && m.rows >= 16 * 256 && m.rows <= 2 * 16 * 256;
    if (wide) nr = 1;
    if (oneshot_fits<WT>(m.cols, NB, nr)) {
        const size_t l = static_cast<size_t>(gemv_lds_bytes<WT>(m.cols, NB));
#define QMV_ONESHOT(NR_, SMAX_, W_) \
    if (nr == NR_ && S <= SMAX_) return gemv_oneshot_launch<WT, SF16, NR_, NB, SMAX_, W_>(m, x, y, l, s);
        QMV_ONESHOT(4, 1, 4)
        QMV_ONESHOT(2, 1, 4)
        QMV_ONESHOT(2, 2, 8)
        QMV_ONESHOT(1, 1, 4)
        if (wide) {
            QMV_ONESHOT(1, 2, 16)
            QMV_ONESHOT(1, 4, 16)
        }
        if (m.rows < 16 * 256) {  // fewer rows: smaller groups spread them over more compute units
            QMV_ONESHOT(1, 2, 4)
            QMV_ONESHOT(1, 4, 4)
        }
        QMV_ONESHOT(1, 2, 8)
        QMV_ONESHOT(1, 4, 8)
        QMV_ONESHOT(1, 8, 16)
        QMV_ONESHOT(1, 12, 16)
        QMV_ONESHOT(1, 16, 16)
#undef QMV_ONESHOT
    }
    constexpr uint32_t kWavesWanted = 256 * 8;
    if (m.rows >= 4 * kWavesWanted) return gemv_launch<WT, SF16, 4, NB>(m, x, y, s);
    if (m.rows >= 2 * kWavesWanted) return gemv_launch<WT, SF16, 2, NB>(m, x, y, s);
    return gemv_launch<WT, SF16, 1, NB>(m, x, y, s);
}

template <uint32_t WT, bool SF16>
hipError_t gemv_batched(const MatView& m, const float* x, float* y,
                        uint32_t batch, hipStream_t s) {
    if (batch == 1 && use_stream<WT>(&m, 1)) return stream_pass<WT, SF16>(&m, 1, x, &y, s);
    uint32_t done = 0;
    while (done < batch) {
        const float* xp = x + static_cast<uint64_t>(done) * m.cols;
        float* yp = y + static_cast<uint64_t>(done) * m.rows;
        const uint32_t nb = pass_vectors<WT>(m.cols, batch - done);
        hipError_t e;
        if (nb == 8) e = gemv_pass<WT, SF16, 8>(m, xp, yp, s);
        else if (nb == 4) e = gemv_pass<WT, SF16, 4>(m, xp, yp, s);
        else if (nb == 2) e = gemv_pass<WT, SF16, 2>(m, xp, yp, s);
        else e = gemv_pass<WT, SF16, 1>(m, xp, yp, s);
        if (e != hipSuccess) return e;
        done += nb;
    }
    return hipSuccess;
}

// Gated launch over row pairs of w1 | w3 (one storage and scale type): NR/2
// rows of each per tile, NB activation vectors, h = act(w1 x) * (w3 x).
template <uint32_t WT, bool SF16, int NR, int NB, int SMAX>
hipError_t gated_launch(const MatView& w1, const MatView& w3, uint32_t act, const float* x,
                        float* h, uint32_t done, hipStream_t s) {
    TileArgs g{};
    g.n = 1;
    g.q[0] = w1.q;
    g.d[0] = w1.d;
    g.q[1] = w3.q;
    g.d[1] = w3.d;
    g.y[0] = h + static_cast<uint64_t>(done) * w1.rows;
    g.rows[0] = w1.rows;
    const uint32_t tiles = (w1.rows + NR / 2 - 1) / (NR / 2);
    g.first[0] = 0;
    g.first[1] = tiles;
    for (uint32_t i = 2; i <= static_cast<uint32_t>(kMaxGroup); ++i) g.first[i] = 0x7FFFFFFFu;
    const uint32_t cols = w1.cols;
    const uint32_t want = (tiles + kStreamWaves - 1) / kStreamWaves;
    const uint32_t blocks = want < 256 ? want : 256;
    const uint32_t per_wg = (tiles + blocks - 1) / blocks;
    const size_t lds = static_cast<size_t>(gemv_lds_bytes<WT>(cols, NB));
    const float* xp = x + static_cast<uint64_t>(done) * cols;
    hipLaunchKernelGGL((gemv_stream_kernel<WT, SF16, NR, NB, SMAX, true>), dim3(blocks),
                       dim3(kStreamWaves * 64), lds, s, g, xp, cols, per_wg, act);
    return hipGetLastError();
}

template <uint32_t WT, bool SF16, int NB>
hipError_t gated_pass(const MatView& w1, const MatView& w3, uint32_t act, const float* x, float* h,
                      uint32_t done, hipStream_t s) {
    const uint32_t S = (w1.cols / DigitLayout<WT>::CW + 63) / 64;
    if (S == 1) return gated_launch<WT, SF16, 4, NB, 1>(w1, w3, act, x, h, done, s);
    if (S == 2) return gated_launch<WT, SF16, 2, NB, 2>(w1, w3, act, x, h, done, s);
    // rows of 3 or 4 steps: one vector per pass (more would spill registers)
    if constexpr (NB == 1) return gated_launch<WT, SF16, 2, 1, 4>(w1, w3, act, x, h, done, s);
    return hipErrorNotSupported;
}

// Vectors per gated pass: 4, 2 or 1, as many as are left and fit 64 KiB of
// LDS; 1 for rows of more than two steps.
template <uint32_t WT>
uint32_t gated_vectors(uint32_t cols, uint32_t left) {
    if ((cols / DigitLayout<WT>::CW + 63) / 64 > 2) return 1;
    uint32_t nb = left >= 4 ? 4 : left >= 2 ? 2 : 1;
    while (nb > 1 && gemv_lds_bytes<WT>(cols, nb) > kOneshotLds) nb /= 2;
    return nb;
}

template <uint32_t WT, bool SF16>
hipError_t gated_batched(const MatView& w1, const MatView& w3, uint32_t act, const float* x,
                         float* h, uint32_t batch, hipStream_t s) {
    uint32_t done = 0;
    while (done < batch) {
        const uint32_t nb = gated_vectors<WT>(w1.cols, batch - done);
        hipError_t e;
        if (nb == 4) e = gated_pass<WT, SF16, 4>(w1, w3, act, x, h, done, s);
        else if (nb == 2) e = gated_pass<WT, SF16, 2>(w1, w3, act, x, h, done, s);
        else e = gated_pass<WT, SF16, 1>(w1, w3, act, x, h, done, s);
        if (e != hipSuccess) return e;
        done += nb;
    }
    return hipSuccess;
}

template <int NR, int NB, int SMAX4>
hipError_t group_launch(const GroupArgs& g, uint32_t blocks, size_t lds, const float* xp,
                        uint32_t cols, hipStream_t s) {
    constexpr int WAVES = 8;
    hipLaunchKernelGGL((gemv_group_kernel<NR, NB, SMAX4, WAVES>), dim3(blocks), dim3(WAVES * 64),
                       lds, s, g, xp, cols);
    return hipGetLastError();
}

// Rows per wave of a grouped launch: 1 (measured faster than 2 for a mixed
// wq | wk | wv group); nr = 2 is built for cols <= 4096.
template <int NB>
hipError_t group_pass(const MatView* ms, uint32_t n, const float* x, float* const* ys,
                      uint32_t done, uint32_t nr, hipStream_t s) {
    constexpr int WAVES = 8;
    const uint32_t cols = ms[0].cols;
    const uint32_t S4 = (cols / 32 + 63) / 64;
    GroupArgs g{};
    g.n = n;
    uint32_t blocks = 0;
    uint64_t lds = 0;
    for (uint32_t i = 0; i < n; ++i) {
        g.q[i] = ms[i].q;
        g.d[i] = ms[i].d;
        g.y[i] = ys[i] + static_cast<uint64_t>(done) * ms[i].rows;
        g.rows[i] = ms[i].rows;
        g.kind[i] = 2 * (ms[i].wtype == kQ8) + ms[i].scale_f16;
        g.first[i] = blocks;
        blocks += (ms[i].rows + WAVES * nr - 1) / (WAVES * nr);
        const uint64_t b = ms[i].wtype == kQ4 ? gemv_lds_bytes<kQ4>(cols, NB) : gemv_lds_bytes<kQ8>(cols, NB);
        lds = b > lds ? b : lds;
    }
    g.first[n] = blocks;
    const float* xp = x + static_cast<uint64_t>(done) * cols;
    const size_t l = static_cast<size_t>(lds);
    if (nr == 2 && S4 <= 2) return group_launch<2, NB, 2>(g, blocks, l, xp, cols, s);
    if (S4 <= 1) return group_launch<1, NB, 1>(g, blocks, l, xp, cols, s);
    if (S4 <= 2) return group_launch<1, NB, 2>(g, blocks, l, xp, cols, s);
    if (S4 <= 4) return group_launch<1, NB, 4>(g, blocks, l, xp, cols, s);
    return group_launch<1, NB, 8>(g, blocks, l, xp, cols, s);
}

}  // namespace

// Batches up to this size run the vector kernel; larger ones the matrix
// cores (each vector pass re-reads the whole matrix).
constexpr uint32_t kGemvMaxBatch = 8;

hipError_t launch_gemv_group(const MatView* ms, uint32_t n, const float* x, float* const* ys,
                             uint32_t batch, void* workspace, hipStream_t s) {
    const uint32_t cols = ms[0].cols;
    const uint32_t S4 = (cols / 32 + 63) / 64;
    const bool fits = n <= static_cast<uint32_t>(kMaxGroup) && batch <= kGemvMaxBatch && S4 <= 8 &&
                      oneshot_fits<kQ4>(cols, 1, 2) && oneshot_fits<kQ8>(cols, 1, 2);
    bool same = true;
    for (uint32_t i = 1; i < n; ++i)
        same = same && ms[i].wtype == ms[0].wtype && ms[i].scale_f16 == ms[0].scale_f16;
    if (n <= static_cast<uint32_t>(kMaxGroup) && batch == 1 && same) {
        if (ms[0].wtype == kQ4 && use_stream<kQ4>(ms, n))
            return ms[0].scale_f16 ? stream_pass<kQ4, true>(ms, n, x, ys, s)
                                   : stream_pass<kQ4, false>(ms, n, x, ys, s);
        if (ms[0].wtype == kQ8 && use_stream<kQ8>(ms, n))
            return ms[0].scale_f16 ? stream_pass<kQ8, true>(ms, n, x, ys, s)
                                   : stream_pass<kQ8, false>(ms, n, x, ys, s);
    }
    if (!fits) {  // one launch per matrix
        for (uint32_t i = 0; i < n; ++i) {
            const hipError_t e = launch_gemv(ms[i], x, ys[i], batch, workspace, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const uint32_t nr = 1;
    uint32_t done = 0;
    while (done < batch) {
        const uint32_t nb = pass_vectors<kQ4>(cols, batch - done);
        hipError_t e;
        if (nb == 8) e = group_pass<8>(ms, n, x, ys, done, nr, s);
        else if (nb == 4) e = group_pass<4>(ms, n, x, ys, done, nr, s);
        else if (nb == 2) e = group_pass<2>(ms, n, x, ys, done, nr, s);
        else e = group_pass<1>(ms, n, x, ys, done, nr, s);
        if (e != hipSuccess) return e;
        done += nb;
    }
    return hipSuccess;
}

bool gemv_gated_fits(const MatView& w1, const MatView& w3) {
    if (w1.wtype != w3.wtype || w1.scale_f16 != w3.scale_f16 || w1.rows != w3.rows ||
        w1.cols != w3.cols)
        return false;
    const uint32_t cw = w1.wtype == kQ4 ? 32 : 16;
    const uint64_t row_bytes = w1.wtype == kQ4 ? w1.cols / 2 : w1.cols;
    return (w1.cols / cw + 63) / 64 <= 4 && 2 * row_bytes < 0xFFFFFFF0ull;
}

hipError_t launch_gemv_gated(const MatView& w1, const MatView& w3, uint32_t act, const float* x,
                             float* h, uint32_t batch, hipStream_t s) {
    if (!gemv_gated_fits(w1, w3) || act > 1) return hipErrorNotSupported;
    if (w1.wtype == kQ4)
        return w1.scale_f16 ? gated_batched<kQ4, true>(w1, w3, act, x, h, batch, s)
                            : gated_batched<kQ4, false>(w1, w3, act, x, h, batch, s);
    return w1.scale_f16 ? gated_batched<kQ8, true>(w1, w3, act, x, h, batch, s)
                        : gated_batched<kQ8, false>(w1, w3, act, x, h, batch, s);
}

size_t gemv_workspace_bytes(const MatView& m, uint32_t batch) {
    if (batch <= kGemvMaxBatch || gemv_mfma_fits(m)) return 0;
    return gemm_workspace_bytes(m, batch, true);
}

hipError_t launch_gemv(const MatView& m, const float* x, float* y,
                       uint32_t batch, void* workspace, hipStream_t s) {
    if (batch > kGemvMaxBatch) {
        if (gemv_mfma_fits(m)) return launch_gemv_mfma(m, x, y, batch, s);
        return launch_gemm(m, x, true, y, batch, workspace, s);
    }
    if (m.wtype == kQ4) {
        return m.scale_f16 ? gemv_batched<kQ4, true>(m, x, y, batch, s)
                           : gemv_batched<kQ4, false>(m, x, y, batch, s);
    }
    return m.scale_f16 ? gemv_batched<kQ8, true>(m, x, y, batch, s)
                       : gemv_batched<kQ8, false>(m, x, y, batch, s);
}

}  // namespace qmv
