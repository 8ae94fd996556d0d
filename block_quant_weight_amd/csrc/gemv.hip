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
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace qmv {
namespace {

constexpr int kWaves = 4;  // wavefronts per workgroup

// Launch-shape override from the environment, for tuning sweeps (the default
// applies when the variable is unset or not a positive number).
uint32_t tune_knob(const char* name, uint32_t dflt) {
    const char* v = getenv(name);
    if (v == nullptr) return dflt;
    const long n = strtol(v, nullptr, 10);
    return n > 0 ? static_cast<uint32_t>(n) : dflt;
}

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
// One-shot kernel: every load of a wave is requested at entry.
//
// A wave owns NR rows and reads all S <= SMAX steps of each (lane l takes
// chunks l, l + 64, ...).  Order of requests:
//   1. the thread's first activation chunk (for the workgroup's LDS copy),
//   2. every quant chunk and scale of the wave's rows (raw buffer loads; a
//      step past the row's end gets an out-of-range offset: zeros, no
//      traffic, and no branch around the load),
//   3. the rest of the activation chunks, if any.
// Then the activations go to LDS in a lane-permuted order (float4 g of
// chunk l + 64k at ((k*G4 + g)*64 + l), so a wave reading step k touches 64
// consecutive 16-byte slots), each with its chunk sum computed in the dot
// product's element order; one barrier; then the rows are multiplied as
// their quants arrive (loads complete in issue order).
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOob = 0xFFFFFFF0u;  // an offset past any buffer's end

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(n), 0x00020000);
}

template <int CW>
__device__ __forceinline__ void lds_read_x(const float4* __restrict__ xl, uint32_t k, int lane,
                                           float (&xs)[CW]) {
    constexpr int G4 = CW / 4;
#pragma unroll
    for (int g = 0; g < G4; ++g) {
        const float4 t = xl[(k * G4 + g) * 64 + lane];
        xs[4 * g + 0] = t.x;
        xs[4 * g + 1] = t.y;
        xs[4 * g + 2] = t.z;
        xs[4 * g + 3] = t.w;
    }
}

template <int CW>
__device__ __forceinline__ void global_read_chunk(const float* __restrict__ xp, float (&xs)[CW]) {
    const float4* p = reinterpret_cast<const float4*>(xp);
#pragma unroll
    for (int g = 0; g < CW / 4; ++g) {
        const float4 t = p[g];
        xs[4 * g + 0] = t.x;
        xs[4 * g + 1] = t.y;
        xs[4 * g + 2] = t.z;
        xs[4 * g + 3] = t.w;
    }
}

// The one-shot product of workgroup `block` (blockIdx.x of a plain launch,
// or the block's index within its matrix in a grouped launch).
template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, int WAVES>
__device__ __forceinline__ void oneshot_body(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const float* __restrict__ x, float* __restrict__ y, uint32_t rows, uint32_t cols,
    uint32_t block, float4* __restrict__ smem) {
    constexpr int CW = (WT == kQ4) ? 32 : 16;   // weights per 16-byte chunk
    constexpr int G4 = CW / 4;
    constexpr int THREADS = WAVES * 64;
    constexpr float OFF = (WT == kQ4) ? 8.f : 128.f;
    constexpr uint32_t SB = SF16 ? 2 : 4;       // bytes per scale
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint32_t nchunks = cols / CW;
    const uint32_t S = (nchunks + 63) / 64;     // <= SMAX (host-checked)
    const uint32_t per_b = S * G4 * 64;          // float4 slots per vector
    float4* xl = smem;
    float* sxl = reinterpret_cast<float*>(smem + static_cast<size_t>(NB) * per_b);

    // ---- 1. first activation chunk of this thread (b = 0.., chunk c) ----
    const uint32_t nstage = NB * nchunks;       // chunks to stage
    float xs0[CW];
    if (static_cast<uint32_t>(tid) < nstage) {
        const uint32_t b = tid / nchunks, c = tid - b * nchunks;
        global_read_chunk<CW>(x + static_cast<uint64_t>(b) * cols + static_cast<uint64_t>(c) * CW,
                              xs0);
    }

    // ---- 2. every quant chunk and scale of this wave's rows ----
    const uint64_t row_bytes = (WT == kQ4) ? (cols >> 1) : cols;
    const uint32_t nblk = cols >> 5;
    const uint32_t row0 = (block * WAVES + wid) * NR;
    const uint32_t wrows = row0 < rows ? min(static_cast<uint32_t>(NR), rows - row0) : 0;
    const uint32_t rb = min(row0, rows - 1);
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(q + static_cast<uint64_t>(rb) * row_bytes, static_cast<uint64_t>(wrows) * row_bytes);
    const __amdgpu_buffer_rsrc_t drs =
        make_rsrc(static_cast<const uint8_t*>(d) + static_cast<uint64_t>(rb) * nblk * SB,
                  static_cast<uint64_t>(wrows) * nblk * SB);
    uint4 qv[NR][SMAX];
    uint32_t dv[NR][SMAX];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t qo = ch < nchunks ? r * static_cast<uint32_t>(row_bytes) + 16 * ch : kOob;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qrs, qo, 0, 0);
            qv[r][k] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const uint32_t ch = lane + 64 * k;
            const uint32_t blk = (WT == kQ4) ? ch : (ch >> 1);
            const uint32_t dofs = ch < nchunks ? (r * nblk + blk) * SB : kOob;
            if constexpr (SF16) dv[r][k] = __builtin_amdgcn_raw_buffer_load_b16(drs, dofs, 0, 0);
            else dv[r][k] = __builtin_amdgcn_raw_buffer_load_b32(drs, dofs, 0, 0);
        }
    }

    // ---- 3. activations -> LDS with chunk sums ----
    auto stage = [&](uint32_t j, const float (&xs)[CW]) {
        const uint32_t b = j / nchunks, c = j - b * nchunks;
        const uint32_t k = c >> 6, l = c & 63;
        float4* dst = xl + b * per_b + (k * G4) * 64 + l;
#pragma unroll
        for (int g = 0; g < G4; ++g)
            dst[g * 64] = make_float4(xs[4 * g], xs[4 * g + 1], xs[4 * g + 2], xs[4 * g + 3]);
        float sx;
        if constexpr (WT == kQ4) sx = q4_xsum(xs); else sx = q8_xsum(xs);
        sxl[b * S * 64 + c] = sx;
    };
    if (static_cast<uint32_t>(tid) < nstage) stage(tid, xs0);
    for (uint32_t j = tid + THREADS; j < nstage; j += THREADS) {
        float xs[CW];
        const uint32_t b = j / nchunks, c = j - b * nchunks;
        global_read_chunk<CW>(x + static_cast<uint64_t>(b) * cols + static_cast<uint64_t>(c) * CW, xs);
        stage(j, xs);
    }
    __syncthreads();
    if (wrows == 0) return;  // uniform per wave, after the barrier

    // ---- 4. multiply ----
    float acc[NB][NR];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[b][r] = 0.f;
#pragma unroll
    for (int k = 0; k < SMAX; ++k) {
        if (k < static_cast<int>(S)) {
            const uint32_t ch = lane + 64 * k;
            const bool valid = ch < nchunks;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float xs[CW];
                lds_read_x<CW>(xl + b * per_b, k, lane, xs);
                const float sx = sxl[b * S * 64 + ch];
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    float raw;
                    if constexpr (WT == kQ4) raw = q4_raw_dot(qv[r][k], xs);
                    else raw = q8_raw_dot(qv[r][k], xs);
                    const float t = fmaf(scale_from_bits<SF16>(dv[r][k]), raw - OFF * sx, acc[b][r]);
                    acc[b][r] = valid ? t : acc[b][r];
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float sum = wave_reduce(acc[b][r]);
            if (lane == 0 && static_cast<uint32_t>(r) < wrows)
                y[static_cast<uint64_t>(b) * rows + row0 + r] = sum;
        }
}

template <uint32_t WT, bool SF16, int NR, int NB, int SMAX, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_oneshot_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d,
    const float* __restrict__ x, float* __restrict__ y, uint32_t rows, uint32_t cols) {
    extern __shared__ float4 smem[];
    oneshot_body<WT, SF16, NR, NB, SMAX, WAVES>(q, d, x, y, rows, cols, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// Grouped launch: several matrices with the same number of columns multiply
// the same activations in one launch (a decode layer's wq | wk | wv, or
// w1 | w3).  Workgroups [first[i], first[i+1]) serve matrix i with the
// one-shot body of its own storage type, one row per wave.  One launch
// instead of several saves each extra launch's fixed start-up and drain.
// ---------------------------------------------------------------------------

constexpr int kMaxGroup = 8;

struct GroupArgs {
    const uint8_t* q[kMaxGroup];
    const void* d[kMaxGroup];
    float* y[kMaxGroup];
    uint32_t rows[kMaxGroup];
    uint32_t kind[kMaxGroup];        // 2 * (wtype == Q8_0) + scale_f16
    uint32_t first[kMaxGroup + 1];   // first workgroup of each matrix
    uint32_t n;
};

template <int NB, int SMAX4, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_group_kernel(GroupArgs g,
                                                                 const float* __restrict__ x,
                                                                 uint32_t cols) {
    extern __shared__ float4 smem[];
    uint32_t i = 0;
    while (i + 1 < g.n && blockIdx.x >= g.first[i + 1]) ++i;  // uniform
    const uint32_t blk = blockIdx.x - g.first[i];
    switch (g.kind[i]) {
        case 0: oneshot_body<kQ4, false, 1, NB, SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
        case 1: oneshot_body<kQ4, true, 1, NB, SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
        case 2: oneshot_body<kQ8, false, 1, NB, 2 * SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
        default: oneshot_body<kQ8, true, 1, NB, 2 * SMAX4, WAVES>(g.q[i], g.d[i], x, g.y[i], g.rows[i], cols, blk, smem); break;
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
    hipLaunchKernelGGL((gemv_oneshot_kernel<WT, SF16, NR, NB, SMAX, WAVES>), dim3(blocks),
                       dim3(WAVES * 64), lds, s, m.q, m.d, x, y, m.rows, m.cols);
    return hipGetLastError();
}

// LDS bytes of the staged activations and their chunk sums.
template <uint32_t WT>
uint64_t gemv_lds_bytes(uint32_t cols, uint32_t nb) {
    constexpr uint32_t CW = (WT == kQ4) ? 32 : 16;
    const uint64_t S = (cols / CW + 63) / 64;
    return static_cast<uint64_t>(nb) * S * 64 * (CW + 1) * 4;
}

// Launch shape: S = steps per row (64 chunks each).  Rows per wave NR: up to
// 4 for S = 1 and 2 for S = 2 (a wave's quant loads stay <= 4 per lane), 1
// beyond, and never so many that fewer than 2048 waves (8 per compute unit)
// remain.  Eight waves per workgroup share one LDS copy of the activations.
// QMV_GEMV_NR / QMV_GEMV_WAVES override (tuning sweeps).
template <uint32_t WT, bool SF16, int NB>
hipError_t gemv_pass(const MatView& m, const float* x, float* y, hipStream_t s) {
    constexpr uint32_t CW = (WT == kQ4) ? 32 : 16;
    const uint32_t S = (m.cols / CW + 63) / 64;
    const uint64_t lds = gemv_lds_bytes<WT>(m.cols, NB);
    const uint64_t row_bytes = (WT == kQ4) ? m.cols / 2 : m.cols;
    if (lds <= 64 * 1024 && S <= 16 && 4 * row_bytes < 0xFFFFFFF0ull) {
        uint32_t nr = S == 1 ? 4 : S == 2 ? 2 : 1;
        while (nr > 1 && m.rows / nr < 2048) nr /= 2;
        nr = tune_knob("QMV_GEMV_NR", nr);
        const uint32_t waves = tune_knob("QMV_GEMV_WAVES", 8);
        const size_t l = static_cast<size_t>(lds);
#define QMV_ONESHOT(NR_, SMAX_)                                                          \
    if (nr == NR_ && S <= SMAX_)                                                         \
        return waves == 8 ? gemv_oneshot_launch<WT, SF16, NR_, NB, SMAX_, 8>(m, x, y, l, s) \
                          : gemv_oneshot_launch<WT, SF16, NR_, NB, SMAX_, 4>(m, x, y, l, s);
        QMV_ONESHOT(4, 1)
        QMV_ONESHOT(2, 1)
        QMV_ONESHOT(2, 2)
        QMV_ONESHOT(1, 1)
        QMV_ONESHOT(1, 2)
        QMV_ONESHOT(1, 4)
        QMV_ONESHOT(1, 8)
        QMV_ONESHOT(1, 16)
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

template <int NB>
hipError_t group_pass(const MatView* ms, uint32_t n, const float* x, float* const* ys,
                      uint32_t done, hipStream_t s) {
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
        blocks += (ms[i].rows + WAVES - 1) / WAVES;
        const uint64_t b = ms[i].wtype == kQ4 ? gemv_lds_bytes<kQ4>(cols, NB) : gemv_lds_bytes<kQ8>(cols, NB);
        lds = b > lds ? b : lds;
    }
    g.first[n] = blocks;
    const float* xp = x + static_cast<uint64_t>(done) * cols;
    const size_t l = static_cast<size_t>(lds);
    if (S4 <= 1) hipLaunchKernelGGL((gemv_group_kernel<NB, 1, WAVES>), dim3(blocks), dim3(WAVES * 64), l, s, g, xp, cols);
    else if (S4 <= 2) hipLaunchKernelGGL((gemv_group_kernel<NB, 2, WAVES>), dim3(blocks), dim3(WAVES * 64), l, s, g, xp, cols);
    else if (S4 <= 4) hipLaunchKernelGGL((gemv_group_kernel<NB, 4, WAVES>), dim3(blocks), dim3(WAVES * 64), l, s, g, xp, cols);
    else hipLaunchKernelGGL((gemv_group_kernel<NB, 8, WAVES>), dim3(blocks), dim3(WAVES * 64), l, s, g, xp, cols);
    return hipGetLastError();
}

}  // namespace

// Batches up to this size run the vector kernel; larger ones the matrix
// cores (each vector pass re-reads the whole matrix).
constexpr uint32_t kGemvMaxBatch = 8;

hipError_t launch_gemv_group(const MatView* ms, uint32_t n, const float* x, float* const* ys,
                             uint32_t batch, hipStream_t s) {
    const uint32_t cols = ms[0].cols;
    const uint32_t S4 = (cols / 32 + 63) / 64;
    bool fits = n <= static_cast<uint32_t>(kMaxGroup) && batch <= kGemvMaxBatch && S4 <= 8;
    for (uint32_t i = 0; fits && i < n; ++i) {
        const uint64_t row_bytes = ms[i].wtype == kQ4 ? cols / 2 : cols;
        const uint64_t lds = ms[i].wtype == kQ4 ? gemv_lds_bytes<kQ4>(cols, 1) : gemv_lds_bytes<kQ8>(cols, 1);
        fits = lds * (batch > 4 ? 8 : batch > 2 ? 4 : batch) <= 64 * 1024 && row_bytes < 0xFFFFFFF0ull;
    }
    if (!fits) {  // one launch per matrix
        for (uint32_t i = 0; i < n; ++i) {
            const hipError_t e = launch_gemv(ms[i], x, ys[i], batch, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    uint32_t done = 0;
    while (done < batch) {
        const uint32_t left = batch - done;
        hipError_t e;
        uint32_t nb;
        if (left >= 8) { nb = 8; e = group_pass<8>(ms, n, x, ys, done, s); }
        else if (left >= 4) { nb = 4; e = group_pass<4>(ms, n, x, ys, done, s); }
        else if (left >= 2) { nb = 2; e = group_pass<2>(ms, n, x, ys, done, s); }
        else { nb = 1; e = group_pass<1>(ms, n, x, ys, done, s); }
        if (e != hipSuccess) return e;
        done += nb;
    }
    return hipSuccess;
}

hipError_t launch_gemv(const MatView& m, const float* x, float* y,
                       uint32_t batch, hipStream_t s) {
    if (batch > kGemvMaxBatch) return launch_gemm(m, x, true, y, batch, nullptr, s);
    if (m.wtype == kQ4) {
        return m.scale_f16 ? gemv_batched<kQ4, true>(m, x, y, batch, s)
                           : gemv_batched<kQ4, false>(m, x, y, batch, s);
    }
    return m.scale_f16 ? gemv_batched<kQ8, true>(m, x, y, batch, s)
                       : gemv_batched<kQ8, false>(m, x, y, batch, s);
}

}  // namespace qmv
