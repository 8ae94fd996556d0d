// Batched decode product on the matrix cores, f16 operands: Y[t][r] =
// sum_c W[r][c] x[t][c] for a Q8_0 matrix with f16 scales and 512 or 1024
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
// tokens of f16 activations in LDS (one row of 2*cols bytes per token, its
// 16-byte chunks XOR-swizzled by the token's low four bits so that a wave's
// fragment reads spread over all 64 banks).  Each
// wave walks tiles of 32 weight rows; tokens are the A operand (two 32-token
// tiles) and weight rows the B operand of v_mfma_f32_32x32x16_f16, so a
// lane's output column is a weight row and stores of 32 consecutive rows per
// token coalesce.  The B operand wants lane (r, h) = (lane % 32, lane / 32)
// to hold 8 + 8 quants of row r (block j, half h); loading that directly
// makes every load instruction touch 32 rows, which the address and L1 units
// serve one lane at a time.  Instead a wave loads four blocks of its 32 rows
// with four instructions of 8 rows x 128 contiguous bytes (whole cache
// lines), writes them to its own 4 KiB LDS slice (16-byte chunks
// XOR-swizzled by row so that both the writes and the reads below are free
// of bank conflicts) and reads them back in the operand layout.  The
// activations are read with the same split of k, so A and B agree on which k
// each step sums.  Loads go by groups of 8 blocks (2 quads of quant loads
// and one 16-byte load of a row's 8 scales) in two register sets, the next
// group in flight while one is multiplied, across tile boundaries; raw
// buffer loads past the wave's last group get an out-of-range offset and
// return zeros, so the loads need no branches.  The per-token output scales
// live in one register (lane t: token t) and are read with readlane.
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
constexpr uint32_t kOob = 0xFFFFFFF0u;
constexpr int kXBytes = kTokens * 2 * kMaxCols;
constexpr int kSlice = 32 * 128;  // a wave's LDS slice: 32 rows x four blocks
// cache-policy bits of the output stores: non-temporal (measured 77.4 ->
// 72.6-74.7 us for 248320 x 1024 at batch 64, bit-identical)
constexpr int kStreamStore = 2;
// cache-policy bits of the weight loads: non-temporal.  Each load
// instruction takes whole 128-byte lines (8 rows x 128 bytes), so no line is
// needed again after its load (with loads of half lines this policy was
// slower: the other half was evicted before its load came).
constexpr int kWeightLoad = 2;

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

// Byte offset in a wave's slice of row n's 16-byte chunk c (0..7) of four
// blocks: chunk index XORed with the row's low three bits, so that 8
// consecutive rows of either access pattern hit 8 different groups of four
// banks.
__device__ __forceinline__ uint32_t slice_off(uint32_t n, uint32_t c) {
    return n * 128 + ((c ^ ((n >> 1) & 7)) << 4);
}

// Byte offset in the activations of token t's 16-byte chunk c (8 values),
// XOR-swizzled the same way.
__device__ __forceinline__ uint32_t x_off(uint32_t t, uint32_t c, uint32_t P) {
    return t * P + ((c ^ (t & 15)) << 4);
}

// Loads of one group of 8 blocks of a tile: the quants, as two quads of four
// blocks, each four loads of 8 rows x 128 contiguous bytes (whole cache
// lines), and this lane's row's 8 scales.
struct Group {
    u32x4 q[2][4];
    u32x4 sc;
};

template <int NJ>
__global__ __launch_bounds__(kWaves * 64) void gemv_mfma_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ d, const float* __restrict__ x,
    float* __restrict__ y, uint32_t rows, uint32_t ntok, float wscale, float inv_wscale) {
    constexpr uint32_t cols = 32 * NJ;
    constexpr uint32_t NG = NJ / 8;   // groups of 8 blocks per row
    static_assert(NG % 2 == 0, "groups alternate between two register sets within a tile");
    __shared__ __align__(16) uint8_t xs[kXBytes];
    __shared__ __align__(16) uint8_t wsl[kWaves * kSlice];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr uint32_t P = 2 * cols;  // LDS bytes per token
    const uint32_t r = lane & 31, h = lane >> 5;
    uint8_t* slice = wsl + wid * kSlice;

    const uint32_t tiles = (rows + 31) / 32;
    const uint32_t first = blockIdx.x * kWaves + wid;
    const uint32_t stride = gridDim.x * kWaves;
    const uint32_t my_tiles = first < tiles ? (tiles - first + stride - 1) / stride : 0;
    const uint32_t ngroups = my_tiles * NG;

    // group G of this wave: tile G / NG (rows from (first + tile * stride) * 32),
    // blocks 8 (G % NG) ...; a group past the wave's last gets out-of-range
    // offsets
    // (a dead group reads through empty buffer ranges: no select around the
    // offsets, which the compiler would turn into branches around the loads)
    // Tile t takes its groups in the order rot(t), rot(t) + 1, ... (mod NG):
    // waves start at different column ranges, which spreads their
    // concurrent reads over the memory channels.
    auto rot = [&](uint32_t tile) { return (first + tile) % NG; };
    auto load_group = [&](uint32_t G, Group& dst) {
        const uint32_t tile = G / NG, g = (G % NG + rot(tile)) % NG;
        const bool live = G < ngroups;
        const uint32_t base = live ? (first + tile * stride) * 32 : 0;
        const __amdgpu_buffer_rsrc_t gq = rsrc(q, live ? rows * cols : 0);
        const __amdgpu_buffer_rsrc_t gd = rsrc(d, live ? rows * NJ * 2 : 0);
        // the scales first: loads complete in order, so the group's first
        // block then waits for its own quants only
        dst.sc = __builtin_amdgcn_raw_buffer_load_b128(gd, (base + r) * NJ * 2 + 16 * g, 0, 0);
#pragma unroll
        for (int qd = 0; qd < 2; ++qd)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t row = base + 8 * i + (lane >> 3);
                const uint32_t off = row * cols + 256 * g + 128 * qd + 16 * (lane & 7);
                dst.q[qd][i] = __builtin_amdgcn_raw_buffer_load_b128(gq, off, 0, kWeightLoad);
            }
    };

    Group ga, gb;
    load_group(0, ga);
    load_group(1, gb);

    // ---- activations -> f16 in LDS: wave w converts tokens w, w + 8, ...,
    // with all of its loads requested first (one round trip, not eight) ----
    constexpr int TPW = kTokens / kWaves;  // tokens per wave
    {
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
                    *reinterpret_cast<uint2*>(xs + x_off(t, c4 >> 1, P) + 8 * (c4 & 1)) =
                        make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
                }
            }
            // (the output scales pass through the start of the slices, free
            // until the first group is multiplied)
            if (lane == 0)
                reinterpret_cast<float*>(wsl)[t] =
                    t >= ntok ? 0.f
                    : finite ? __builtin_amdgcn_ldexpf(1.0f, -sh) * inv_wscale
                             : __builtin_bit_cast(float, 0x7FC00000u);
        }
    }
    __syncthreads();
    // lane t keeps token t's output scale (read back per store by bpermute)
    const float tscale = reinterpret_cast<const float*>(wsl)[lane];
    __syncthreads();

    const __amdgpu_buffer_rsrc_t yrs = rsrc(y, ntok * rows * 4);
    f32x16 acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mt][e] = 0.f;

    // multiplies group G (blocks 8g .. 8g + 7 of its tile) into acc
    auto run_group = [&](const Group& gr, uint32_t g) {
#pragma unroll
        for (int qd = 0; qd < 2; ++qd) {
            // quad qd to the slice in the loaded layout, then back per block
            // in the operand layout
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4*>(slice + slice_off(8 * i + (lane >> 3), lane & 7)) = gr.q[qd][i];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int jj = 4 * qd + b;         // block within the group
                const uint32_t j = 8 * g + jj;     // block within the row
                const u32x4 w = *reinterpret_cast<const u32x4*>(slice + slice_off(r, 2 * b + h));
                const uint32_t sbits = gr.sc[jj / 2] >> (16 * (jj % 2));
                const _Float16 ds = static_cast<_Float16>(
                    static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sbits))) * wscale);
                const f16x2 dd = {ds, ds};
                f16x8 wf[2];
                dequant16(w, dd, wf);
                f16x8 xf[2][2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const uint32_t t = 32 * mt + r, c = 4 * j + 2 * h;
                    xf[mt][0] = *reinterpret_cast<const f16x8*>(xs + x_off(t, c, P));
                    xf[mt][1] = *reinterpret_cast<const f16x8*>(xs + x_off(t, c + 1, P));
                }
#pragma unroll
                for (int k = 0; k < 2; ++k)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[mt][k], wf[k], acc[mt], 0, 0, 0);
            }
        }
    };
    // stores tile `tile` (raw buffer stores: a token or row past the end gets
    // an out-of-range offset and is dropped) and clears acc
    auto store_tile = [&](uint32_t tile) {
        const uint32_t row = (first + tile * stride) * 32 + r;
        const bool rok = row < rows;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t t = 32 * mt + 8 * (e / 4) + 4 * h + (e % 4);
                const uint32_t off = (rok && t < ntok) ? (t * rows + row) * 4 : kOob;
                // the store takes the 32-bit pattern (an unsigned int);
                // non-temporal: the logits are not read again here
                // token t = t0 + 4h: the scales of both halves by readlane
                // (a constant lane each), then a select
                const int t0 = 32 * mt + 8 * (e / 4) + (e % 4);
                const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tscale), t0));
                const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tscale), t0 + 4));
                const float ts = h ? s1 : s0;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[mt][e] * ts),
                                                      yrs, off, 0, kStreamStore);
                acc[mt][e] = 0.f;
            }
    };

    // tiles of NG groups (NG even): group g of a tile runs from register set
    // g % 2, which is then refilled with the group two ahead (the next tile's
    // first groups at the end), so the sequence is static and the tile's
    // outputs are stored after its last group
    for (uint32_t tile = 0; tile < my_tiles; ++tile) {
        // (scheduling barriers keep each group's work in place: letting the
        // scheduler interleave whole groups runs out of registers)
#pragma unroll
        for (uint32_t g = 0; g < NG; g += 2) {
            run_group(ga, (g + rot(tile)) % NG);
            __builtin_amdgcn_sched_barrier(0);
            load_group(tile * NG + g + 2, ga);
            __builtin_amdgcn_sched_barrier(0);
            run_group(gb, (g + 1 + rot(tile)) % NG);
            __builtin_amdgcn_sched_barrier(0);
            load_group(tile * NG + g + 3, gb);
            __builtin_amdgcn_sched_barrier(0);
        }
        store_tile(tile);
    }
}

}  // namespace

bool gemv_mfma_fits(const MatView& m) {
    // Q8_0 with f16 scales, cols 512 or 1024 (an even number of groups of 8
    // blocks, activations of one pass in LDS), and weights and outputs within
    // 32-bit buffer offsets
    return m.wtype == kQ8 && m.scale_f16 && (m.cols == 512 || m.cols == 1024) &&
           static_cast<uint64_t>(m.rows) * m.cols < 0xFFFFFFF0ull &&
           static_cast<uint64_t>(m.rows) * kTokens * 4 < 0xFFFFFFF0ull;
}

hipError_t launch_gemv_mfma(const MatView& m, const float* x, float* y, uint32_t batch,
                            hipStream_t s) {
    if (!gemv_mfma_fits(m)) return hipErrorNotSupported;
    const float wscale = ldexpf(1.0f, 8 - m.dexp);
    const float inv = ldexpf(1.0f, m.dexp - 8);
    const uint32_t tiles = (m.rows + 31) / 32;
    const uint32_t want = (tiles + kWaves - 1) / kWaves;
    const uint32_t blocks = want < 256 ? want : 256;
    for (uint32_t done = 0; done < batch; done += kTokens) {
        const uint32_t nt = batch - done < static_cast<uint32_t>(kTokens) ? batch - done : kTokens;
        const uint8_t* q = m.q;
        const uint16_t* d = static_cast<const uint16_t*>(m.d);
        const float* xp = x + static_cast<uint64_t>(done) * m.cols;
        float* yp = y + static_cast<uint64_t>(done) * m.rows;
        if (m.cols == 512)
            hipLaunchKernelGGL(gemv_mfma_kernel<16>, dim3(blocks), dim3(kWaves * 64), 0, s, q, d, xp, yp, m.rows, nt, wscale, inv);
        else
            hipLaunchKernelGGL(gemv_mfma_kernel<32>, dim3(blocks), dim3(kWaves * 64), 0, s, q, d, xp, yp, m.rows, nt, wscale, inv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmv
