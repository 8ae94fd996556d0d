// Prefill product (GEMM) on the gfx950 matrix cores, with f16 operands.
//
// Y[t][r] = sum_c W[r][c] * X[t][c] (Krafla ".mlb model, version 1" page,
// "Body"; w = q * d for Q8_0, w = (nibble - 8) * d for Q4_0, where the
// first 16 elements of a block take the low halves of its 16 bytes in order
// and the last 16 the high halves, sections "Q8_0" and "Q4_0"),
// t over the batch of activation rows.  This is the one place where the
// product is a dense contraction, so it runs on v_mfma_f32_32x32x16_f16
// (measured at 1.76 PFLOP/s back to back on this GPU, against 1.2 for the
// 16x16x32 form).
//
// Numbers.  Each operand is held in f16 with a power-of-two scale chosen so
// that the f16 values neither overflow nor lose relative precision:
//   - weight w[r][c] enters as fl16(v * d * 2^(8 - E_r)), E_r the binary
//     exponent of row r's largest finite scale magnitude (recorded at
//     upload): the largest weight of a row stays below 2^15 and every
//     weight of a block whose scale is within 2^20 of the row's largest is
//     rounded once, to within 2^-11 relative (f32 scales: rounded to f32
//     first, then to f16);
//   - activation x[t][c] enters as fl16(x * 2^(14 - E_t)), E_t the exponent
//     of token t's largest magnitude, computed by a staging kernel (below):
//     a bf16 value within 2^31 of that largest converts exactly, an f32
//     value within 2^28 of it to within 2^-11 relative; a token holding inf
//     or NaN becomes NaN, and so do its outputs;
//   - the matrix cores multiply the f16 values exactly and accumulate in
//     float32; the output is scaled back by 2^-(8 - E_r + 14 - E_t) (exact).
// A bf16 product is therefore within 2^-11 * sum_c |W[r][c]| |X[t][c]| plus
// the float32 accumulation of the exact one, and an f32-activation product
// within about 2^-10 * sum_c |W[r][c]| |X[t][c]|.
//
// Staging.  A first kernel writes the scaled f16 activations in the order
// in which the matrix cores read their A operand: for a tile of 32 tokens
// and a block of 32 columns, two contiguous 1 KiB fragments (k slices s = 0,
// 1) whose 16-byte piece 32 h + m holds token m's columns 8 g .. 8 g + 7 of
// the block, g = 2 s + h.  A wave then loads each A operand with one fully
// coalesced 1 KiB load, and the activations never pass through LDS.
//
// Product kernel.  A workgroup of 8 waves owns 256 tokens x 128 matrix rows
// and walks its slice of K in steps of two blocks of 32 columns.  Wave (wm,
// kg) multiplies tokens [64 wm, 64 wm + 64) of the tile by the tile's four
// 32-row tiles over block kg of every step (2 x 4 x 2 products per step).
// Per step, the workgroup decodes the tile's weights once into LDS in the
// B-operand order (fragments of 32 rows x 16 columns; lane 32 h + n of a
// fragment = row n's columns 8 g .. 8 g + 7 of the block, g = 2 s + h),
// double-buffered, with one barrier per step.  Each thread decodes one half
// block per step: a Q4_0 half block (bytes 8 h .. 8 h + 7) holds element
// groups g = h (low nibbles) and g = 2 + h (high); a Q8_0 half block (bytes
// 16 h .. 16 h + 15) holds g = 2 h and 2 h + 1.  Four consecutive threads
// take one row's two blocks of a step, so that a wave's quant load covers
// 16 rows x 32 (or 64) contiguous bytes, the pattern the address units
// serve fastest.  Each step first requests its activations one step ahead
// and then its weights three steps ahead (loads complete in order, so the
// activations never wait behind a weight load of the same step; a second
// step of activations in flight measured slower); all loads
// are raw buffer loads, with an out-of-range offset (zeros, no traffic)
// past any edge.  At the end the two k groups exchange half of their sums
// through LDS, and each wave scales and stores two of the four row tiles
// (token shifts from LDS, raw buffer stores that drop what lies past the
// last token or row).
//
// Placement.  Workgroups are dealt to the 8 XCDs round-robin by launch
// index; the launch index is mapped so that each XCD gets a contiguous run
// of tiles, which share one tile of staged activations (and one K slice)
// in that XCD's L2.  When the tiles are too few for the compute units, K
// is split and a second kernel adds the slices' partial sums in slice order
// (deterministic).
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace qmv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kOob = 0xFFFFFFF0u;  // an offset past any buffer's end

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// ---------------------------------------------------------------------------
// Activation staging: one workgroup per kStageTokens consecutive tokens of a
// 32-token tile (padding tokens up to a multiple of 32 write zeros).  Lane
// kStageTokens * j + m of a wave holds token m's pieces (8 values each), so
// that a load reads 64 / kStageTokens consecutive pieces of each token's row
// and a store writes kStageTokens consecutive 16-byte slots of one fragment
// line (the slots of the tile's tokens for one piece are adjacent).  Every
// piece of a chunk is requested before any is used, so a token costs one
// round trip to memory (rows longer than a chunk are read twice).
// ---------------------------------------------------------------------------

constexpr int kTokenTop = 14;     // a token's largest staged magnitude is in [2^13, 2^14)
constexpr int kTokensPerTile = 32;
constexpr int kStageTokens = 2;   // tokens per workgroup (divides 32; 4 and 8 measured slower: fewer workgroups)
constexpr int kStageThreads = 256 * (kStageTokens > 2 ? kStageTokens / 2 : 1);
template <bool XF32>
constexpr int stage_pieces() { return XF32 ? 8 : 16; }  // pieces per thread per chunk

template <bool XF32>
struct Piece {
    uint32_t r[XF32 ? 8 : 4];
};

template <bool XF32>
__device__ __forceinline__ Piece<XF32> load_piece(const uint8_t* __restrict__ xr, uint32_t p, bool ok) {
    Piece<XF32> v;
    if constexpr (XF32) {
        const uint4 a = ok ? reinterpret_cast<const uint4*>(xr)[2 * p] : make_uint4(0, 0, 0, 0);
        const uint4 b = ok ? reinterpret_cast<const uint4*>(xr)[2 * p + 1] : make_uint4(0, 0, 0, 0);
        v.r[0] = a.x; v.r[1] = a.y; v.r[2] = a.z; v.r[3] = a.w;
        v.r[4] = b.x; v.r[5] = b.y; v.r[6] = b.z; v.r[7] = b.w;
    } else {
        const uint4 a = ok ? reinterpret_cast<const uint4*>(xr)[p] : make_uint4(0, 0, 0, 0);
        v.r[0] = a.x; v.r[1] = a.y; v.r[2] = a.z; v.r[3] = a.w;
    }
    return v;
}

template <bool XF32>
__device__ __forceinline__ float piece_value(const Piece<XF32>& v, int i) {
    if constexpr (XF32) return __builtin_bit_cast(float, v.r[i]);
    else return __builtin_bit_cast(float, (i & 1) ? (v.r[i >> 1] & 0xFFFF0000u) : (v.r[i >> 1] << 16));
}

template <bool XF32>
__device__ __forceinline__ uint32_t piece_max(const Piece<XF32>& v) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __builtin_bit_cast(uint32_t, piece_value<XF32>(v, i)) & 0x7FFFFFFFu);
    return m;
}

template <bool XF32>
__device__ __forceinline__ uint4 piece_f16(const Piece<XF32>& v, int sh, bool bad) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16x2 h = {static_cast<_Float16>(__builtin_amdgcn_ldexpf(piece_value<XF32>(v, 2 * i), sh)),
                         static_cast<_Float16>(__builtin_amdgcn_ldexpf(piece_value<XF32>(v, 2 * i + 1), sh))};
        o[i] = bad ? 0x7E007E00u : __builtin_bit_cast(uint32_t, h);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

template <bool XF32>
__global__ __launch_bounds__(kStageThreads) void stage_x_kernel(const void* __restrict__ x, uint32_t M,
                                                                uint32_t K, uint4* __restrict__ xs,
                                                                int32_t* __restrict__ tshift) {
    constexpr int T = kStageTokens, J = 64 / T, W = kStageThreads / 64, NP = stage_pieces<XF32>();
    constexpr uint32_t LANES = kStageThreads / T;  // lanes per token
    constexpr uint32_t CH = LANES * NP;            // pieces per token per chunk
    __shared__ uint32_t red[W * T];
    // token group of this workgroup: workgroups go to the 8 XCDs
    // round-robin, so contiguous runs of groups are given to one XCD (when
    // the padded batch allows) and each 32-token fragment is assembled in
    // one L2, not written in parts from eight
    const uint32_t nwg = gridDim.x, id = blockIdx.x;
    const uint32_t grp = (nwg % (8 * (kTokensPerTile / T))) == 0 ? (id & 7) * (nwg >> 3) + (id >> 3) : id;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t m = lane % T, j = lane / T;
    const uint32_t t = grp * T + m;
    const bool real = t < M;
    const uint32_t npiece = K / 8, KB = K / 32;
    const uint32_t mt = t / kTokensPerTile, mm = t % kTokensPerTile;
    // piece p (block p / 4, group g = p % 4: slice g / 2, half g % 2) goes to
    // fragment (mt, p / 4, g / 2), slot 32 (g % 2) + mm
    uint4* const dst = xs + static_cast<uint64_t>(mt) * KB * 128 + mm;
    auto slot = [&](uint32_t p) { return (p >> 2) * 128 + ((p >> 1) & 1) * 64 + (p & 1) * 32; };
    // this lane's pieces of a chunk: c0 + w J + j + LANES i
    const uint32_t p_lane = w * J + j;
    const uint8_t* xr = static_cast<const uint8_t*>(x) + static_cast<uint64_t>(real ? t : 0) * K * (XF32 ? 4 : 2);
    // largest magnitude as an integer maximum of the magnitude bits, so that
    // inf and NaN win over every finite value
    Piece<XF32> v[NP];
    uint32_t mx = 0;
    for (uint32_t c0 = 0; c0 < npiece; c0 += CH) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const uint32_t p = c0 + p_lane + LANES * i;
            v[i] = load_piece<XF32>(xr, p, real && p < npiece);
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) mx = max(mx, piece_max<XF32>(v[i]));
    }
    // over the lanes of the same token (lane bits above those of m), then
    // over the waves
#pragma unroll
    for (int d = T; d < 64; d *= 2)
        mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), d)));
    if (j == 0) red[w * T + m] = mx;
    __syncthreads();
    mx = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) mx = max(mx, red[k * T + m]);
    const bool bad = mx >= 0x7F800000u;
    const int sh = (bad || mx == 0) ? 0 : kTokenTop - __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, mx));
    // the last chunk is still in registers; earlier ones are read again
    const uint32_t last = npiece == 0 ? 0 : (npiece - 1) / CH * CH;
    for (uint32_t c0 = 0; c0 < last; c0 += CH) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const uint32_t p = c0 + p_lane + LANES * i;
            const Piece<XF32> u = load_piece<XF32>(xr, p, real && p < npiece);
            if (p < npiece) dst[slot(p)] = piece_f16<XF32>(u, sh, bad);
        }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const uint32_t p = last + p_lane + LANES * i;
        if (p < npiece) dst[slot(p)] = piece_f16<XF32>(v[i], sh, bad);
    }
    if (w == 0 && j == 0) tshift[t] = sh;
}

// ---------------------------------------------------------------------------
// Product kernel.
// ---------------------------------------------------------------------------

namespace mm {

constexpr int kThreads = 512;

// floor(2^32 / n) + 1 (n >= 2; 0 for n = 1): for every 32-bit i,
// __umulhi(i, that) is i / n or one more, since that exceeds 2^32 / n by at
// most 1.
inline uint32_t reciprocal(uint32_t n) {
    return n < 2 ? 0u : static_cast<uint32_t>((uint64_t{1} << 32) / n + 1);
}

// i / n (returned) and i % n (in rem) for wave-uniform i and n from the
// reciprocal r above, in scalar registers.
__device__ __forceinline__ uint32_t div_by(uint32_t i, uint32_t n, uint32_t r, uint32_t& rem) {
    uint32_t q = n == 1 ? i : __umulhi(i, r);
    uint32_t m = i - q * n;
    if (static_cast<int32_t>(m) < 0) {  // one too many
        q -= 1;
        m += n;
    }
    rem = m;
    return q;
}
constexpr int kWeightTop = 8;  // a row's largest |scale| * 2^(8 - E_r) is below 2^8

// B fragments in LDS: 1 KiB of operand (lanes 0-31 then lanes 32-63, 512
// bytes each, with 64 bytes between the halves), fragments 1280 bytes apart,
// and fragment f = (2 b + s) * 4 + j (block b of a step, k slice s, row
// tile j) shifted by 32 b + 64 s bytes.  A wave's 16-byte fragment read
// stays 256 contiguous bytes per 16 lanes (a read's 16-lane phase over the
// 64 banks), and the decode's 16-byte writes fall on 8 different 16-byte
// groups of each 128 bytes per 8 consecutive lanes (a write's phase).
constexpr uint32_t kFragStride = 1280;
constexpr uint32_t frag_off(uint32_t b, uint32_t f, uint32_t slot) {
    return f * kFragStride + b * 32 + ((f >> 2) & 1) * 64 + (slot >> 5) * 64 + slot * 16;
}

template <uint32_t WT, bool SF16>
struct Cfg {
    static constexpr int NT = 4;                          // 32-row tiles per workgroup (frag_off assumes 4)
    static constexpr int KG = 2;                          // blocks per step = k groups of waves
    static constexpr int WM = 4;                          // token waves of 64 per k group
    static constexpr int BM = 64 * WM;                    // tokens per tile
    static constexpr int BN = 32 * NT;                    // matrix rows per tile
    static constexpr int QW = WT == kQ4 ? 2 : 4;          // quant words per half block
    static constexpr uint32_t BLK_Q = WT == kQ4 ? 16 : 32;  // quant bytes per block
    static constexpr uint32_t SB = SF16 ? 2 : 4;            // bytes per scale
    static constexpr int STAGE = 2 * KG * NT * kFragStride + 256;  // one B stage
    // at the end each wave hands half its row tiles to the wave of the other
    // k group through LDS (the stages are free then), after the tile's token
    // shifts
    static constexpr int RED = KG * WM * (NT / 2) * 2 * 16 * 64 * 4;
    static constexpr int TSH = RED;
    static constexpr int LDS = 2 * STAGE > RED + BM * 4 ? 2 * STAGE : RED + BM * 4;
    static_assert(KG == 2, "two k groups share the output tiles");
    static constexpr int RA = 2;                          // A register sets (one step ahead)
    static constexpr int D = 3;                           // weight register sets (D steps ahead)
    static constexpr int UNROLL = 6;
    static_assert(UNROLL % RA == 0 && UNROLL % D == 0 && UNROLL % 2 == 0, "");
    static_assert(2 * BN * KG == kThreads, "one half block per thread per step");
};

// One step's weight data of a thread: its half block's quants and scale.
template <int QW>
struct WSet {
    uint32_t q[QW];
    uint32_t d;
};

// Decode one half block into its two 16-byte B pieces (8 f16 weights each).
// dh: f16 {d', d'} (f16 scales) ; df, mo: d' and -OFF * d' (f32 scales).
template <uint32_t WT, bool SF16, int QW>
__device__ __forceinline__ void decode_half(const uint32_t (&q)[QW], f16x2 dh, float df, float mo,
                                            uint4& p0, uint4& p1) {
    // the code bytes: Q4_0 nibbles (p0 from the low ones), Q8_0 q + 128
    uint32_t c[4];
    if constexpr (WT == kQ4) {
        uint32_t mask = 0x0F0F0F0Fu;
        asm("" : "+v"(mask));
        c[0] = q[0] & mask;
        c[1] = q[1] & mask;
        c[2] = (q[0] >> 4) & mask;
        c[3] = (q[1] >> 4) & mask;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = q[i] ^ 0x80808080u;
    }
    uint32_t o[8];
    if constexpr (SF16) {
        // f16 1024 + u from a code byte u by a byte permute, an exact f16
        // subtraction of 1024 + OFF, and one rounding in the multiply by d'
        const _Float16 off = static_cast<_Float16>(WT == kQ4 ? -1032.f : -1152.f);
        const f16x2 bias = {off, off};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, c[i], 0x04010400u);
            const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, c[i], 0x04030402u);
            o[2 * i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, lo) + bias) * dh);
            o[2 * i + 1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, hi) + bias) * dh);
        }
    } else {
        // fl32(u * d' - OFF * d') = fl32(v * d') in one fused operation, then
        // rounded to f16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2 a = {static_cast<_Float16>(fmaf(ubyte_f32<0>(c[i]), df, mo)),
                             static_cast<_Float16>(fmaf(ubyte_f32<1>(c[i]), df, mo))};
            const f16x2 b = {static_cast<_Float16>(fmaf(ubyte_f32<2>(c[i]), df, mo)),
                             static_cast<_Float16>(fmaf(ubyte_f32<3>(c[i]), df, mo))};
            o[2 * i] = __builtin_bit_cast(uint32_t, a);
            o[2 * i + 1] = __builtin_bit_cast(uint32_t, b);
        }
    }
    p0 = make_uint4(o[0], o[1], o[2], o[3]);
    p1 = make_uint4(o[4], o[5], o[6], o[7]);
}

template <uint32_t WT, bool SF16>
__global__ __launch_bounds__(kThreads) void gemm_f16_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d, const int32_t* __restrict__ rexp,
    const uint4* __restrict__ xs, const int32_t* __restrict__ tshift, float* __restrict__ out,
    uint32_t M, uint32_t N, uint32_t K, uint32_t tiles_n, uint32_t tiles_m, uint32_t kb_split,
    uint32_t inv_tiles_n, uint32_t inv_tiles_m) {
    using C = Cfg<WT, SF16>;
    constexpr int NT = C::NT, KG = C::KG, QW = C::QW, RA = C::RA, D = C::D;
    constexpr uint32_t SB = C::SB, BLK_Q = C::BLK_Q;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % C::WM, kg = wid / C::WM;

    // launch index -> tile: each XCD (launch index mod 8) gets a contiguous
    // run of tile indexes L = (split * tiles_m + tile_m) * tiles_n + tile_n
    const uint32_t nwg = gridDim.x, id = blockIdx.x;
    const uint32_t L = (nwg & 7) == 0 ? (id & 7) * (nwg >> 3) + (id >> 3) : id;
    // (divisions by multiplication with the host's reciprocals, in scalar
    // registers: a plain division runs on the vector units, and the buffer
    // descriptors derived from its result would then be used through a loop
    // over their distinct values at every load)
    uint32_t tile_n, tile_m;
    const uint32_t g = div_by(L, tiles_n, inv_tiles_n, tile_n);
    const uint32_t split = div_by(g, tiles_m, inv_tiles_m, tile_m);
    const uint32_t n0 = tile_n * C::BN, m0 = tile_m * C::BM;
    const uint32_t KB = K / 32;
    const uint32_t kb0 = split * kb_split;
    const uint32_t kbe = min(KB, kb0 + kb_split);
    const uint32_t S = (kbe - kb0 + KG - 1) / KG;  // steps
    const uint32_t MT = (M + kTokensPerTile - 1) / kTokensPerTile;  // staged token tiles
    // (offsets of token tiles past MT stay below 2^32: MT * KB * 2048 < 2^31)

    // weights: buffers over this tile's rows
    const uint32_t row_bytes = WT == kQ4 ? K / 2 : K;
    const uint32_t nrows = min(static_cast<uint32_t>(C::BN), N - n0);
    const __amdgpu_buffer_rsrc_t qr = rsrc(q + static_cast<uint64_t>(n0) * row_bytes, nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t dr =
        rsrc(static_cast<const uint8_t*>(d) + static_cast<uint64_t>(n0) * KB * SB, nrows * KB * SB);
    const __amdgpu_buffer_rsrc_t xr = rsrc(xs, MT * KB * 2048);

    // ---- this thread's half block of every step: row r = tid / 4, block
    // b = (tid / 2) % 2 of the step, half h = tid % 2.  Four consecutive
    // lanes read one row's 2 blocks (the address units serve such loads
    // about four times faster than loads whose consecutive lanes are in
    // different rows). ----
    const uint32_t ur = tid >> 2, ub = (tid >> 1) & 1, uh = tid & 1;
    const uint32_t uj = ur >> 5, un = ur & 31;
    const bool uok = ur < nrows;
    const uint32_t uq = ur * row_bytes + (WT == kQ4 ? 8 : 16) * uh;
    const uint32_t ud = ur * KB * SB;
    // pieces (slice s, lane half hh): Q4_0 low nibbles (0, h), high (1, h);
    // Q8_0 (h, 0) and (h, 1)
    const uint32_t us0 = WT == kQ4 ? 0 : uh, uh0 = WT == kQ4 ? uh : 0;
    const uint32_t us1 = WT == kQ4 ? 1 : uh, uh1 = WT == kQ4 ? uh : 1;
    const uint32_t lds_lo = frag_off(ub, (ub * 2 + us0) * NT + uj, 32 * uh0 + un);
    const uint32_t lds_hi = frag_off(ub, (ub * 2 + us1) * NT + uj, 32 * uh1 + un);
    const int ushift = uok ? kWeightTop - rexp[n0 + ur] : 0;
    // the tile's token shifts (zero past the last token), kept for the end
    const uint32_t mrows = min(static_cast<uint32_t>(C::BM), M - m0);
    const int32_t tsh_mine = tid < C::BM
        ? static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(rsrc(tshift + m0, mrows * 4), tid * 4, 0, 0))
        : 0;

    auto load_w = [&](uint32_t s, WSet<QW>& w) {
        const uint32_t kb = kb0 + s * KG + ub;
        const bool ok = uok && kb < kbe;
        const uint32_t qo = ok ? uq + kb * BLK_Q : kOob;
        const uint32_t dof = ok ? ud + kb * SB : kOob;
        if constexpr (WT == kQ4) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(qr, qo, 0, 0);
            w.q[0] = v[0];
            w.q[1] = v[1];
        } else {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qr, qo, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) w.q[i] = v[i];
        }
        if constexpr (SF16) w.d = __builtin_amdgcn_raw_buffer_load_b16(dr, dof, 0, 0);
        else w.d = __builtin_amdgcn_raw_buffer_load_b32(dr, dof, 0, 0);
    };
    auto decode = [&](const WSet<QW>& w, uint32_t stage) {
        const float dv = __builtin_amdgcn_ldexpf(scale_from_bits<SF16>(w.d), ushift);
        const _Float16 dh = static_cast<_Float16>(dv);
        uint4 p0, p1;
        decode_half<WT, SF16, QW>(w.q, f16x2{dh, dh}, dv, (WT == kQ4 ? -8.f : -128.f) * dv, p0, p1);
        *reinterpret_cast<uint4*>(lds + stage + lds_lo) = p0;
        *reinterpret_cast<uint4*>(lds + stage + lds_hi) = p1;
    };

    // ---- A operands: token tiles 2 wm, 2 wm + 1 of the tile, both slices of
    // block kg of step s.  No condition guards these loads (a condition
    // here becomes a branch whose other side drains every outstanding
    // load): a block past the slice is taken from the same token's row,
    // clamped to its last block, and meets weights of zero (the weight loads
    // past the slice return zeros); a token tile past the staged ones lies
    // past the buffer's end and reads zeros. ----
    const uint32_t mt0 = tile_m * (C::BM / kTokensPerTile) + 2 * wm;
    auto load_a = [&](uint32_t s, f16x8 (&a)[2][2]) {
        const uint32_t kb = min(kb0 + s * KG + kg, KB - 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const uint32_t off = ((((mt0 + i) * KB + kb) * 2 + sl) * 64 + lane) * 16;
                a[sl][i] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            }
    };
    f32x16 acc[2][NT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    auto compute = [&](uint32_t stage, const f16x8 (&a)[2][2]) {
        const uint8_t* bs = lds + stage;
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            f16x8 bf[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bf[j] = *reinterpret_cast<const f16x8*>(bs + frag_off(kg, (kg * 2 + sl) * NT + j, lane));
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[sl][i], bf[j], acc[i][j], 0, 0, 0);
        }
    };
    // Instruction order within a step (a hint to the scheduler, which would
    // otherwise bunch the decode after the products): B reads two ahead of
    // the products that use them, the decode's vector instructions between
    // the products.
    auto order = [&]() {
        constexpr int NMF = 2 * NT * 2;                          // products per step
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // B reads
#pragma unroll
        for (int k = 0; k < NMF; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one product
            if (k % 2 == 0 && k / 2 + 2 < 2 * NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // vector ops
        }
    };

    constexpr uint32_t ST0 = 0, ST1 = C::STAGE;
    WSet<QW> w[D];
    f16x8 a[RA][2][2];
#pragma unroll
    for (int k = 0; k < RA - 1; ++k) load_a(k, a[k]);
#pragma unroll
    for (int k = 0; k < D; ++k) load_w(k, w[k]);
    decode(w[0], ST0);
    __syncthreads();
    // step s: the A operands of step s + RA - 1, then the weights of step
    // s + D, are requested (in that order, so that the activations never
    // wait behind a weight load issued in the same step), step s is
    // multiplied from LDS stage s & 1, and the weights of step s + 1 are
    // decoded into the other stage.  The last step decodes (zeros) into the
    // unused stage.
    uint32_t s = 0;
#define QMV_STEP(K_)                                                \
    load_a(s + RA - 1, a[((K_) + RA - 1) % RA]);                    \
    __builtin_amdgcn_sched_barrier(0);                              \
    load_w(s + D, w[(K_) % D]);                                     \
    __builtin_amdgcn_sched_barrier(0);                              \
    compute((K_) & 1 ? ST1 : ST0, a[(K_) % RA]);                    \
    decode(w[((K_) + 1) % D], (K_) & 1 ? ST0 : ST1);                \
    order();                                                        \
    __syncthreads();                                                \
    if (++s >= S) break;
    for (;;) {
        QMV_STEP(0)
        QMV_STEP(1)
        QMV_STEP(2)
        QMV_STEP(3)
        QMV_STEP(4)
        QMV_STEP(5)
    }
#undef QMV_STEP

    // ---- the k groups' sums meet in LDS: k group 0 finishes row tiles 0
    // and 1, k group 1 tiles 2 and 3; each hands the other pair to its
    // partner wave ----
    float* red = reinterpret_cast<float*>(lds);
    int32_t* tsl = reinterpret_cast<int32_t*>(lds + C::TSH);
    auto hand = [&](auto JO) {
        constexpr int jo = decltype(JO)::value;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    red[((((kg * C::WM + wm) * 2 + jj) * 2 + i) * 16 + v) * 64 + lane] = acc[i][jo + jj][v];
    };
    if (kg == 0) hand(std::integral_constant<int, 2>{});
    else hand(std::integral_constant<int, 0>{});
    if (tid < C::BM) tsl[tid] = tsh_mine;
    __syncthreads();

    // ---- epilogue: lane holds row n = lane % 32 of each 32x32 tile and
    // tokens 8 (v / 4) + 4 (lane / 32) + v % 4; outputs scaled back by
    // powers of two and stored through a buffer over the tile's tokens
    // (stores past the last token or row are dropped) ----
    const uint32_t mw = 64 * wm + 4 * (lane >> 5);  // first token, tile-relative
    int4 ts[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) ts[i][g4] = *reinterpret_cast<const int4*>(tsl + mw + 32 * i + 8 * g4);
    const __amdgpu_buffer_rsrc_t orr =
        rsrc(out + (static_cast<uint64_t>(split) * M + m0) * N + n0, mrows * N * 4);
    const __amdgpu_buffer_rsrc_t er = rsrc(rexp + n0, nrows * 4);
    // a tile's output fits one 32-bit buffer range unless rows are very
    // many (2^22 or more): then plain stores with a bounds test
    const bool ranged = N < (1u << 22);
    float* const obase = out + (static_cast<uint64_t>(split) * M + m0) * N + n0;
    auto finish = [&](auto JK) {
        constexpr int jk = decltype(JK)::value;
        const int partner = (1 - kg) * C::WM + wm;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const uint32_t nl = 32 * (jk + jj) + (lane & 31);  // tile-relative row
            const int rsh = kWeightTop - static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(er, nl * 4, 0, 0));
            const uint32_t ob = nl < nrows ? nl * 4 : kOob;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float sum = acc[i][jk + jj][v] + red[(((partner * 2 + jj) * 2 + i) * 16 + v) * 64 + lane];
                    const int t = ts[i][v >> 2][v & 3];
                    const uint32_t ml = mw + 32 * i + 8 * (v >> 2) + (v & 3);
                    const float val = __builtin_amdgcn_ldexpf(sum, -(rsh + t));
                    if (ranged) {
                        const uint32_t off = nl < nrows ? ml * N * 4 + ob : kOob;
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), orr, off, 0, 0);
                    } else if (nl < nrows && ml < mrows) {
                        obase[static_cast<uint64_t>(ml) * N + nl] = val;
                    }
                }
        }
    };
    if (kg == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, 2>{});
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

}  // namespace mm

// ---------------------------------------------------------------------------
// Host side: the launch plan.
// ---------------------------------------------------------------------------

// Largest batch of one staged pass: the staged activations (2 bytes per
// value) stay within 32-bit buffer offsets.
uint32_t pass_tokens(uint32_t cols) {
    const uint64_t per_tile = uint64_t{kTokensPerTile} * cols * 2;
    uint64_t tiles = (uint64_t{0x7FFFFFFF}) / per_tile;
    if (tiles > (1u << 20)) tiles = 1u << 20;
    return static_cast<uint32_t>(tiles * kTokensPerTile);
}

struct Plan {
    uint32_t tiles_n = 0, tiles_m = 0, splits = 1, kb_split = 0;
    uint32_t pass = 0;              // tokens per staged pass
};

Plan make_plan(const MatView& m, uint32_t batch) {
    Plan p;
    p.pass = batch < pass_tokens(m.cols) ? batch : pass_tokens(m.cols);
    const uint32_t M = p.pass;
    constexpr uint32_t bm = 256, kg = 2;
    p.tiles_m = (M + bm - 1) / bm;
    p.tiles_n = (m.rows + 127) / 128;
    const uint32_t KB = m.cols / 32;
    const uint32_t steps = (KB + kg - 1) / kg;
    // too few tiles for 256 compute units: split K, keeping >= 8 steps a slice
    uint32_t splits = 1;
    while (uint64_t{p.tiles_n} * p.tiles_m * splits * 2 <= 320 && steps / (splits * 2) >= 8) splits *= 2;
    const uint32_t per = (steps + splits - 1) / splits;
    p.kb_split = per * kg;
    p.splits = (KB + p.kb_split - 1) / p.kb_split;
    return p;
}

uint64_t staged_bytes(uint32_t tokens, uint32_t cols) {
    const uint64_t mp = (uint64_t{tokens} + kTokensPerTile - 1) / kTokensPerTile * kTokensPerTile;
    return mp * cols * 2 + ((mp * 4 + 255) & ~uint64_t{255});
}

template <uint32_t WT, bool SF16>
hipError_t launch_mm(const MatView& m, const uint4* xs, const int32_t* tsh, float* out,
                     uint32_t M, const Plan& p, hipStream_t s) {
    const uint64_t nwg = uint64_t{p.tiles_n} * p.tiles_m * p.splits;
    if (nwg > 0x7FFFFFFFull) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mm::gemm_f16_kernel<WT, SF16>), dim3(static_cast<uint32_t>(nwg)),
                       dim3(mm::kThreads), 0, s, m.q, m.d, m.rexp, xs, tsh, out, M, m.rows, m.cols,
                       p.tiles_n, p.tiles_m, p.kb_split, mm::reciprocal(p.tiles_n),
                       mm::reciprocal(p.tiles_m));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_splitk_sum(const float* part, float* y, uint64_t total, uint32_t splits,
                             hipStream_t s) {
    const bool vec = total % 4 == 0;
    const uint64_t blocks = ((vec ? total / 4 : total) + 255) / 256;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (vec)
        hipLaunchKernelGGL(mm::splitk_reduce_kernel<true>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(256), 0, s, part, y, total, splits);
    else
        hipLaunchKernelGGL(mm::splitk_reduce_kernel<false>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(256), 0, s, part, y, total, splits);
    return hipGetLastError();
}

// Bytes of partial sums one pass of M tokens needs (0 without a split).
static uint64_t partial_bytes(const MatView& m, uint32_t M) {
    const Plan p = make_plan(m, M);
    return p.splits > 1 ? uint64_t{p.splits} * M * m.rows * 4 : 0;
}

size_t gemm_workspace_bytes(const MatView& m, uint32_t batch, bool /*x_f32*/) {
    const Plan p = make_plan(m, batch);
    // the staged activations of the largest pass, then the partial sums of
    // whichever pass (the full one or the last, shorter one) needs more
    uint64_t part = partial_bytes(m, p.pass);
    const uint32_t rest = batch % p.pass;
    if (rest != 0) {
        const uint64_t r = partial_bytes(m, rest);
        part = r > part ? r : part;
    }
    return static_cast<size_t>(staged_bytes(p.pass, m.cols) + part);
}

hipError_t launch_gemm(const MatView& m, const void* x, bool x_f32, float* y, uint32_t batch,
                       void* workspace, hipStream_t s) {
    if (workspace == nullptr) return hipErrorInvalidValue;
    // the scale array is addressed through one 32-bit buffer range
    if (uint64_t{m.rows} * (m.cols / 32) * (m.scale_f16 ? 2 : 4) >= 0xFFFFFFF0ull)
        return hipErrorNotSupported;
    const Plan p0 = make_plan(m, batch);
    if (p0.pass == 0) return hipErrorInvalidValue;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    for (uint32_t done = 0; done < batch;) {
        const uint32_t M = batch - done < p0.pass ? batch - done : p0.pass;
        const Plan p = M == p0.pass ? p0 : make_plan(m, M);
        const uint64_t mp = (uint64_t{M} + kTokensPerTile - 1) / kTokensPerTile * kTokensPerTile;
        uint4* xs = reinterpret_cast<uint4*>(ws);
        int32_t* tsh = reinterpret_cast<int32_t*>(ws + mp * m.cols * 2);
        float* part = reinterpret_cast<float*>(ws + staged_bytes(p0.pass, m.cols));
        const uint8_t* xp = static_cast<const uint8_t*>(x) + uint64_t{done} * m.cols * (x_f32 ? 4 : 2);
        float* yp = y + uint64_t{done} * m.rows;
        if (mp > 0x7FFFFFFFull) return hipErrorInvalidValue;
        const dim3 sg(static_cast<uint32_t>(mp / kStageTokens));
        if (x_f32)
            hipLaunchKernelGGL(stage_x_kernel<true>, sg, dim3(kStageThreads), 0, s, xp, M, m.cols, xs, tsh);
        else
            hipLaunchKernelGGL(stage_x_kernel<false>, sg, dim3(kStageThreads), 0, s, xp, M, m.cols, xs, tsh);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        float* out = p.splits > 1 ? part : yp;
        if (m.wtype == kQ4)
            e = m.scale_f16 ? launch_mm<kQ4, true>(m, xs, tsh, out, M, p, s)
                            : launch_mm<kQ4, false>(m, xs, tsh, out, M, p, s);
        else
            e = m.scale_f16 ? launch_mm<kQ8, true>(m, xs, tsh, out, M, p, s)
                            : launch_mm<kQ8, false>(m, xs, tsh, out, M, p, s);
        if (e != hipSuccess) return e;
        if (p.splits > 1) {
            e = launch_splitk_sum(part, yp, uint64_t{M} * m.rows, p.splits, s);
            if (e != hipSuccess) return e;
        }
        done += M;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Fixed scratch for callers that cannot allocate (qmv_gemm_noalloc): one
// array per GPU, held until the process ends.  Its address on a device is
// found once, with that device current; host code uses only that address.
// Every call on a GPU shares the array: calls that overlap on one GPU race.
// Nothing in it needs clearing (the staging and product kernels write
// every byte they read).
// ---------------------------------------------------------------------------
constexpr size_t kGemmScratchBytes = size_t{64} << 20;
static __device__ __align__(256) uint8_t scratch[kGemmScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t gemm_scratch(void** ptr, size_t* bytes) {
    *ptr = nullptr;
    *bytes = 0;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kGemmScratchBytes;
    return hipSuccess;
}

hipError_t launch_gemm_within(const MatView& m, const void* x, bool x_f32, float* y,
                              uint32_t batch, void* workspace, size_t ws_bytes, hipStream_t s) {
    if (workspace == nullptr || batch == 0) return hipErrorInvalidValue;
    // the largest pass (a multiple of 32 tokens, or the whole batch) whose
    // workspace fits
    uint32_t n = batch;
    while (gemm_workspace_bytes(m, n, x_f32) > ws_bytes) {
        if (n <= kTokensPerTile) return hipErrorNotSupported;
        n = (n / 2 + kTokensPerTile - 1) / kTokensPerTile * kTokensPerTile;
    }
    const uint64_t xs = uint64_t{m.cols} * (x_f32 ? 4 : 2);
    for (uint32_t done = 0; done < batch;) {
        const uint32_t k = batch - done < n ? batch - done : n;
        const hipError_t e = launch_gemm(m, static_cast<const uint8_t*>(x) + uint64_t{done} * xs, x_f32,
                                         y + uint64_t{done} * m.rows, k, workspace, s);
        if (e != hipSuccess) return e;
        done += k;
    }
    return hipSuccess;
}

}  // namespace qmv
