// Prefill product (GEMM) on the gfx950 matrix cores, with f16 operands.
//
// Y[t][r] = sum_c W[r][c] * X[t][c] (Krafla ".mlb model, version 1" page,
// "Body"; w = q * d for Q8_0, w = (nibble - 8) * d for Q4_0 with byte j of a
// block holding element j low and j + 16 high, sections "Q8_0" and "Q4_0"),
// t over the batch of activation rows.  This is the one place where the
// product is a dense contraction, so it runs on v_mfma_f32_16x16x32_f16.
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
// in which the matrix cores read their A operand: for a tile of 16 tokens
// and a block of 32 columns, one contiguous 1 KiB fragment whose 16-byte
// piece l = 16 g + m holds token m's columns 8 g .. 8 g + 7.  A wave then
// loads each A operand with one fully coalesced 1 KiB load, and the
// activations never pass through LDS.
//
// Product kernel.  A workgroup of 8 waves owns BM = 64 * WMW tokens x BN =
// 16 * NT matrix rows and walks its slice of K in steps of KG = 8 / WMW
// blocks of 32 columns.  Wave (wm, kg) multiplies tokens [64 wm, 64 wm + 64)
// of the tile by the NT row tiles over block kg of every step (4 x NT
// 16x16x32 products per step), the KG groups' sums meeting in LDS at the end.
// Per step, the workgroup decodes the tile's weights once into LDS, in the
// B-operand order (1 KiB per 16 rows x 32 columns, lane piece 16 g + n =
// row n's columns 8 g .. 8 g + 7), double-buffered; each thread decodes
// half blocks: a Q4_0 half block (bytes 8 h .. 8 h + 7) holds columns
// 8 h .. 8 h + 7 in its low nibbles and 16 + 8 h .. in its high nibbles,
// so its two pieces are g = h and g = 2 + h; a Q8_0 half block (bytes
// 16 h .. 16 h + 15) gives g = 2 h and 2 h + 1.  Sixteen consecutive
// threads take sixteen consecutive rows, so that their pieces fill 256
// contiguous bytes of LDS (every bank once) and a wave's quant loads cover
// 16 rows x 32 bytes.  Weight loads run DEPTH steps ahead in a ring of
// register sets, activation loads one step ahead; all loads are raw buffer
// loads, with an out-of-range offset (zeros, no traffic) past any edge.
//
// Placement.  Workgroups are dealt to the 8 XCDs round-robin by launch
// index; the launch index is mapped so that each XCD gets a contiguous run
// of tiles, which share one tile of staged activations (and one K slice)
// in that XCD's L2.  When the tiles are too few for the compute units, K
// is split and a second kernel adds the slices' partial sums in slice order
// (deterministic).
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
// Activation staging: one workgroup per token (and one per padding token up
// to a multiple of 16, which writes zeros).
// ---------------------------------------------------------------------------

constexpr int kTokenTop = 14;  // a token's largest staged magnitude is in [2^13, 2^14)

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

// The 8 values of piece p (columns 8p .. 8p + 7) of token row xr as float32.
template <bool XF32>
__device__ __forceinline__ void load_piece(const void* __restrict__ xr, uint32_t p, float (&v)[8]) {
    if constexpr (XF32) {
        const float4* s = reinterpret_cast<const float4*>(xr) + 2 * p;
        const float4 a = s[0], b = s[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 w = reinterpret_cast<const uint4*>(xr)[p];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, ws[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, ws[i] & 0xFFFF0000u);
        }
    }
}

template <bool XF32>
__global__ __launch_bounds__(256) void stage_x_kernel(const void* __restrict__ x, uint32_t M,
                                                      uint32_t K, uint4* __restrict__ xs,
                                                      int32_t* __restrict__ tshift) {
    __shared__ uint32_t red[4];
    const uint32_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const uint32_t npiece = K / 8, KB = K / 32;
    const uint32_t mt = t >> 4, m = t & 15;
    // piece p goes to fragment (mt, p / 4), slot 16 (p % 4) + m
    uint4* const dst = xs + static_cast<uint64_t>(mt) * KB * 64 + m;
    auto slot = [&](uint32_t p) { return (p >> 2) * 64 + (p & 3) * 16; };
    if (t >= M) {
        for (uint32_t p = tid; p < npiece; p += 256) dst[slot(p)] = make_uint4(0, 0, 0, 0);
        if (tid == 0) tshift[t] = 0;
        return;
    }
    const uint8_t* xr = static_cast<const uint8_t*>(x) + static_cast<uint64_t>(t) * K * (XF32 ? 4 : 2);
    // largest magnitude as an integer maximum of the magnitude bits, so that
    // inf and NaN win over every finite value
    uint32_t mx = 0;
    for (uint32_t p = tid; p < npiece; p += 256) {
        float v[8];
        load_piece<XF32>(xr, p, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = max(mx, __builtin_bit_cast(uint32_t, v[i]) & 0x7FFFFFFFu);
    }
    mx = wave_max_u32(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const bool bad = mx >= 0x7F800000u;
    const int sh = (bad || mx == 0) ? 0 : kTokenTop - __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, mx));
    for (uint32_t p = tid; p < npiece; p += 256) {
        float v[8];
        load_piece<XF32>(xr, p, v);
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f16x2 h = {static_cast<_Float16>(__builtin_amdgcn_ldexpf(v[2 * i], sh)),
                       static_cast<_Float16>(__builtin_amdgcn_ldexpf(v[2 * i + 1], sh))};
            o[i] = bad ? 0x7E007E00u : __builtin_bit_cast(uint32_t, h);
        }
        dst[slot(p)] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (tid == 0) tshift[t] = sh;
}

// ---------------------------------------------------------------------------
// Product kernel.
// ---------------------------------------------------------------------------

namespace mm {

constexpr int kThreads = 512;
constexpr int kWeightTop = 8;  // a row's largest |scale| * 2^(8 - E_r) is below 2^8

template <uint32_t WT, int NT, int WMW>
struct Cfg {
    static constexpr int KG = 8 / WMW;                   // k groups = blocks per step
    static constexpr int BM = 64 * WMW;                  // tokens per tile
    static constexpr int BN = 16 * NT;                   // matrix rows per tile
    static constexpr int UNITS = 2 * BN * KG;            // half blocks decoded per step
    static constexpr int UPT = (UNITS + kThreads - 1) / kThreads;
    static constexpr int QW = WT == kQ4 ? 2 : 4;         // quant words per half block
    static constexpr int STAGE = KG * NT * 1024;         // bytes of one LDS stage
    // the k groups' partial sums meet in LDS, JR row tiles at a time
    static constexpr int RED_J = (KG - 1) * WMW * 4096;  // bytes per row tile
    static constexpr int JR = (128 * 1024) / RED_J < NT ? (128 * 1024) / RED_J : NT;
    // two stages, then 1 KiB that threads without a half block write their
    // (zero) pieces to, so that the decode needs no branch
    static constexpr int DUMMY = 2 * STAGE;
    static constexpr int LDS = DUMMY + 1024 > JR * RED_J ? DUMMY + 1024 : JR * RED_J;
    // steps of weight loads in flight: a ring of register sets, shorter when
    // a thread decodes several half blocks per step
    static constexpr int DEPTH = UPT == 1 ? 4 : 2;
};

// One step's weight data of a thread: its half blocks' quants and scales.
template <int UPT, int QW>
struct WSet {
    uint32_t q[UPT][QW];
    uint32_t d[UPT];
};

// Decode one half block into its two 16-byte B pieces (8 f16 weights each).
// dh: f16 {d', d'} (f16 scales) ; df, mo: d' and -OFF * d' (f32 scales).
template <uint32_t WT, bool SF16, int QW>
__device__ __forceinline__ void decode_half(const uint32_t (&q)[QW], f16x2 dh, float df, float mo,
                                            uint4& p0, uint4& p1) {
    if constexpr (SF16) {
        // f16 1024 + u from a code byte u by a byte permute, an exact f16
        // subtraction of 1024 + OFF, and one rounding in the multiply by d'
        auto pair = [](uint32_t u, bool upper) {
            return __builtin_amdgcn_perm(0x64646464u, u, upper ? 0x04030402u : 0x04010400u);
        };
        const _Float16 off = static_cast<_Float16>(WT == kQ4 ? -1032.f : -1152.f);
        const f16x2 bias = {off, off};
        auto w2 = [&](uint32_t u, bool upper) {
            return __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, pair(u, upper)) + bias) * dh);
        };
        if constexpr (WT == kQ4) {
            uint32_t mask = 0x0F0F0F0Fu;
            asm("" : "+v"(mask));
            const uint32_t l0 = q[0] & mask, l1 = q[1] & mask;
            const uint32_t h0 = (q[0] >> 4) & mask, h1 = (q[1] >> 4) & mask;
            p0 = make_uint4(w2(l0, false), w2(l0, true), w2(l1, false), w2(l1, true));
            p1 = make_uint4(w2(h0, false), w2(h0, true), w2(h1, false), w2(h1, true));
        } else {
            const uint32_t u0 = q[0] ^ 0x80808080u, u1 = q[1] ^ 0x80808080u;
            const uint32_t u2 = q[2] ^ 0x80808080u, u3 = q[3] ^ 0x80808080u;
            p0 = make_uint4(w2(u0, false), w2(u0, true), w2(u1, false), w2(u1, true));
            p1 = make_uint4(w2(u2, false), w2(u2, true), w2(u3, false), w2(u3, true));
        }
    } else {
        // fl32(u * d' - OFF * d') = fl32(v * d') in one fused operation, then
        // rounded to f16
        auto w2 = [&](uint32_t u, bool upper) {
            const float a = upper ? ubyte_f32<2>(u) : ubyte_f32<0>(u);
            const float b = upper ? ubyte_f32<3>(u) : ubyte_f32<1>(u);
            const f16x2 h = {static_cast<_Float16>(fmaf(a, df, mo)), static_cast<_Float16>(fmaf(b, df, mo))};
            return __builtin_bit_cast(uint32_t, h);
        };
        if constexpr (WT == kQ4) {
            uint32_t mask = 0x0F0F0F0Fu;
            asm("" : "+v"(mask));
            const uint32_t l0 = q[0] & mask, l1 = q[1] & mask;
            const uint32_t h0 = (q[0] >> 4) & mask, h1 = (q[1] >> 4) & mask;
            p0 = make_uint4(w2(l0, false), w2(l0, true), w2(l1, false), w2(l1, true));
            p1 = make_uint4(w2(h0, false), w2(h0, true), w2(h1, false), w2(h1, true));
        } else {
            const uint32_t u0 = q[0] ^ 0x80808080u, u1 = q[1] ^ 0x80808080u;
            const uint32_t u2 = q[2] ^ 0x80808080u, u3 = q[3] ^ 0x80808080u;
            p0 = make_uint4(w2(u0, false), w2(u0, true), w2(u1, false), w2(u1, true));
            p1 = make_uint4(w2(u2, false), w2(u2, true), w2(u3, false), w2(u3, true));
        }
    }
}

template <uint32_t WT, bool SF16, int NT, int WMW>
__global__ __launch_bounds__(kThreads) void gemm_f16_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d, const int32_t* __restrict__ rexp,
    const uint4* __restrict__ xs, const int32_t* __restrict__ tshift, float* __restrict__ out,
    uint32_t M, uint32_t N, uint32_t K, uint32_t tiles_n, uint32_t tiles_m, uint32_t kb_split) {
    using C = Cfg<WT, NT, WMW>;
    constexpr int KG = C::KG, UPT = C::UPT, QW = C::QW;
    constexpr uint32_t SB = SF16 ? 2 : 4;
    constexpr uint32_t BLK_Q = WT == kQ4 ? 16 : 32;  // quant bytes per block
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % WMW, kg = wid / WMW;

    // launch index -> tile: each XCD (launch index mod 8) gets a contiguous
    // run of tile indexes L = (split * tiles_m + tile_m) * tiles_n + tile_n
    const uint32_t nwg = gridDim.x, id = blockIdx.x;
    const uint32_t L = (nwg & 7) == 0 ? (id & 7) * (nwg >> 3) + (id >> 3) : id;
    const uint32_t tile_n = L % tiles_n, g = L / tiles_n;
    const uint32_t tile_m = g % tiles_m, split = g / tiles_m;
    const uint32_t n0 = tile_n * C::BN, m0 = tile_m * C::BM;
    const uint32_t KB = K / 32;
    const uint32_t kb0 = split * kb_split;
    const uint32_t kbe = min(KB, kb0 + kb_split);
    const uint32_t S = (kbe - kb0 + KG - 1) / KG;  // steps
    const uint32_t MT = (M + 15) / 16;             // staged token tiles

    // weights: buffers over this tile's rows
    const uint32_t row_bytes = WT == kQ4 ? K / 2 : K;
    const uint32_t nrows = min(static_cast<uint32_t>(C::BN), N - n0);
    const __amdgpu_buffer_rsrc_t qr = rsrc(q + static_cast<uint64_t>(n0) * row_bytes, nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t dr =
        rsrc(static_cast<const uint8_t*>(d) + static_cast<uint64_t>(n0) * KB * SB, nrows * KB * SB);
    const __amdgpu_buffer_rsrc_t xr = rsrc(xs, MT * KB * 1024);

    // this thread's half blocks: unit u = ((j * KG + b) * 2 + h) * 16 + rr
    // (units past the last get no data and write to the dummy slot)
    uint32_t uq[UPT], ud[UPT], ub[UPT];
    uint32_t lds_lo[UPT], lds_hi[UPT];
    bool uok[UPT], udummy[UPT];
    int ushift[UPT];
#pragma unroll
    for (int p = 0; p < UPT; ++p) {
        const uint32_t u = tid + kThreads * p;
        const uint32_t rr = u & 15, h = (u >> 4) & 1, b = (u >> 5) % KG, j = (u >> 5) / KG;
        const uint32_t r = 16 * j + rr;
        udummy[p] = u >= static_cast<uint32_t>(C::UNITS);
        uok[p] = !udummy[p] && r < nrows;
        uq[p] = r * row_bytes + (WT == kQ4 ? 8 : 16) * h;
        ud[p] = r * KB * SB;
        ub[p] = b;
        const uint32_t g0 = WT == kQ4 ? h : 2 * h, g1 = WT == kQ4 ? 2 + h : 2 * h + 1;
        const uint32_t frag = (b * NT + (j < NT ? j : 0)) * 1024;
        lds_lo[p] = frag + (16 * g0 + rr) * 16;
        lds_hi[p] = frag + (16 * g1 + rr) * 16;
        ushift[p] = uok[p] ? kWeightTop - rexp[n0 + r] : 0;
    }

    auto load_w = [&](uint32_t s, WSet<UPT, QW>& w) {
#pragma unroll
        for (int p = 0; p < UPT; ++p) {
            const uint32_t kb = kb0 + s * KG + ub[p];
            const bool ok = uok[p] && kb < kbe;
            const uint32_t qo = ok ? uq[p] + kb * BLK_Q : kOob;
            const uint32_t dof = ok ? ud[p] + kb * SB : kOob;
            if constexpr (WT == kQ4) {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(qr, qo, 0, 0);
                w.q[p][0] = v[0];
                w.q[p][1] = v[1];
            } else {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qr, qo, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) w.q[p][i] = v[i];
            }
            if constexpr (SF16) w.d[p] = __builtin_amdgcn_raw_buffer_load_b16(dr, dof, 0, 0);
            else w.d[p] = __builtin_amdgcn_raw_buffer_load_b32(dr, dof, 0, 0);
        }
    };
    auto decode = [&](const WSet<UPT, QW>& w, uint32_t stage) {
#pragma unroll
        for (int p = 0; p < UPT; ++p) {
            const float dv = __builtin_amdgcn_ldexpf(scale_from_bits<SF16>(w.d[p]), ushift[p]);
            const _Float16 dh = static_cast<_Float16>(dv);
            uint4 p0, p1;
            decode_half<WT, SF16, QW>(w.q[p], f16x2{dh, dh}, dv, (WT == kQ4 ? -8.f : -128.f) * dv,
                                      p0, p1);
            const uint32_t lo = udummy[p] ? C::DUMMY + (lds_lo[p] & 1023) : stage + lds_lo[p];
            const uint32_t hi = udummy[p] ? C::DUMMY + (lds_hi[p] & 1023) : stage + lds_hi[p];
            *reinterpret_cast<uint4*>(lds + lo) = p0;
            *reinterpret_cast<uint4*>(lds + hi) = p1;
        }
    };
    // A operands: token tiles 4 wm .. 4 wm + 3 of the tile, block kg of step s
    const uint32_t mt0 = tile_m * (C::BM / 16) + 4 * wm;
    auto load_a = [&](uint32_t s, f16x8 (&a)[4]) {
        const uint32_t kb = kb0 + s * KG + kg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t mt = mt0 + i;
            const uint32_t off = (kb < kbe && mt < MT) ? ((mt * KB + kb) * 64 + lane) * 16 : kOob;
            a[i] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        }
    };
    f32x4 acc[4][NT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](uint32_t stage, const f16x8 (&a)[4]) {
        const uint8_t* bs = lds + stage + kg * NT * 1024 + lane * 16;
        f16x8 b[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) b[j] = *reinterpret_cast<const f16x8*>(bs + j * 1024);
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    };
    // Instruction order of a step (a hint to the scheduler, which otherwise
    // sinks the loads to the end of the step and the decode after every
    // matrix-core product): the step's loads first, then the products, two
    // B reads ahead, with the decode's vector instructions and LDS writes
    // placed between them.
    constexpr int kLoads = 4 + UPT * 2;
    auto order = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x020, kLoads, 0);  // buffer loads
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // B reads 0, 1
#pragma unroll
        for (int j = 0; j < NT; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two vector ops
            }
            if (j + 2 < NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 2 * UPT, 0);  // decoded pieces
    };

    constexpr int D = C::DEPTH;
    WSet<UPT, QW> w[D];
    f16x8 a[2][4];
#pragma unroll
    for (int k = 0; k < D; ++k) load_w(k, w[k]);
    load_a(0, a[0]);
    decode(w[0], 0);
    __syncthreads();
    // step s: A operands of step s + 1 and weights of step s + D are
    // requested, step s is multiplied from LDS stage s & 1, and the weights
    // of step s + 1 are decoded into the other stage.  The last step decodes
    // (zeros) into the unused stage.  Four steps per iteration, so that
    // every register set is named at compile time.
    uint32_t s = 0;
#define QMV_STEP(K_)                                                \
    load_a(s + 1, a[((K_) + 1) & 1]);                               \
    load_w(s + D, w[(K_) % D]);                                     \
    compute(((K_) & 1) * C::STAGE, a[(K_) & 1]);                    \
    decode(w[((K_) + 1) % D], (((K_) + 1) & 1) * C::STAGE);         \
    order();                                                        \
    __syncthreads();                                                \
    if (++s >= S) break;
    for (;;) {
        QMV_STEP(0)
        QMV_STEP(1)
        QMV_STEP(2)
        QMV_STEP(3)
    }
#undef QMV_STEP

    // ---- the k groups' sums meet in LDS (the stages are free now) ----
    if constexpr (KG > 1) {
        float* red = reinterpret_cast<float*>(lds);
#pragma unroll
        for (int j0 = 0; j0 < NT; j0 += C::JR) {
            if (kg > 0) {
#pragma unroll
                for (int jj = 0; jj < C::JR; ++jj)
                    if (j0 + jj < NT)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                red[((((jj * (KG - 1) + kg - 1) * WMW + wm) * 4 + i) * 4 + v) * 64 + lane] =
                                    acc[i][j0 + jj][v];
            }
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int jj = 0; jj < C::JR; ++jj)
                    if (j0 + jj < NT)
#pragma unroll
                        for (int gg = 1; gg < KG; ++gg)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
#pragma unroll
                                for (int v = 0; v < 4; ++v)
                                    acc[i][j0 + jj][v] +=
                                        red[((((jj * (KG - 1) + gg - 1) * WMW + wm) * 4 + i) * 4 + v) * 64 + lane];
            }
            __syncthreads();
        }
        if (kg > 0) return;
    }

    // ---- epilogue: lane holds row n = lane % 16 of each 16x16 tile and
    // tokens 4 (lane / 16) + v; outputs scaled back by powers of two ----
    float* o = out + static_cast<uint64_t>(split) * M * N;
    const uint32_t mw = m0 + 64 * wm + 4 * (lane >> 4);
    int tsh[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint32_t m = mw + 16 * i + v;
            tsh[i][v] = m < M ? tshift[m] : 0;
        }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const uint32_t n = n0 + 16 * j + (lane & 15);
        if (n >= N) continue;
        const int rsh = kWeightTop - rexp[n];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t m = mw + 16 * i + v;
                if (m < M)
                    o[static_cast<uint64_t>(m) * N + n] =
                        __builtin_amdgcn_ldexpf(acc[i][j][v], -(rsh + tsh[i][v]));
            }
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

}  // namespace mm

// ---------------------------------------------------------------------------
// Host side: the launch plan.
// ---------------------------------------------------------------------------

// Largest batch of one staged pass: the staged activations (2 bytes per
// value) stay within 32-bit buffer offsets.
uint32_t pass_tokens(uint32_t cols) {
    const uint64_t per_tile = uint64_t{16} * cols * 2;
    uint64_t tiles = (uint64_t{0x7FFFFFFF}) / per_tile;
    if (tiles > (1u << 20)) tiles = 1u << 20;
    return static_cast<uint32_t>(tiles * 16);
}

struct Plan {
    int nt = 8, wmw = 4;            // row tiles of 16 per workgroup, token waves of 64
    uint32_t tiles_n = 0, tiles_m = 0, splits = 1, kb_split = 0;
    uint32_t pass = 0;              // tokens per staged pass
};

Plan make_plan(const MatView& m, uint32_t batch) {
    Plan p;
    p.pass = batch < pass_tokens(m.cols) ? batch : pass_tokens(m.cols);
    const uint32_t M = p.pass;
    p.wmw = M <= 64 ? 1 : M <= 128 ? 2 : 4;
    const uint32_t bm = 64u * p.wmw, kg = 8u / p.wmw;
    p.tiles_m = (M + bm - 1) / bm;
    const uint32_t KB = m.cols / 32;
    const uint32_t steps = (KB + kg - 1) / kg;
    // Row tiles of 128 or 112 rows, whichever leaves fewer compute units
    // idle over the launch's rounds of 256 workgroups (14336 rows: 128 tiles
    // of 112 rows fill two token tiles' 256 workgroups exactly); then K is
    // split while the tiles are too few and every slice keeps >= 8 steps.
    // (batches of at most 64 take 112-row tiles only: at 128 rows, with four
    // half blocks to decode per thread, the kernel runs out of registers)
    double best = -1.0;
    for (int nt : {8, 7}) {
        if (p.wmw == 1 && nt == 8) continue;
        const uint32_t bn = 16u * nt;
        const uint32_t tn = (m.rows + bn - 1) / bn;
        uint32_t splits = 1;
        while (uint64_t{tn} * p.tiles_m * splits * 2 <= 320 && steps / (splits * 2) >= 8) splits *= 2;
        const uint64_t wgs = uint64_t{tn} * p.tiles_m * splits;
        const uint64_t rounds = (wgs + 255) / 256;
        const double eff = static_cast<double>(m.rows) / (static_cast<double>(tn) * bn) *
                           static_cast<double>(wgs) / static_cast<double>(rounds * 256);
        if (eff > best + 1e-9) {
            best = eff;
            p.nt = nt;
            p.tiles_n = tn;
            p.splits = splits;
        }
    }
    const uint32_t per = (steps + p.splits - 1) / p.splits;
    p.kb_split = per * kg;
    p.splits = (KB + p.kb_split - 1) / p.kb_split;
    return p;
}

uint64_t staged_bytes(uint32_t tokens, uint32_t cols) {
    const uint64_t mp = (uint64_t{tokens} + 15) / 16 * 16;
    return mp * cols * 2 + ((mp * 4 + 255) & ~uint64_t{255});
}

template <uint32_t WT, bool SF16, int NT, int WMW>
hipError_t launch_mm(const MatView& m, const uint4* xs, const int32_t* tsh, float* out,
                     uint32_t M, const Plan& p, hipStream_t s) {
    const uint64_t nwg = uint64_t{p.tiles_n} * p.tiles_m * p.splits;
    if (nwg > 0x7FFFFFFFull) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mm::gemm_f16_kernel<WT, SF16, NT, WMW>), dim3(static_cast<uint32_t>(nwg)),
                       dim3(mm::kThreads), 0, s, m.q, m.d, m.rexp, xs, tsh, out, M, m.rows, m.cols,
                       p.tiles_n, p.tiles_m, p.kb_split);
    return hipGetLastError();
}

template <uint32_t WT, bool SF16>
hipError_t launch_mm_shape(const MatView& m, const uint4* xs, const int32_t* tsh, float* out,
                           uint32_t M, const Plan& p, hipStream_t s) {
#define QMV_MM(NT_, WMW_) \
    if (p.nt == NT_ && p.wmw == WMW_) return launch_mm<WT, SF16, NT_, WMW_>(m, xs, tsh, out, M, p, s);
    QMV_MM(8, 4)
    QMV_MM(7, 4)
    QMV_MM(8, 2)
    QMV_MM(7, 2)
    QMV_MM(8, 1)
    QMV_MM(7, 1)
#undef QMV_MM
    return hipErrorInvalidValue;
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
    const Plan p0 = make_plan(m, batch);
    if (p0.pass == 0) return hipErrorInvalidValue;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    for (uint32_t done = 0; done < batch;) {
        const uint32_t M = batch - done < p0.pass ? batch - done : p0.pass;
        const Plan p = M == p0.pass ? p0 : make_plan(m, M);
        const uint64_t mp = (uint64_t{M} + 15) / 16 * 16;
        uint4* xs = reinterpret_cast<uint4*>(ws);
        int32_t* tsh = reinterpret_cast<int32_t*>(ws + mp * m.cols * 2);
        float* part = reinterpret_cast<float*>(ws + staged_bytes(p0.pass, m.cols));
        const uint8_t* xp = static_cast<const uint8_t*>(x) + uint64_t{done} * m.cols * (x_f32 ? 4 : 2);
        float* yp = y + uint64_t{done} * m.rows;
        if (mp > 0x7FFFFFFFull) return hipErrorInvalidValue;
        if (x_f32)
            hipLaunchKernelGGL(stage_x_kernel<true>, dim3(static_cast<uint32_t>(mp)), dim3(256), 0, s,
                               xp, M, m.cols, xs, tsh);
        else
            hipLaunchKernelGGL(stage_x_kernel<false>, dim3(static_cast<uint32_t>(mp)), dim3(256), 0, s,
                               xp, M, m.cols, xs, tsh);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        float* out = p.splits > 1 ? part : yp;
        if (m.wtype == kQ4)
            e = m.scale_f16 ? launch_mm_shape<kQ4, true>(m, xs, tsh, out, M, p, s)
                            : launch_mm_shape<kQ4, false>(m, xs, tsh, out, M, p, s);
        else
            e = m.scale_f16 ? launch_mm_shape<kQ8, true>(m, xs, tsh, out, M, p, s)
                            : launch_mm_shape<kQ8, false>(m, xs, tsh, out, M, p, s);
        if (e != hipSuccess) return e;
        if (p.splits > 1) {
            e = launch_splitk_sum(part, yp, uint64_t{M} * m.rows, p.splits, s);
            if (e != hipSuccess) return e;
        }
        done += M;
    }
    return hipSuccess;
}

}  // namespace qmv
