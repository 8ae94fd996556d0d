// Prefill product on Q8_0-quantized activations, on the int8 matrix cores.
//
// The page's CPU path quantizes the activations per block of 32 (the .mlb
// page, "Quantization rule": int8 quants xq with a float32 scale dx per
// block) and multiplies them by the weight codes block by block in
// integers.  Here, for tokens t and weight rows r:
//   y[t][r] = sum_b fl(dw[r,b] * dx[t,b]) * s[t,r,b],
//   s[t,r,b] = sum_j v[r,32b+j] * xq[t,32b+j]    (exact int32),
// with the block combine accumulated in float32.  K = 32 is one block, so
// one v_mfma_i32_32x32x32_i8 computes the exact block sums s of a 32 x 32
// output tile, which are then scaled and added to float32 accumulators
// (one conversion, one scale product and one multiply-add per output per
// block: the vector units, not the matrix cores, set the pace).
//
// Work split: a workgroup of 4 waves owns BM tokens (128, or 64 for batches
// of at most 64) x 128 weight rows and walks its slice of K in steps of two
// blocks; when the tiles alone leave compute units idle, K is split into
// slices whose partial sums a second kernel adds in slice order.  Each step's activation quants, weight
// codes (Q4_0 nibbles turned into signed bytes n - 8 on the way: elements
// 0..15 of a block are the low halves of its bytes, 16..31 the high halves)
// and both scale sets go through registers into a double-buffered LDS, one
// step ahead; each wave multiplies BM/2 tokens x 64 rows (BM/64 x 2 tiles).
// Tokens are the A operand and weight rows the B operand, so each lane's
// outputs belong to one weight row and 32 lanes store 32 consecutive rows.
// A and B fragments take the same 16 bytes of a block per half-wave, so the
// two operands agree on which k each byte is.
#include "device_common.h"
#include "kernels.h"

namespace qmv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 128;            // weight rows per workgroup
constexpr int BK = 64;             // two blocks per step
constexpr int PITCH = BK + 16;     // LDS bytes per token / row (spreads banks)
constexpr uint32_t kOob = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// One step's global data held by a thread: block (t & 1) of token t / 2 and
// of weight row t / 2.
struct I8Stage {
    u32x4 x[2];   // 32 activation quants
    u32x4 w[2];   // Q8_0: 32 codes; Q4_0: w[0] = the 16 packed bytes
    float dx, dw;
};

// signed n - 8 for the four nibbles in the low halves of the bytes of u
__device__ __forceinline__ uint32_t nib_to_i8(uint32_t u) {
    return ((u & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}

// NW waves per workgroup: NW / 2 along the tokens, 2 along the rows.  With
// 8 waves, waves 0-3 stage the activations and waves 4-7 the weights; the
// launcher uses 4 (8 waves of one token tile each measured 127 us against
// 108 us for 14336 x 4096 x 512).
template <uint32_t WT, bool SF16, int BM, int NW>
__global__ __launch_bounds__(NW * 64) void gemm_q8act_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ d, const int8_t* __restrict__ xq,
    const float* __restrict__ dx, float* __restrict__ y, uint32_t M, uint32_t N, uint32_t K,
    uint32_t k_per_split) {
    constexpr int TI = BM / (16 * NW);  // token tiles of 32 per wave
    __shared__ __attribute__((aligned(16))) uint8_t Xs[2][BM * PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t Ws[2][BN * PITCH];
    __shared__ __attribute__((aligned(16))) float Dx[2][2][BM];
    __shared__ __attribute__((aligned(16))) float Dw[2][2][BN];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    const uint32_t m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const uint32_t nb = K >> 5;
    // this workgroup's slice of K: blocks [kb / 32, ke / 32)
    const uint32_t kb = blockIdx.z * k_per_split, ke = min(K, kb + k_per_split);
    const uint32_t nbe = ke >> 5;
    const uint32_t row_bytes = (WT == kQ4) ? (K >> 1) : K;
    const __amdgpu_buffer_rsrc_t xr = rsrc(xq, static_cast<uint64_t>(M) * K);
    const __amdgpu_buffer_rsrc_t sr = rsrc(dx, static_cast<uint64_t>(M) * nb * 4);
    const __amdgpu_buffer_rsrc_t qr = rsrc(q, static_cast<uint64_t>(N) * row_bytes);
    const __amdgpu_buffer_rsrc_t dr = rsrc(d, static_cast<uint64_t>(N) * nb * (SF16 ? 2 : 4));

    // this thread's slot in a step: token / row (tid % 256) / 2, block tid & 1
    const uint32_t slot = static_cast<uint32_t>(tid & 255) >> 1, half = tid & 1;
    const uint32_t tok = m0 + slot, row = n0 + slot;
    const bool doX = NW == 4 || tid < 256, doW = NW == 4 || tid >= 256;  // wave-uniform

    auto fetch = [&](uint32_t k0, I8Stage& st) {
        const uint32_t b = (k0 >> 5) + half;   // block index within the row
        const bool kin = b < nbe;
        const bool tin = doX && kin && (BM == 128 || slot < BM) && tok < M;
        const bool rin = doW && kin && row < N;
        const uint32_t xo = tin ? tok * K + 32 * b : kOob;
        st.x[0] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo, 0, 0);
        st.x[1] = __builtin_amdgcn_raw_buffer_load_b128(xr, tin ? xo + 16 : kOob, 0, 0);
        st.dx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, tin ? (tok * nb + b) * 4 : kOob, 0, 0));
        if constexpr (WT == kQ4) {
            st.w[0] = __builtin_amdgcn_raw_buffer_load_b128(qr, rin ? row * row_bytes + 16 * b : kOob, 0, 0);
        } else {
            const uint32_t wo = rin ? row * row_bytes + 32 * b : kOob;
            st.w[0] = __builtin_amdgcn_raw_buffer_load_b128(qr, wo, 0, 0);
            st.w[1] = __builtin_amdgcn_raw_buffer_load_b128(qr, rin ? wo + 16 : kOob, 0, 0);
        }
        if constexpr (SF16) {
            const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b16(dr, rin ? (row * nb + b) * 2 : kOob, 0, 0);
            st.dw = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
        } else {
            st.dw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dr, rin ? (row * nb + b) * 4 : kOob, 0, 0));
        }
    };
    auto store = [&](const I8Stage& st, int buf) {
        if (doX && (BM == 128 || slot < BM)) {  // slots past BM hold no activations
            uint8_t* xs = Xs[buf] + slot * PITCH + 32 * half;
            *reinterpret_cast<u32x4*>(xs) = st.x[0];
            *reinterpret_cast<u32x4*>(xs + 16) = st.x[1];
            Dx[buf][half][slot] = st.dx;
        }
        if (!doW) return;
        uint8_t* ws = Ws[buf] + slot * PITCH + 32 * half;
        if constexpr (WT == kQ4) {
            const u32x4 p = st.w[0];
            const u32x4 lo = {nib_to_i8(p[0]), nib_to_i8(p[1]), nib_to_i8(p[2]), nib_to_i8(p[3])};
            const u32x4 hi = {nib_to_i8(p[0] >> 4), nib_to_i8(p[1] >> 4), nib_to_i8(p[2] >> 4),
                              nib_to_i8(p[3] >> 4)};
            *reinterpret_cast<u32x4*>(ws) = lo;        // elements 0..15
            *reinterpret_cast<u32x4*>(ws + 16) = hi;   // elements 16..31
        } else {
            *reinterpret_cast<u32x4*>(ws) = st.w[0];
            *reinterpret_cast<u32x4*>(ws + 16) = st.w[1];
        }
        Dw[buf][half][slot] = st.dw;
    };

    f32x16 acc[TI][2];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    const i32x16 zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const int r32 = lane & 31, h = lane >> 5;

    auto compute = [&](int buf) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            i32x4 a[TI], b[2];
#pragma unroll
            for (int i = 0; i < TI; ++i)
                a[i] = *reinterpret_cast<const i32x4*>(Xs[buf] + (wm * 32 * TI + 32 * i + r32) * PITCH + 32 * bb + 16 * h);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const i32x4*>(Ws[buf] + (wn * 64 + 32 * j + r32) * PITCH + 32 * bb + 16 * h);
            float dwj[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) dwj[j] = Dw[buf][bb][wn * 64 + 32 * j + r32];
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                // the scales of this lane's 16 tokens: 8 (v / 4) + 4 h + v % 4
                float dxi[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 t4 = *reinterpret_cast<const float4*>(&Dx[buf][bb][wm * 32 * TI + 32 * i + 8 * g + 4 * h]);
                    dxi[4 * g] = t4.x;
                    dxi[4 * g + 1] = t4.y;
                    dxi[4 * g + 2] = t4.z;
                    dxi[4 * g + 3] = t4.w;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const i32x16 s = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[i][j][v] = fmaf(static_cast<float>(s[v]), dxi[v] * dwj[j], acc[i][j][v]);
                }
            }
        }
    };

    I8Stage sa, sb;
    fetch(kb, sa);
    store(sa, 0);
    fetch(kb + BK, sb);
    __syncthreads();
    int cur = 0;
    for (uint32_t k0 = kb; k0 < ke; k0 += BK) {
        compute(cur);
        // the next step's data into the other buffer, the one after into sa
        store(sb, cur ^ 1);
        fetch(k0 + 2 * BK, sb);
        __syncthreads();
        cur ^= 1;
    }

    // lane: weight row n = 32 j + lane % 32, tokens 8 (v / 4) + 4 h + v % 4;
    // slice z's partial sums go to y + z M N
    y += static_cast<uint64_t>(blockIdx.z) * M * N;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t n = n0 + wn * 64 + 32 * j + r32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t t = m0 + wm * 32 * TI + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (t < M && n < N) y[static_cast<uint64_t>(t) * N + n] = acc[i][j][v];
            }
        }
}

template <int BM, int NW>
hipError_t q8act_launch(const MatView& m, const int8_t* xq, const float* dx, float* out,
                        uint32_t batch, uint32_t splits, uint32_t k_per_split, hipStream_t s) {
    const uint32_t gm = (batch + BM - 1) / BM;
    if (gm > 65535u || splits > 65535u) return hipErrorInvalidValue;
    const dim3 grid((m.rows + BN - 1) / BN, gm, splits), block(NW * 64);
    if (m.wtype == kQ4) {
        if (m.scale_f16)
            hipLaunchKernelGGL((gemm_q8act_kernel<kQ4, true, BM, NW>), grid, block, 0, s, m.q, m.d, xq, dx, out, batch, m.rows, m.cols, k_per_split);
        else
            hipLaunchKernelGGL((gemm_q8act_kernel<kQ4, false, BM, NW>), grid, block, 0, s, m.q, m.d, xq, dx, out, batch, m.rows, m.cols, k_per_split);
    } else {
        if (m.scale_f16)
            hipLaunchKernelGGL((gemm_q8act_kernel<kQ8, true, BM, NW>), grid, block, 0, s, m.q, m.d, xq, dx, out, batch, m.rows, m.cols, k_per_split);
        else
            hipLaunchKernelGGL((gemm_q8act_kernel<kQ8, false, BM, NW>), grid, block, 0, s, m.q, m.d, xq, dx, out, batch, m.rows, m.cols, k_per_split);
    }
    return hipGetLastError();
}

// Launch shape: token tile, and the K slices.  Tiles of 128 tokens (64 for
// batches of at most 64); while there are fewer than 384 workgroups (1.5 per
// compute unit) and each slice keeps at least 8 steps, K is split in two
// again.
struct Q8Plan {
    bool small = false;
    uint32_t splits = 1, k_per_split = 0;
};

Q8Plan q8_plan(const MatView& m, uint32_t batch) {
    Q8Plan p;
    p.small = batch <= 64;
    const uint32_t bm = p.small ? 64 : 128;
    const uint64_t tiles = uint64_t{(m.rows + BN - 1) / BN} * ((batch + bm - 1) / bm);
    const uint32_t steps = (m.cols + BK - 1) / BK;
    uint32_t splits = 1;
    while (tiles * splits < 384 && steps / (2 * splits) >= 8) splits *= 2;
    const uint32_t per = (steps + splits - 1) / splits;
    p.k_per_split = per * BK;
    p.splits = (m.cols + p.k_per_split - 1) / p.k_per_split;
    return p;
}

bool q8act_fits(const MatView& m, uint32_t batch) {
    // 32-bit buffer offsets over the activations, their scales, the codes
    // and the weight scales
    const uint64_t qbytes = (m.wtype == kQ4) ? uint64_t{m.rows} * m.cols / 2 : uint64_t{m.rows} * m.cols;
    return uint64_t{batch} * m.cols < 0xFFFFFFF0ull && qbytes < 0xFFFFFFF0ull &&
           uint64_t{m.rows} * (m.cols / 32) * 4 < 0xFFFFFFF0ull;
}

}  // namespace

size_t gemm_q8act_workspace_bytes(const MatView& m, uint32_t batch) {
    if (!q8act_fits(m, batch)) return 0;
    const Q8Plan p = q8_plan(m, batch);
    return p.splits > 1 ? static_cast<size_t>(p.splits) * batch * m.rows * sizeof(float) : 0;
}

hipError_t launch_gemm_q8act(const MatView& m, const int8_t* xq, const float* dx, float* y,
                             uint32_t batch, float* workspace, hipStream_t s) {
    if (!q8act_fits(m, batch)) return hipErrorNotSupported;
    const Q8Plan p = q8_plan(m, batch);
    float* out = p.splits > 1 ? workspace : y;
    if (out == nullptr) return hipErrorInvalidValue;
    const hipError_t e = p.small ? q8act_launch<64, 4>(m, xq, dx, out, batch, p.splits, p.k_per_split, s)
                                 : q8act_launch<128, 4>(m, xq, dx, out, batch, p.splits, p.k_per_split, s);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_sum(workspace, y, uint64_t{batch} * m.rows, p.splits, s);
}

}  // namespace qmv
