// Projection-cache populate (prefill) for gfx950.
//
// C-Kernel-Engine, "Whisper: Trace One Encoder Tensor into Every Decoder
// Layer", "The concept": one encoder memory E feeds every decoder layer's own
// K and V projections, K_l = E x WK_l and V_l = E x WV_l. All 2L projections
// read the same E, so they form one grouped contraction
//     C[m][n] = sum_k E[m][k] * W(n)[k][n mod HD],   m < B*T, n < 2*L*HD,
// where column block n / HD selects WK_0..WK_{L-1}, WV_0..WV_{L-1}.
// The page's prefill emits token-major rows and then re-lays them head-major
// with a separate transpose ("Deliberate failure"); here the epilogue writes
// each accumulator straight to its head-major slot Kc/Vc[l][b][h][t][d].
//
// A dense contraction, so it runs on the matrix cores (MFMA):
//   fp32 inputs: v_mfma_f32_32x32x2_f32, fp32 products and accumulation;
//   bf16 inputs: v_mfma_f32_32x32x16_bf16, fp32 accumulation, result rounded
//                to nearest-even bf16 when stored.
// Workgroup = 4 waves in a WGM x WGN grid; each wave owns a (BM/WGM) x (BN/WGN)
// sub-tile made of 32x32 MFMA blocks. Operand tiles are staged through LDS.
#include "cke_device.h"
#include "cke_internal.h"

#include <cstring>

namespace cke {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16_bf __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_bf lds_v4i16;

struct GemmArgs {
    const void* E;
    WeightTable wt;
    void* Kc;
    void* Vc;
    int M, dm, T, L, B, H, D;
    const float* pos;    // memory lift only: [pos_rows][H*D] or nullptr
    int pos_rows;
};

// Row of a 32x32 MFMA accumulator block held in register r of `lane`
// (column = lane % 32).
__device__ __forceinline__ int acc_row(int lane, int r) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <typename TOUT>
__device__ __forceinline__ void store_out(TOUT* C, size_t idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* C, size_t idx, float v) { C[idx] = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* C, size_t idx, float v) {
    C[idx] = to_bf16_bits(v);
}

template <int BM, int BN, int WGM, int WGN, typename TOUT>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                         int m0, int p, int col0)
{
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l = p < a.L ? p : p - a.L;
    const size_t TD = (size_t)a.T * a.D;
    TOUT* C = static_cast<TOUT*>(p < a.L ? a.Kc : a.Vc) + (size_t)l * a.B * a.H * TD;
    // address = row part ((b*H)*T + t)*D + column part h*T*D + d: the column
    // part is fixed per block column, the row part per accumulator register,
    // so the divisions run once per row and once per column, not per element
    size_t coff[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = col0 + wn * WTN + nb * 32 + (lane & 31);
        const int h = col / a.D;
        coff[nb] = (size_t)h * TD + (col - h * a.D);
    }
    const int rbase = m0 + wm * WTM;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = rbase + mb * 32 + acc_row(lane, r);
            if (row < a.M) {
                const int b = row / a.T;
                TOUT* Cr = C + (size_t)b * a.H * TD + (size_t)(row - b * a.T) * a.D;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) store_out<TOUT>(Cr, coff[nb], acc[mb][nb][r]);
            }
        }
}

// Memory-lift epilogue for accumulators laid out as in epilogue (lane l holds
// column l % 32 of each 32x32 block, register r its row acc_row(l, r)):
// C[m][n] = gelu(acc) (+ pos[m % pos_rows][n]), C token-major [M][H*D]. Each
// store covers 32 consecutive columns of one row per half-wave.
template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void epilogue_lift(const GemmArgs& a, const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                              int m0, int n0)
{
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int N = a.H * a.D;
    float* C = static_cast<float*>(a.Kc);
    auto gelu = [](float v) { return 0.5f * v * (1.f + erff(v * 0.70710678118654752f)); };
    const int col = n0 + wn * WTN + (lane & 31);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WTM + mb * 32 + acc_row(lane, r);
            if (row < a.M) {
                float* Cr = C + (size_t)row * N + col;
                const float* P = a.pos ? a.pos + (size_t)(row % a.pos_rows) * N + col : nullptr;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float v = gelu(acc[mb][nb][r]);
                    if (P) v += P[nb * 32];
                    Cr[nb * 32] = v;
                }
            }
        }
}

// Raw accumulators of one k slice, token-major P[m][n] (N columns), in the
// layout of epilogue_lift.
template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void epilogue_partial(float* P, int M, int N,
                                                 const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                                 int m0, int n0)
{
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int col = n0 + wn * WTN + (lane & 31);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WTM + mb * 32 + acc_row(lane, r);
            if (row < M) {
                float* Pr = P + (size_t)row * N + col;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) Pr[nb * 32] = acc[mb][nb][r];
            }
        }
}

// fp32 operands on v_mfma_f32_32x32x2_f32. LDS holds both tiles k-major:
// As[k][m] (transposed on store) and Bs[k][n], so a half-wave reads 32
// consecutive floats per operand.
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(256) void populate_f32_kernel(GemmArgs a)
{
    constexpr int BK = 16;
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    static_assert(WGM * WGN == 4 && MB >= 1 && NB >= 1, "tile config");
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int HD = a.H * a.D;
    const int m0 = blockIdx.x * BM;
    const int n0 = blockIdx.y * BN;
    const int p = n0 / HD;
    const int col0 = n0 - p * HD;
    const float* __restrict__ E = static_cast<const float*>(a.E);
    const float* __restrict__ W = static_cast<const float*>(a.wt.w[p]);

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int k0 = 0; k0 < a.dm; k0 += BK) {
#pragma unroll
        for (int idx = tid; idx < BM * BK / 4; idx += 256) {
            const int r = idx / (BK / 4), c4 = (idx % (BK / 4)) * 4;
            const int m = m0 + r;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m < a.M) v = *reinterpret_cast<const float4*>(E + (size_t)m * a.dm + k0 + c4);
            As[c4 + 0][r] = v.x;
            As[c4 + 1][r] = v.y;
            As[c4 + 2][r] = v.z;
            As[c4 + 3][r] = v.w;
        }
#pragma unroll
        for (int idx = tid; idx < BK * BN / 4; idx += 256) {
            const int r = idx / (BN / 4), c4 = (idx % (BN / 4)) * 4;
            *reinterpret_cast<float4*>(&Bs[r][c4]) =
                *reinterpret_cast<const float4*>(W + (size_t)(k0 + r) * HD + col0 + c4);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            float av[MB], bv[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) av[mb] = As[kk + (lane >> 5)][wm * WTM + mb * 32 + (lane & 31)];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) bv[nb] = Bs[kk + (lane >> 5)][wn * WTN + nb * 32 + (lane & 31)];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
        }
        __syncthreads();
    }
    epilogue<BM, BN, WGM, WGN, float>(a, acc, m0, p, col0);
}

// bf16 operands on v_mfma_f32_32x32x16_bf16. Each lane feeds 8 consecutive k
// of one row (A) and of one column (B), so LDS holds As[m][k] as loaded and
// Bs[n][k], transposed while storing. Rows are padded by 8 elements.
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(256) void populate_bf16_kernel(GemmArgs a)
{
    constexpr int BK = 32, LDK = BK + 8;
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    static_assert(WGM * WGN == 4 && MB >= 1 && NB >= 1, "tile config");
    __shared__ __attribute__((aligned(16))) uint16_t As[BM][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int HD = a.H * a.D;
    const int m0 = blockIdx.x * BM;
    const int n0 = blockIdx.y * BN;
    const int p = n0 / HD;
    const int col0 = n0 - p * HD;
    const uint16_t* __restrict__ E = static_cast<const uint16_t*>(a.E);
    const uint16_t* __restrict__ W = static_cast<const uint16_t*>(a.wt.w[p]);

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int k0 = 0; k0 < a.dm; k0 += BK) {
#pragma unroll
        for (int idx = tid; idx < BM * BK / 8; idx += 256) {
            const int r = idx / (BK / 8), c8 = (idx % (BK / 8)) * 8;
            const int m = m0 + r;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (m < a.M) v = *reinterpret_cast<const uint4*>(E + (size_t)m * a.dm + k0 + c8);
            *reinterpret_cast<uint4*>(&As[r][c8]) = v;
        }
#pragma unroll
        for (int idx = tid; idx < BK * BN / 8; idx += 256) {
            const int r = idx / (BN / 8), c8 = (idx % (BN / 8)) * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(W + (size_t)(k0 + r) * HD + col0 + c8);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Bs[c8 + 2 * j][r] = (uint16_t)(w4[j] & 0xffffu);
                Bs[c8 + 2 * j + 1][r] = (uint16_t)(w4[j] >> 16);
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 av[MB], bv[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                av[mb] = *reinterpret_cast<const bf16x8*>(&As[wm * WTM + mb * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                bv[nb] = *reinterpret_cast<const bf16x8*>(&Bs[wn * WTN + nb * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
        }
        __syncthreads();
    }
    epilogue<BM, BN, WGM, WGN, uint16_t>(a, acc, m0, p, col0);
}

// Large bf16 tiles: 256 threads as 2x2 waves, each wave a (BM/2)x(BN/2)
// block of 32x32x16 MFMAs (accumulators in AGPRs), BK = 64.
//  * E rows are staged as loaded: As[m][k].
//  * W is [k][n] in memory but a B fragment needs 8 consecutive k of one
//    column, so W is transposed while it is staged: each thread loads an
//    8(k) x 8(n) block (eight 16-byte row pieces), transposes it in registers
//    with v_perm_b32 (two 16-bit halves per output word) and writes eight
//    16-byte column pieces: Bs[n][k]. Both fragments are then one ds_read_b128.
//    Adjacent lanes take adjacent k-chunks of the same 8 columns, so the 16
//    lanes of a write phase cover 16 distinct 16-byte bank slots (rows are
//    BK+8 elements = an odd number of 16-byte slots apart), and each global
//    load instruction still reads 8 full 128-byte row segments.
//  * LDS is double buffered: the next k-tile is loaded into registers while
//    the current one is multiplied, then stored to the other buffer; one
//    barrier per k-tile.
//  * Tiles are ordered in groups of GROUP_M row tiles (a group walks all
//    column tiles) and the linear tile index is dealt to the 8 XCDs in
//    contiguous ranges, so workgroups sharing an XCD's L2 share E rows and
//    W columns.
template <int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void populate_bf16_big_kernel(GemmArgs a, int num_m, int num_n)
{
    constexpr int NT = WGM * WGN * 64;
    constexpr int LDK = BK + 8;
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    constexpr int A_VEC = BM * BK / 8 / NT;           // 16-byte A pieces per thread
    constexpr int B_BLOCKS = (BK / 8) * (BN / 8);      // 8x8 blocks of the W tile
    constexpr int GROUP_M = 8;
    static_assert(MB >= 1 && NB >= 1 && A_VEC >= 1 && BM * BK / 8 % NT == 0, "tile");
    static_assert(B_BLOCKS % NT == 0 || B_BLOCKS < NT, "tile");
    constexpr int B_PER_T = B_BLOCKS >= NT ? B_BLOCKS / NT : 1;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

    const int ntiles = num_m * num_n;
    const int per_xcd = (ntiles + 7) / 8;
    const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (tile >= ntiles) return;
    const int group = tile / (GROUP_M * num_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(num_m - first_m, GROUP_M);
    const int pid_m = first_m + (tile % (GROUP_M * num_n)) % gsize;
    const int pid_n = (tile % (GROUP_M * num_n)) / gsize;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int HD = a.H * a.D;
    const int m0 = pid_m * BM;
    const int n0 = pid_n * BN;
    const int p = n0 / HD;
    const int col0 = n0 - p * HD;
    const uint16_t* __restrict__ E = static_cast<const uint16_t*>(a.E);
    const uint16_t* __restrict__ W = static_cast<const uint16_t*>(a.wt.w[p]);

    uint4 ra[A_VEC];
    uint4 rb[B_PER_T][8];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 8), c8 = (idx % (BK / 8)) * 8;
            const int m = m0 + r;
            ra[i] = m < a.M ? *reinterpret_cast<const uint4*>(E + (size_t)m * a.dm + k0 + c8)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int blk = tid + i * NT;   // block: k-chunk fastest (LDS bank spread)
            if (blk < B_BLOCKS) {
                const int kb8 = blk % (BK / 8), nb8 = blk / (BK / 8);
                const uint16_t* src = W + (size_t)(k0 + kb8 * 8) * HD + col0 + nb8 * 8;
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[i][r] = *reinterpret_cast<const uint4*>(src + (size_t)r * HD);
            }
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 8), c8 = (idx % (BK / 8)) * 8;
            *reinterpret_cast<uint4*>(&As[buf][r * LDK + c8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int blk = tid + i * NT;
            if (blk < B_BLOCKS) {
                const int kb8 = blk % (BK / 8), nb8 = blk / (BK / 8);
                // rows r = k (8 of them), words c = n pairs; output column n
                // holds words kp = (k=2kp, k=2kp+1) of that n
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    uint32_t lo[4], hi[4];
#pragma unroll
                    for (int kp = 0; kp < 4; ++kp) {
                        const uint4& r0 = rb[i][2 * kp];
                        const uint4& r1 = rb[i][2 * kp + 1];
                        const uint32_t a0 = c == 0 ? r0.x : (c == 1 ? r0.y : (c == 2 ? r0.z : r0.w));
                        const uint32_t a1 = c == 0 ? r1.x : (c == 1 ? r1.y : (c == 2 ? r1.z : r1.w));
                        lo[kp] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // n = 2c
                        hi[kp] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // n = 2c + 1
                    }
                    const int n = nb8 * 8 + 2 * c;
                    *reinterpret_cast<uint4*>(&Bs[buf][n * LDK + kb8 * 8]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                    *reinterpret_cast<uint4*>(&Bs[buf][(n + 1) * LDK + kb8 * 8]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                }
            }
        }
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    const int nk = a.dm / BK;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tiles((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 av[MB], bv[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                av[mb] = *reinterpret_cast<const bf16x8*>(
                    &As[buf][(wm * WTM + mb * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                bv[nb] = *reinterpret_cast<const bf16x8*>(
                    &Bs[buf][(wn * WTN + nb * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }
    epilogue<BM, BN, WGM, WGN, uint16_t>(a, acc, m0, p, col0);
}

// fp32 operands on v_mfma_f32_32x32x2_f32 with the same pipeline as the
// fp32 populate as three bf16 products ("bf16x3"): each fp32 operand x is
// split while it is staged into x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi) (both nearest-even; |x - hi - lo| <= 2^-17 |x|), and the
// tile product is hi.hi + hi.lo + lo.hi on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation (the dropped lo.lo term is below 2^-16 of each product). Three
// bf16 MFMAs do the work of 48 fp32 ones (v_mfma_f32_32x32x2_f32), so this
// beats the native fp32 path by several times for products of fp32 size.
// Structure as populate_bf16_big_kernel (register-staged, W transposed while
// staged, double-buffered LDS), with separate hi and lo tiles for both operands:
//  * E: each thread loads 16-byte pieces (4 fp32 of one row) and writes their
//    hi and lo halves (8 bytes each) to Ah[m][k], Al[m][k];
//  * W: each thread loads an 8(k) x 2(n) block (eight 8-byte row pieces) and
//    writes, per column, its 8 k values as one 16-byte hi and one 16-byte lo
//    piece of Bh[n][k], Bl[n][k].
template <int BM, int BN, int BK, int WGM, int WGN, bool LIFT = false>
__global__ __launch_bounds__(WGM * WGN * 64) void populate_f32x3_kernel(GemmArgs a, int num_m, int num_n)
{
    constexpr int NT = WGM * WGN * 64;
    constexpr int LDK = BK + 8;
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    constexpr int A_VEC = BM * BK / 4 / NT;        // 16-byte E pieces per thread
    constexpr int B_BLOCKS = (BK / 8) * (BN / 2);   // 8x2 blocks of the W tile
    constexpr int B_PER = B_BLOCKS >= NT ? B_BLOCKS / NT : 1;
    constexpr int GROUP_M = 8;
    static_assert(MB >= 1 && NB >= 1 && A_VEC >= 1 && (BM * BK / 4) % NT == 0, "tile");
    static_assert(B_BLOCKS % NT == 0 || B_BLOCKS < NT, "W blocks per thread");
    __shared__ __attribute__((aligned(16))) uint16_t Ah[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Al[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bh[2][BN * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bl[2][BN * LDK];

    const int ntiles = num_m * num_n;
    const int per_xcd = (ntiles + 7) / 8;
    const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (tile >= ntiles) return;
    const int group = tile / (GROUP_M * num_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(num_m - first_m, GROUP_M);
    const int pid_m = first_m + (tile % (GROUP_M * num_n)) % gsize;
    const int pid_n = (tile % (GROUP_M * num_n)) / gsize;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int HD = a.H * a.D;
    const int m0 = pid_m * BM;
    const int n0 = pid_n * BN;
    const int p = n0 / HD;
    const int col0 = n0 - p * HD;
    const float* __restrict__ E = static_cast<const float*>(a.E);
    const float* __restrict__ W = static_cast<const float*>(a.wt.w[p]);

    // split two floats into packed bf16 (hi, lo) words
    auto split2 = [](float x0, float x1, uint32_t& hi, uint32_t& lo) {
        const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
        const __bf16 l0 = (__bf16)(x0 - (float)h0), l1 = (__bf16)(x1 - (float)h1);
        hi = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lo = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    };

    float4 ra[A_VEC];
    float2 rb[B_PER][8];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 4), c4 = (idx % (BK / 4)) * 4;
            const int m = m0 + r;
            ra[i] = m < a.M ? *reinterpret_cast<const float4*>(E + (size_t)m * a.dm + k0 + c4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int blk = tid + i * NT;   // block: k-chunk fastest
            if (blk < B_BLOCKS) {
                const int kb8 = blk % (BK / 8), nb2 = blk / (BK / 8);
                const float* src = W + (size_t)(k0 + kb8 * 8) * HD + col0 + nb2 * 2;
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[i][r] = *reinterpret_cast<const float2*>(src + (size_t)r * HD);
            }
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 4), c4 = (idx % (BK / 4)) * 4;
            uint32_t h01, l01, h23, l23;
            split2(ra[i].x, ra[i].y, h01, l01);
            split2(ra[i].z, ra[i].w, h23, l23);
            *reinterpret_cast<uint2*>(&Ah[buf][r * LDK + c4]) = make_uint2(h01, h23);
            *reinterpret_cast<uint2*>(&Al[buf][r * LDK + c4]) = make_uint2(l01, l23);
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int blk = tid + i * NT;
            if (blk < B_BLOCKS) {
                const int kb8 = blk % (BK / 8), nb2 = blk / (BK / 8);
                // column n = nb2*2 + j takes k values rb[i][0..7].{x,y}[j]
                uint32_t h[2][4], l[2][4];
#pragma unroll
                for (int kp = 0; kp < 4; ++kp) {
                    split2(rb[i][2 * kp].x, rb[i][2 * kp + 1].x, h[0][kp], l[0][kp]);
                    split2(rb[i][2 * kp].y, rb[i][2 * kp + 1].y, h[1][kp], l[1][kp]);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = nb2 * 2 + j;
                    *reinterpret_cast<uint4*>(&Bh[buf][n * LDK + kb8 * 8]) =
                        make_uint4(h[j][0], h[j][1], h[j][2], h[j][3]);
                    *reinterpret_cast<uint4*>(&Bl[buf][n * LDK + kb8 * 8]) =
                        make_uint4(l[j][0], l[j][1], l[j][2], l[j][3]);
                }
            }
        }
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    const int nk = a.dm / BK;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tiles((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 ah[MB], al[MB], bh[NB], bl[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int off = (wm * WTM + mb * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5);
                ah[mb] = *reinterpret_cast<const bf16x8*>(&Ah[buf][off]);
                al[mb] = *reinterpret_cast<const bf16x8*>(&Al[buf][off]);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int off = (wn * WTN + nb * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5);
                bh[nb] = *reinterpret_cast<const bf16x8*>(&Bh[buf][off]);
                bl[nb] = *reinterpret_cast<const bf16x8*>(&Bl[buf][off]);
            }
            // one pass over the blocks per product term: consecutive MFMAs
            // write different accumulators (see populate_planes_x3_kernel)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bh[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bl[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bh[nb], acc[mb][nb], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }
    if constexpr (LIFT)
        epilogue_lift<BM, BN, WGM, WGN>(a, acc, m0, n0);
    else
        epilogue<BM, BN, WGM, WGN, float>(a, acc, m0, p, col0);
}

constexpr int vmcnt_wait(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// global_load_lds_dwordx4: each lane's 16 bytes from src land at LDS address
// lds_base + lane*16 (lds_base wave-uniform, through M0). Issued from inline
// assembly so that the compiler neither tracks nor waits on it: the stream
// kernel orders these loads itself with explicit vmcnt waits and barriers.
// An SALU write of M0 needs one wait state before a load that writes LDS
// through it, hence the s_nop. Nothing else in the kernel keeps a value in M0.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
                 "s"(lds_base)
                 : "memory");
}

// One ring slot: A tile then B tile, BK = 32.
template <int BM, int BN>
struct StreamSlot {
    uint16_t a[BM * 32];
    uint16_t b[32 * BN];
};

template <int BM, int BN, int WGM, int WGN>
struct StreamTile {
    static constexpr int BK = 32;
    static constexpr int NT = WGM * WGN * 64;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    static constexpr int A_LD = BM * BK / 8 / NT;   // direct loads per thread per slot
    static constexpr int B_LD = BK * BN / 8 / NT;
    static constexpr int BROW = BN / 8;             // 16-byte pieces per B row
    static_assert((BM * BK / 8) % NT == 0 && (BK * BN / 8) % NT == 0 && MB >= 1 && NB >= 1, "tile");
    static_assert(BROW >= 16, "B swizzle needs >= 16 pieces per row");
};

// Issue the direct loads of k-tile kt into one ring slot.
template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void stream_issue(StreamSlot<BM, BN>& slot, const uint16_t* __restrict__ E,
                                             const uint16_t* __restrict__ W, int kt, int m0, int M,
                                             int dm, int HD, int col0, int wave, int lane)
{
    using T = StreamTile<BM, BN, WGM, WGN>;
    const int k0 = kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
        const int s = (wave * T::A_LD + i) * 64 + lane;   // 16-byte slot in the A tile
        const int row = s >> 2, piece = (s & 3) ^ ((row >> 2) & 3);
        const int m = min(m0 + row, M - 1);
        dma16(E + (size_t)m * dm + k0 + piece * 8, lds_addr(slot.a + (wave * T::A_LD + i) * 64 * 8));
    }
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
        const int s = (wave * T::B_LD + i) * 64 + lane;
        const int row = s / T::BROW, piece = (s % T::BROW) ^ (4 * (row & 3));
        dma16(W + (size_t)(k0 + row) * HD + col0 + piece * 8, lds_addr(slot.b + (wave * T::B_LD + i) * 64 * 8));
    }
}

// Read the fragments of one 16-deep k step of a ring slot for the transposed
// product C^T = W^T E^T: the W side (MFMA A operand, rows = output columns n)
// through ds_read_b64_tr_b16, the E side (MFMA B operand, columns = output
// rows m) as 16-byte row pieces.
template <int BM, int BN, int WGM, int WGN>
struct FragsT {
    bf16x8 w[StreamTile<BM, BN, WGM, WGN>::NB];
    bf16x8 e[StreamTile<BM, BN, WGM, WGN>::MB];
};

template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void read_frags_t(const StreamSlot<BM, BN>& slot, int kk, int wm, int wn, int lane,
                                             FragsT<BM, BN, WGM, WGN>& f)
{
    using T = StreamTile<BM, BN, WGM, WGN>;
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        const int row = wm * T::WTM + mb * 32 + (lane & 31);
        const int piece = ((kk >> 3) + (lane >> 5)) ^ ((row >> 2) & 3);
        f.e[mb] = *reinterpret_cast<const bf16x8*>(slot.a + row * T::BK + piece * 8);
    }
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) {
        const int g = (lane >> 4) & 3, L = lane & 15;
        const int ncol = wn * T::WTN + nb * 32 + 16 * (g & 1) + 4 * (L & 3);
        v4i16_bf h[2];
#pragma unroll
        for (int jr = 0; jr < 2; ++jr) {
            const int krow = kk + 8 * (g >> 1) + 4 * jr + (L >> 2);
            const int piece = (ncol >> 3) ^ (4 * (krow & 3));
            h[jr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(slot.b + krow * BN + piece * 8 + (ncol & 7)));
        }
        bf16x8 b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[j] = __builtin_bit_cast(__bf16, (short)h[0][j]);
            b[4 + j] = __builtin_bit_cast(__bf16, (short)h[1][j]);
        }
        f.w[nb] = b;
    }
}

template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void mfma_frags_t(
    const FragsT<BM, BN, WGM, WGN>& f,
    f32x16 (&acc)[StreamTile<BM, BN, WGM, WGN>::NB][StreamTile<BM, BN, WGM, WGN>::MB])
{
    using T = StreamTile<BM, BN, WGM, WGN>;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
            acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[nb], f.e[mb], acc[nb][mb], 0, 0, 0);
}

// Two floats to packed bf16 (nearest-even), the first in the low half: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Store a transposed accumulator tile (acc[nb][mb] holds C^T: register r of
// lane L is output column n = 8*(r/4) + 4*(L/32) + r%4 and output row
// m = L%32 of its 32x32 block; four consecutive columns of one row lie in one
// head since D is a multiple of 4) through LDS so that global writes are whole rows: for a fixed head the tile's rows
// t .. t+BM-1 of one stream are contiguous in Kc/Vc[l][b][h][t][d], so each
// wave writes 64 x 16 consecutive bytes per store. `stage` is at least
// BM*BN*2 bytes of LDS no wave reads any more; the caller has passed a barrier
// after its last read. Staging layout: [head j][row m][D] bf16, 16-byte pieces
// of a row XOR-swizzled by (m % (D/8)) and the two 8-byte halves of a piece
// swapped when bit 3 of m is set, so that the 8-byte writes of 32 consecutive
// rows and the 16-byte reads of consecutive pieces spread over the banks.
template <int BM, int BN, int WGM, int WGN, int DC = 0>
__device__ __forceinline__ void epilogue_t_lds(
    const GemmArgs& a,
    const f32x16 (&acc)[StreamTile<BM, BN, WGM, WGN>::NB][StreamTile<BM, BN, WGM, WGN>::MB], int m0, int p,
    int col0, int wm, int wn, int lane, uint16_t* stage)
{
    using T = StreamTile<BM, BN, WGM, WGN>;
    constexpr int NT = T::NT;
    // DC: head_dim known at compile time (0: read it from the arguments); with
    // it every staging offset below folds to a per-lane base plus a constant
    const int Dv = DC ? DC : a.D;
    const int lgD = DC ? __builtin_ctz(DC) : __builtin_ctz(a.D);
    const int lgP = lgD - 3;              // log2 of 16-byte pieces per row
    const int PD = 1 << lgP;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = wn * T::WTN + nb * 32 + 8 * g + 4 * (lane >> 5);
            const int j = n >> lgD, d = n & (Dv - 1);
            const int q = d >> 3, half = (d >> 2) & 1;
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb) {
                const int m = wm * T::WTM + mb * 32 + (lane & 31);
                const f32x16& v = acc[nb][mb];
                uint2 w;
                w.x = pack_bf16x2(v[4 * g], v[4 * g + 1]);
                w.y = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
                const int off = ((j * BM + m) << lgD) + ((q ^ (m & (PD - 1))) << 3) +
                                ((half ^ ((m >> 3) & 1)) << 2);
                *reinterpret_cast<uint2*>(stage + off) = w;
            }
        }
    __syncthreads();
    const int l = p < a.L ? p : p - a.L;
    uint16_t* C = static_cast<uint16_t*>(p < a.L ? a.Kc : a.Vc);
    const size_t TD = (size_t)a.T * Dv;
    const int h0 = col0 >> lgD;
    const int b0 = m0 / a.T, t0 = m0 - b0 * a.T;
    const int tid = threadIdx.x;
    // Thread tid always stores 16-byte piece q of its rows m = tid / PD + r * (NT / PD),
    // r < PD, in each of the tile's BN / D heads: one row address per r, then one
    // add per head.
    const int q = tid & (PD - 1);
    const int mstep = NT >> lgP;
    const int heads = BN >> lgD;
    for (int r = 0; r < PD; ++r) {
        const int m = (tid >> lgP) + r * mstep;
        if (m0 + m >= a.M) break;   // m grows with r
        int t = t0 + m, b = b0;
        if (t >= a.T) {
            if (a.T >= BM) { t -= a.T; b += 1; }
            else { b += t / a.T; t -= (t / a.T) * a.T; }
        }
        const int soff = (m << lgD) + ((q ^ (m & (PD - 1))) << 3);
        const bool swap = (m >> 3) & 1;
        uint16_t* dst = C + ((size_t)(l * a.B + b) * a.H + h0) * TD + (size_t)t * Dv + q * 8;
        for (int j = 0; j < heads; ++j) {
            uint4 v = *reinterpret_cast<const uint4*>(stage + soff + ((j * BM) << lgD));
            if (swap) { const uint32_t x = v.x, y = v.y; v.x = v.z; v.y = v.w; v.z = x; v.w = y; }
            *reinterpret_cast<uint4*>(dst + j * TD) = v;
        }
    }
}

// epilogue_t_lds for an fp8 E4M3 cache: each lane's four consecutive columns
// become one 4-byte word (clamped to +-448, nearest-even), staged as
// [head j][row m][D] bytes and written to global memory in 16-byte pieces
// (16 dims of one row). In the staging, the pieces of row m are XOR-swizzled
// by m % (D/16) and the four words of a piece rotated by XOR with
// (m >> 2) % 4, so that the 4-byte writes of 32 consecutive rows spread over
// the banks. `stage` is at least BM*BN bytes, free as for epilogue_t_lds.
template <int BM, int BN, int WGM, int WGN, int DC = 0>
__device__ __forceinline__ void epilogue_t_lds_fp8(
    const GemmArgs& a,
    const f32x16 (&acc)[StreamTile<BM, BN, WGM, WGN>::NB][StreamTile<BM, BN, WGM, WGN>::MB], int m0, int p,
    int col0, int wm, int wn, int lane, uint8_t* stage)
{
    using T = StreamTile<BM, BN, WGM, WGN>;
    constexpr int NT = T::NT;
    const int Dv = DC ? DC : a.D;         // DC as in epilogue_t_lds
    const int lgD = DC ? __builtin_ctz(DC) : __builtin_ctz(a.D);
    const int lgP = lgD - 4;              // log2 of 16-byte pieces per row
    const int PD = 1 << lgP;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = wn * T::WTN + nb * 32 + 8 * g + 4 * (lane >> 5);
            const int j = n >> lgD, d = n & (Dv - 1);
            const int q = d >> 4, wd = (d >> 2) & 3;
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb) {
                const int m = wm * T::WTM + mb * 32 + (lane & 31);
                const f32x16& v = acc[nb][mb];
                const uint32_t w = pack4_fp8(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
                const int off = ((j * BM + m) << lgD) + ((q ^ (m & (PD - 1))) << 4) +
                                ((wd ^ ((m >> 2) & 3)) << 2);
                *reinterpret_cast<uint32_t*>(stage + off) = w;
            }
        }
    __syncthreads();
    const int l = p < a.L ? p : p - a.L;
    uint8_t* C = static_cast<uint8_t*>(p < a.L ? a.Kc : a.Vc);
    const size_t TD = (size_t)a.T * Dv;
    const int h0 = col0 >> lgD;
    const int b0 = m0 / a.T, t0 = m0 - b0 * a.T;
    const int tid = threadIdx.x;
    // as in epilogue_t_lds: piece q of rows m = tid / PD + r * (NT / PD) in every head
    const int q = tid & (PD - 1);
    const int mstep = NT >> lgP;
    const int heads = BN >> lgD;
    for (int r = 0; r < PD; ++r) {
        const int m = (tid >> lgP) + r * mstep;
        if (m0 + m >= a.M) break;   // m grows with r
        int t = t0 + m, b = b0;
        if (t >= a.T) {
            if (a.T >= BM) { t -= a.T; b += 1; }
            else { b += t / a.T; t -= (t / a.T) * a.T; }
        }
        const int soff = (m << lgD) + ((q ^ (m & (PD - 1))) << 4);
        const int rot = (m >> 2) & 3;   // word k of the piece sits at k ^ rot
        uint8_t* dst = C + ((size_t)(l * a.B + b) * a.H + h0) * TD + (size_t)t * Dv + q * 16;
        for (int j = 0; j < heads; ++j) {
            uint4 v = *reinterpret_cast<const uint4*>(stage + soff + ((j * BM) << lgD));
            if (rot & 1) { uint32_t x = v.x; v.x = v.y; v.y = x; x = v.z; v.z = v.w; v.w = x; }
            if (rot & 2) { uint32_t x = v.x; v.x = v.z; v.z = x; x = v.y; v.y = v.w; v.w = x; }
            *reinterpret_cast<uint4*>(dst + j * TD) = v;
        }
    }
}

// bf16 populate for gfx950. Four waves (one per SIMD) each own a 128x128
// block of a 256x256 output tile. The product is formed transposed (W^T as
// the MFMA A operand, E^T as B) so that each lane ends up with four
// consecutive output columns of one row.
//  * operand tiles move global -> LDS with global_load_lds_dwordx4 (each lane's
//    16 bytes land at the instruction's LDS base + lane*16; no staging
//    registers) into a ring of NSLOT slots of BK = 32;
//  * W stays in its [k][n] layout in LDS and its fragments are read with
//    ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
//    i%4 of the 8 bytes addressed by lane 4j + i/4 (j = 0..3), so when four
//    lanes per row address four consecutive k-rows x 16 columns, lane i gets
//    four consecutive k of column i. Two such reads give a 32x32x16 operand;
//  * the 16-byte pieces of each LDS row are XOR-swizzled by row so that
//    fragment reads hit distinct banks: E rows (BK = 32 -> 4 pieces)
//    piece ^ ((row >> 2) & 3); W rows piece ^ 4*(row & 3). The direct loads
//    pick, per lane, the global piece that belongs in the lane's LDS slot;
//  * rows of E past M are clamped to row M-1 for loading; their products
//    only reach output rows that are never stored;
//  * within k-tile s the fragment reads of its second k step are issued
//    before the MFMAs of its first; the barrier that publishes k-tile s+1
//    sits between the two MFMA groups and the first reads of k-tile s+1 are
//    issued right after it, so LDS reads overlap MFMAs across k-tiles;
//  * at the barrier for k-tile s+1 every wave has finished its reads of
//    k-tile s-1 (they fed MFMAs issued before it), so that slot is refilled
//    with k-tile s-1+NSLOT: NSLOT-2 k-tiles are in flight while one is
//    multiplied. A thread waits for its own loads with an explicit vmcnt,
//    the barrier then makes every thread's loads visible;
//  * the finished tile is staged through the ring (epilogue_t_lds, or
//    epilogue_t_lds_fp8 for an fp8 cache) and written as whole rows.
template <int BM, int BN, int NSLOT, bool FP8, int DC = 0>
__global__ __launch_bounds__(256) void populate_bf16_w4_kernel(GemmArgs a, int num_m, int num_n)
{
    static_assert(BM == 256, "the LDS epilogue indexes 256 rows per head block");
    constexpr int WGM = 2, WGN = 2;
    using T = StreamTile<BM, BN, WGM, WGN>;
    using F = FragsT<BM, BN, WGM, WGN>;
    constexpr int LD_PER_SLOT = T::A_LD + T::B_LD;
    static_assert(NSLOT >= 3 && (NSLOT - 2) * LD_PER_SLOT <= 63, "ring depth");
#ifndef CKE_POP_GROUP_M
#define CKE_POP_GROUP_M 8
#endif
    constexpr int GROUP_M = CKE_POP_GROUP_M;
    __shared__ __attribute__((aligned(1024))) StreamSlot<BM, BN> ring[NSLOT];

    const int ntiles = num_m * num_n;
    const int per_xcd = (ntiles + 7) / 8;
    const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (tile >= ntiles) return;
    const int group = tile / (GROUP_M * num_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(num_m - first_m, GROUP_M);
    const int pid_m = first_m + (tile % (GROUP_M * num_n)) % gsize;
    const int pid_n = (tile % (GROUP_M * num_n)) / gsize;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int HD = a.H * a.D;
    const int m0 = pid_m * BM;
    const int n0 = pid_n * BN;
    const int p = n0 / HD;
    const int col0 = n0 - p * HD;
    const uint16_t* __restrict__ E = static_cast<const uint16_t*>(a.E);
    const uint16_t* __restrict__ W = static_cast<const uint16_t*>(a.wt.w[p]);

    f32x16 acc[T::NB][T::MB];
#pragma unroll
    for (int i = 0; i < T::NB; ++i)
#pragma unroll
        for (int j = 0; j < T::MB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = a.dm / T::BK;
    // Before the wait for k-tile j, k-tiles 0..min(j + NSLOT - 3, nk - 1) have
    // been issued (0..NSLOT-2 for j = 0); wait until only the later ones are
    // outstanding, then barrier so that every thread's loads of j are visible.
    auto sync_tile = [&](int j) {
        const int issued = min(j == 0 ? NSLOT - 2 : j + NSLOT - 3, nk - 1);
        const int later = issued - j;
        if (later >= 3)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(3 * LD_PER_SLOT));
        else if (later == 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * LD_PER_SLOT));
        else if (later == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(LD_PER_SLOT));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __builtin_amdgcn_s_barrier();
    };
    static_assert(NSLOT - 2 <= 3, "sync_tile handles up to three k-tiles in flight");

    for (int t = 0; t < NSLOT - 1 && t < nk; ++t)
        stream_issue<BM, BN, WGM, WGN>(ring[t], E, W, t, m0, a.M, a.dm, HD, col0, wave, lane);
    sync_tile(0);
    F cur, nxt;
    read_frags_t<BM, BN, WGM, WGN>(ring[0], 0, wm, wn, lane, cur);
    // The last k-tile is peeled off so that the loop body has no join between
    // the reads for k-tile s+1 and the MFMAs that follow them (a join would
    // make the compiler wait for those reads there).
    int slot = 0;
    for (int s = 0; s + 1 < nk; ++s) {
        read_frags_t<BM, BN, WGM, WGN>(ring[slot], 16, wm, wn, lane, nxt);
        mfma_frags_t<BM, BN, WGM, WGN>(cur, acc);
        const int next_slot = slot + 1 == NSLOT ? 0 : slot + 1;
        sync_tile(s + 1);
        const int t = s - 1 + NSLOT;
        const int fill = slot == 0 ? NSLOT - 1 : slot - 1;
        if (t < nk)
            stream_issue<BM, BN, WGM, WGN>(ring[fill], E, W, t, m0, a.M, a.dm, HD, col0, wave, lane);
        read_frags_t<BM, BN, WGM, WGN>(ring[next_slot], 0, wm, wn, lane, cur);
        mfma_frags_t<BM, BN, WGM, WGN>(nxt, acc);
        slot = next_slot;
    }
    read_frags_t<BM, BN, WGM, WGN>(ring[slot], 16, wm, wn, lane, nxt);
    mfma_frags_t<BM, BN, WGM, WGN>(cur, acc);
    mfma_frags_t<BM, BN, WGM, WGN>(nxt, acc);
    static_assert(NSLOT * sizeof(StreamSlot<BM, BN>) >= BM * BN * 2, "ring too small to stage the tile");
    __syncthreads();
    if constexpr (FP8)
        epilogue_t_lds_fp8<BM, BN, WGM, WGN, DC>(a, acc, m0, p, col0, wm, wn, lane,
                                             reinterpret_cast<uint8_t*>(&ring[0]));
    else
        epilogue_t_lds<BM, BN, WGM, WGN, DC>(a, acc, m0, p, col0, wm, wn, lane,
                                         reinterpret_cast<uint16_t*>(&ring[0]));
}

// ------------------------------------------------- fp32 from split planes
// fp32 products as three bf16 products, with every operand split ONCE into
// bf16 planes hi = bf16(x), lo = bf16(x - hi) (both nearest-even) by a
// prologue into caller workspace, instead of once per tile load: Whisper
// Base's E is read by 24 column tiles and each weight by 12 row tiles, and
// the per-tile split made the fp32 kernel bound by its vector work.
//
// Planes: E (or a lift input x) keeps its layout, [M][K] in both planes;
// each weight W [K][N] is split and transposed to [N][K], so that both
// operands of the product are rows with k contiguous and one loader serves
// both.

// hi/lo planes of n8 groups of 8 consecutive floats (layout kept).
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ x, size_t n8,
                                                         uint16_t* __restrict__ hi,
                                                         uint16_t* __restrict__ lo)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
        const float4 a = reinterpret_cast<const float4*>(x)[2 * i];
        const float4 b = reinterpret_cast<const float4*>(x)[2 * i + 1];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t h[4], l[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const __bf16 h0 = (__bf16)v[2 * j], h1 = (__bf16)v[2 * j + 1];
            const __bf16 l0 = (__bf16)(v[2 * j] - (float)h0), l1 = (__bf16)(v[2 * j + 1] - (float)h1);
            h[j] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
            l[j] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
        reinterpret_cast<uint4*>(hi)[i] = make_uint4(h[0], h[1], h[2], h[3]);
        reinterpret_cast<uint4*>(lo)[i] = make_uint4(l[0], l[1], l[2], l[3]);
    }
}

// Weight j of the table, W [K][N] fp32, to planes [N][K]: hi at
// planes + j*2*N*K, lo N*K elements after it. Grid (N/64, K/64, matrices);
// a 64 x 64 block goes through LDS as packed (hi | lo << 16) words, padded
// rows (65 words) so both the transposed writes and the row reads spread
// over the banks. (A k-blocked layout, a k-tile of consecutive rows in one
// contiguous run, made the product 3x slower: all tiles then read the same
// narrow address window at once.)
__global__ __launch_bounds__(256) void split_transpose_kernel(WeightTable wt, int K, int N,
                                                              uint16_t* __restrict__ planes)
{
    __shared__ uint32_t sh[64 * 65];
    const float* __restrict__ W = static_cast<const float*>(wt.w[blockIdx.z]);
    uint16_t* __restrict__ Wh = planes + (size_t)blockIdx.z * 2 * N * K;
    uint16_t* __restrict__ Wl = Wh + (size_t)N * K;
    const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + i * 256;
        const int k = idx >> 4, c4 = (idx & 15) * 4;
        const float4 v = *reinterpret_cast<const float4*>(W + (size_t)(k0 + k) * N + n0 + c4);
        const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const __bf16 h = (__bf16)f[j];
            const __bf16 l = (__bf16)(f[j] - (float)h);
            sh[(c4 + j) * 65 + k] = (uint32_t)__builtin_bit_cast(uint16_t, h) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
        }
    }
    __syncthreads();
    const int n = tid >> 2, kc = (tid & 3) * 16;
    uint32_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t w0 = sh[n * 65 + kc + 2 * j], w1 = sh[n * 65 + kc + 2 * j + 1];
        h[j] = (w0 & 0xffffu) | (w1 << 16);
        l[j] = (w0 >> 16) | (w1 & 0xffff0000u);
    }
    uint4* dh = reinterpret_cast<uint4*>(Wh + (size_t)(n0 + n) * K + k0 + kc);
    uint4* dl = reinterpret_cast<uint4*>(Wl + (size_t)(n0 + n) * K + k0 + kc);
    dh[0] = make_uint4(h[0], h[1], h[2], h[3]);
    dh[1] = make_uint4(h[4], h[5], h[6], h[7]);
    dl[0] = make_uint4(l[0], l[1], l[2], l[3]);
    dl[1] = make_uint4(l[4], l[5], l[6], l[7]);
}

// One ring slot of the planes product: the hi and lo planes of the E tile
// (BM rows) and of the transposed W tile (BN rows), each row BK k values.
// BK = 32: four 16-byte pieces per row, piece p of row r stored at position
// p ^ ((r >> 2) & 3) so that a fragment read of 32 rows spreads over the
// banks. BK = 16: two pieces per row, swapped in rows with bit 3 set (rows r
// and r + 8 of a fragment read would otherwise hit the same banks: counters
// showed four conflict cycles per read).
template <int BM, int BN, int BK>
struct PlaneSlot {
    uint16_t ah[BM * BK];
    uint16_t al[BM * BK];
    uint16_t bh[BN * BK];
    uint16_t bl[BN * BK];
};

template <int BK>
__device__ __forceinline__ int plane_pos(int row, int piece) {
    if constexpr (BK == 32) return piece ^ ((row >> 2) & 3);
    else return piece ^ ((row >> 3) & 1);
}

// Grid: one workgroup of 4 waves (2 x 2) per BM x BN output tile, tiles in
// the grouped, XCD-ordered sequence of the other populate kernels. Operands
// move global -> LDS with global_load_lds_dwordx4 into a ring of NSLOT slots
// (NSLOT-2 k-tiles in flight while one is multiplied; one barrier per
// k-tile), as in populate_bf16_w4_kernel. Each 16-deep k step multiplies
// lo.hi + hi.lo + hi.hi into fp32 accumulators (small terms first); the
// accumulators are in the layout of epilogue (head-major fp32 stores) and
// epilogue_lift (token-major GELU + positions).
//   Ep: E planes, hi then lo, each [M][K]; Wp: per column block j = n / HD
//   (n / N for the lift), hi and lo planes [HD][K] at Wp + j*2*HD*K.
// 128 x 128 tiles (64 x 64 per wave) suit outputs with few columns; 192 x
// 256 tiles (96 x 128 per wave) stream 40% fewer operand bytes per product
// and cover 1500 memory rows with eight row tiles.
template <int BM, int BN, int BK, int NSLOT, bool LIFT>
__global__ __launch_bounds__(256) void populate_planes_x3_kernel(GemmArgs a, const uint16_t* __restrict__ Ep,
                                                                 const uint16_t* __restrict__ Wp, int K,
                                                                 int num_m, int num_n, int splits,
                                                                 float* __restrict__ part)
{
    constexpr int WGM = 2, WGN = 2;
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    constexpr int PPR = BK / 8;                                  // 16-byte pieces per row
    constexpr int A_BLK = BM * PPR / 64, B_BLK = BN * PPR / 64;   // 64-piece blocks per plane
    constexpr int LPT = (2 * A_BLK + 2 * B_BLK) / 4;              // loads per thread per slot
    constexpr int LD_PER_SLOT = LPT;
    static_assert((BM * PPR) % 64 == 0 && (BN * PPR) % 64 == 0 && (2 * A_BLK + 2 * B_BLK) % 4 == 0,
                  "pieces per slot");
    static_assert(BK == 16 || BK == 32, "k-tile depth");
    static_assert(NSLOT >= 3 && (NSLOT - 2) * LD_PER_SLOT <= 63 && NSLOT - 2 <= 3, "ring depth");
    constexpr int GROUP_M = 8;
    __shared__ __attribute__((aligned(1024))) PlaneSlot<BM, BN, BK> ring[NSLOT];

    // work item = (k slice, tile), slice-major, dealt to the XCDs in
    // contiguous ranges so that one XCD's tiles share panels at the same k
    const int ntiles = num_m * num_n;
    const int per_xcd = (ntiles * splits + 7) / 8;
    const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= ntiles * splits) return;
    const int slice = item / ntiles;
    const int tile = item - slice * ntiles;
    const int k_len = K / splits;                  // a multiple of BK, checked at launch
    const int k_first = slice * k_len;
    const int group = tile / (GROUP_M * num_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(num_m - first_m, GROUP_M);
    const int pid_m = first_m + (tile % (GROUP_M * num_n)) % gsize;
    const int pid_n = (tile % (GROUP_M * num_n)) / gsize;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int HD = a.H * a.D;
    const int m0 = pid_m * BM;
    const int n0 = pid_n * BN;
    const int p = n0 / HD;
    const int col0 = n0 - p * HD;
    const size_t MK = (size_t)a.M * K;
    const uint16_t* __restrict__ Eh = Ep;
    const uint16_t* __restrict__ El = Ep + MK;
    const uint16_t* __restrict__ Wh = Wp + (size_t)p * 2 * HD * K + (size_t)col0 * K;
    const uint16_t* __restrict__ Wl = Wh + (size_t)HD * K;

    // The slot's 16-byte pieces form one list, plane by plane (E hi, E lo,
    // W hi, W lo), dealt to the waves in blocks of 64 (one dma16 each), so
    // every thread issues LPT loads whatever the split between the planes.
    auto issue = [&](PlaneSlot<BM, BN, BK>& slot, int kt) {
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int blk = wave * LPT + j;                      // wave-uniform
            const bool on_a = blk < 2 * A_BLK;
            const int in_plane = on_a ? (blk < A_BLK ? blk : blk - A_BLK)
                                      : (blk - 2 * A_BLK < B_BLK ? blk - 2 * A_BLK : blk - 2 * A_BLK - B_BLK);
            const bool lo = on_a ? blk >= A_BLK : blk - 2 * A_BLK >= B_BLK;
            const int s = in_plane * 64 + lane;
            const int row = s / PPR;
            const int piece = plane_pos<BK>(row, s % PPR);
            const uint16_t* src = on_a ? (lo ? El : Eh) + (size_t)min(m0 + row, a.M - 1) * K
                                       : (lo ? Wl : Wh) + (size_t)row * K;
            uint16_t* dst = on_a ? (lo ? slot.al : slot.ah) : (lo ? slot.bl : slot.bh);
            dma16(src + k_first + kt * BK + piece * 8,
                  __builtin_amdgcn_readfirstlane(lds_addr(dst + in_plane * 64 * 8)));
        }
    };
    struct Frags {
        bf16x8 ah[MB], al[MB], bh[NB], bl[NB];
    };
    auto read = [&](const PlaneSlot<BM, BN, BK>& slot, int kk, Frags& f) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = wm * WTM + mb * 32 + (lane & 31);
            const int piece = plane_pos<BK>(row, (kk >> 3) + (lane >> 5));
            f.ah[mb] = *reinterpret_cast<const bf16x8*>(slot.ah + row * BK + piece * 8);
            f.al[mb] = *reinterpret_cast<const bf16x8*>(slot.al + row * BK + piece * 8);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int row = wn * WTN + nb * 32 + (lane & 31);
            const int piece = plane_pos<BK>(row, (kk >> 3) + (lane >> 5));
            f.bh[nb] = *reinterpret_cast<const bf16x8*>(slot.bh + row * BK + piece * 8);
            f.bl[nb] = *reinterpret_cast<const bf16x8*>(slot.bl + row * BK + piece * 8);
        }
    };
    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // Three passes over the blocks, one per product term, so consecutive
    // MFMAs write different accumulators: three back-to-back products into
    // one accumulator each wait for the previous result, which left the
    // matrix pipe idle for most of every k step.
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.al[mb], f.bh[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[mb], f.bl[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[mb], f.bh[nb], acc[mb][nb], 0, 0, 0);
    };

    const int nk = k_len / BK;
    // before the wait for k-tile j, k-tiles 0..min(j + NSLOT - 3, nk - 1) have
    // been issued (0..NSLOT-2 for j = 0): wait until only the later ones are
    // outstanding, then a barrier makes every thread's loads of j visible
    auto sync_tile = [&](int j) {
        const int issued = min(j == 0 ? NSLOT - 2 : j + NSLOT - 3, nk - 1);
        const int later = issued - j;
        if (later >= 3)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(3 * LD_PER_SLOT));
        else if (later == 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * LD_PER_SLOT));
        else if (later == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(LD_PER_SLOT));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __builtin_amdgcn_s_barrier();
    };
    for (int t = 0; t < NSLOT - 1 && t < nk; ++t) issue(ring[t], t);
    sync_tile(0);
    Frags cur;
    read(ring[0], 0, cur);
    int slot = 0;
    if constexpr (BK == 32) {
        Frags nxt;
        for (int s = 0; s + 1 < nk; ++s) {   // last k-tile peeled: no join before its MFMAs
            read(ring[slot], 16, nxt);
            mma(cur);
            const int next_slot = slot + 1 == NSLOT ? 0 : slot + 1;
            sync_tile(s + 1);
            const int t = s - 1 + NSLOT;
            const int fill = slot == 0 ? NSLOT - 1 : slot - 1;
            if (t < nk) issue(ring[fill], t);
            read(ring[next_slot], 0, cur);
            mma(nxt);
            slot = next_slot;
        }
        read(ring[slot], 16, nxt);
        mma(cur);
        mma(nxt);
    } else {
        // one 16-deep step per k-tile: k-tile s+1 is read right after its
        // barrier and its reads overlap the products of k-tile s; at that
        // barrier every wave has consumed k-tile s-1, whose slot is refilled.
        // Two k-tiles per pass with two fragment buffers that alternate, so
        // no fragment register is written while products still read it.
        Frags nxt;
        auto step = [&](int s, const Frags& have, Frags& next) {
            const int next_slot = slot + 1 == NSLOT ? 0 : slot + 1;
            sync_tile(s + 1);
            const int t = s - 1 + NSLOT;
            const int fill = slot == 0 ? NSLOT - 1 : slot - 1;
            if (t < nk) issue(ring[fill], t);
            read(ring[next_slot], 0, next);
            mma(have);
            slot = next_slot;
        };
        // one exit from the loop: the accumulators keep their registers
        int s = 0;
        while (s + 2 < nk) {
            step(s, cur, nxt);
            step(s + 1, nxt, cur);
            s += 2;
        }
        if (nk - s == 2) {
            step(s, cur, nxt);
            mma(nxt);
        } else {
            mma(cur);
        }
    }
    if constexpr (LIFT) {
        if (part)   // one k slice: raw sums, reduced by lift_reduce_kernel
            epilogue_partial<BM, BN, WGM, WGN>(part + (size_t)slice * a.M * (a.H * a.D), a.M, a.H * a.D,
                                               acc, m0, n0);
        else
            epilogue_lift<BM, BN, WGM, WGN>(a, acc, m0, n0);
    } else {
        epilogue<BM, BN, WGM, WGN, float>(a, acc, m0, p, col0);
    }
}

// out[m][n] = gelu(sum over s of part[s][m][n], s ascending) + pos[m % pos_rows][n]:
// the k slices of a split lift, four consecutive columns per thread.
__global__ __launch_bounds__(256) void lift_reduce_kernel(const float* __restrict__ part, int splits,
                                                          int M, int N, const float* __restrict__ pos,
                                                          int pos_rows, float* __restrict__ out)
{
    const size_t MN = (size_t)M * N;
    const size_t n4 = MN / 4;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        float4 v = reinterpret_cast<const float4*>(part)[i];
        for (int sl = 1; sl < splits; ++sl) {
            const float4 w = reinterpret_cast<const float4*>(part + (size_t)sl * MN)[i];
            v.x += w.x;
            v.y += w.y;
            v.z += w.z;
            v.w += w.w;
        }
        auto gelu = [](float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); };
        v.x = gelu(v.x);
        v.y = gelu(v.y);
        v.z = gelu(v.z);
        v.w = gelu(v.w);
        if (pos) {
            const size_t e = i * 4;
            const int m = (int)(e / N), n = (int)(e - (size_t)m * N);
            const float4 q = *reinterpret_cast<const float4*>(pos + (size_t)(m % pos_rows) * N + n);
            v.x += q.x;
            v.y += q.y;
            v.z += q.z;
            v.w += q.w;
        }
        reinterpret_cast<float4*>(out)[i] = v;
    }
}

// fp32 populate for gfx950 on v_mfma_f32_32x32x2_f32: 64x64 output tiles,
// four waves (2x2) of 32x32. Same scheme as the bf16 kernel, at fp32 widths:
//  * the product is formed transposed, C^T = W^T E^T: lane l's A operand is
//    W[k][n] (n = l%32, k = kk + l/32) and its B operand E[m][k] (m = l%32),
//    so both tiles stay in LDS as loaded and each lane finally holds four
//    consecutive output columns of one row;
//  * operands move global -> LDS with global_load_lds_dwordx4 into a ring of
//    NSLOT slots of BK = 16 or 32 (a 64xBK E tile and a BKx64 W tile,
//    BK/16 16-byte pieces of each per thread), so NSLOT-1 k-tiles are in
//    flight; a thread
//    waits for its own loads with vmcnt, then one barrier per k-tile makes
//    every thread's loads visible. After that barrier every wave has finished
//    k-tile s-1, whose slot is refilled with k-tile s-1+NSLOT;
//  * E rows (BK/4 16-byte pieces) hold global piece p at position
//    p ^ ((m >> 1) & 3) (BK 16) or p ^ (m & 7) (BK 32), W rows
//    (sixteen pieces) at p ^ 8*(k & 1), so the
//    fragment reads of 32 rows / two k-rows spread over the banks;
//  * rows of E past M are clamped to M-1 for loading and never stored;
//  * the finished tile is staged through the ring as [head][row][D] and
//    written as whole rows (a head's 64 rows of one stream are contiguous).
// Requires D <= 64 with 64 % D == 0 (a tile holds whole heads).
template <int NSLOT, int BK, bool LIFT = false>
__global__ __launch_bounds__(256) void populate_f32_dma_kernel(GemmArgs a, int num_m, int num_n)
{
    constexpr int BM = 64, BN = 64, NT = 256, GROUP_M = 8;
    static_assert(BK == 16 || BK == 32, "k-tile");
    constexpr int APR = BK / 4;                // 16-byte pieces per E row
    constexpr int SLOT = BM * BK + BK * BN;   // floats
    constexpr int A_LD = BM * APR / NT, B_LD = BK * (BN / 4) / NT;
    constexpr int LD_PER_SLOT = A_LD + B_LD;   // loads per thread per k-tile
    static_assert(NSLOT >= 2 && (NSLOT - 1) * LD_PER_SLOT <= 63, "ring depth");
    static_assert(NSLOT * SLOT >= BM * BN, "ring too small to stage the tile");
    __shared__ __attribute__((aligned(1024))) float ring[NSLOT * SLOT];

    const int ntiles = num_m * num_n;
    const int per_xcd = (ntiles + 7) / 8;
    const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (tile >= ntiles) return;
    const int group = tile / (GROUP_M * num_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(num_m - first_m, GROUP_M);
    const int pid_m = first_m + (tile % (GROUP_M * num_n)) % gsize;
    const int pid_n = (tile % (GROUP_M * num_n)) / gsize;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int HD = a.H * a.D;
    const int m0 = pid_m * BM;
    const int n0 = pid_n * BN;
    const int p = n0 / HD;
    const int col0 = n0 - p * HD;
    const float* __restrict__ E = static_cast<const float*>(a.E);
    const float* __restrict__ W = static_cast<const float*>(a.wt.w[p]);
    // E row m holds global piece p at LDS position p ^ e_swz(m): the 16-byte
    // reads of eight consecutive rows then hit eight distinct groups of four
    // banks (rows are 64 or 128 bytes, the LDS has 32 banks of 4 bytes)
    auto e_swz = [](int m) { return APR == 4 ? (m >> 1) & 3 : m & 7; };

    // this thread's pieces: E piece tid + i*NT (row x / APR, LDS position
    // x % APR), W piece tid + i*NT (row x / 16)
    const float* a_src[A_LD];
    const float* b_src[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int x = tid + i * NT, row = x / APR, pos = x % APR;
        a_src[i] = E + (size_t)min(m0 + row, a.M - 1) * a.dm + ((pos ^ e_swz(row)) << 2);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int x = tid + i * NT, row = x >> 4, pos = x & 15;
        b_src[i] = W + (size_t)row * HD + col0 + ((pos ^ (8 * (row & 1))) << 2);
    }
    auto issue = [&](int slot, int kt) {
        float* A = ring + slot * SLOT;
        float* B = A + BM * BK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) dma16(a_src[i] + kt * BK, lds_addr(A + (i * NT + wave * 64) * 4));
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            dma16(b_src[i] + (size_t)kt * BK * HD, lds_addr(B + (i * NT + wave * 64) * 4));
    };
    const int nk = a.dm / BK;
    auto sync_tile = [&](int j) {
        const int issued = min(j == 0 ? NSLOT - 1 : j + NSLOT - 2, nk - 1);
        const int later = issued - j;
        if (later >= 3)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(3 * LD_PER_SLOT));
        else if (later == 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * LD_PER_SLOT));
        else if (later == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(LD_PER_SLOT));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __builtin_amdgcn_s_barrier();
    };
    static_assert(NSLOT - 1 <= 3, "sync_tile handles up to three k-tiles in flight");

    // k order inside a k-tile: the two half-waves of an MFMA step take k from
    // separate halves of the tile (step s: k = s for lanes 0-31 and
    // k = BK/2 + s for lanes 32-63; any order is exact as long as both
    // operands follow it). A lane's E values for the whole tile are then BK/2
    // consecutive k of its row: BK/8 16-byte reads instead of BK/2 4-byte ones.
    const int n_l = wn * 32 + (lane & 31);
    const int m_l = wm * 32 + (lane & 31);
    const int kh = lane >> 5;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    for (int t = 0; t < NSLOT && t < nk; ++t) issue(t, t);
    int slot = 0;
    for (int s = 0; s < nk; ++s) {
        sync_tile(s);
        if (s >= 1 && s - 1 + NSLOT < nk) issue(slot == 0 ? NSLOT - 1 : slot - 1, s - 1 + NSLOT);
        const float* A = ring + slot * SLOT;
        const float* B = A + BM * BK;
        float4 ep[BK / 8];
#pragma unroll
        for (int c = 0; c < BK / 8; ++c)
            ep[c] = *reinterpret_cast<const float4*>(A + m_l * BK + (((kh * (BK / 8) + c) ^ e_swz(m_l)) << 2));
#pragma unroll
        for (int st = 0; st < BK / 2; ++st) {
            const int k = kh * (BK / 2) + st;
            const float wv = B[k * BN + (((n_l >> 2) ^ (8 * (k & 1))) << 2) + (n_l & 3)];
            const float4& e4 = ep[st >> 2];
            const float ev = (st & 3) == 0 ? e4.x : (st & 3) == 1 ? e4.y : (st & 3) == 2 ? e4.z : e4.w;
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wv, ev, acc, 0, 0, 0);
        }
        slot = slot + 1 == NSLOT ? 0 : slot + 1;
    }

    if constexpr (LIFT) {
        // memory lift: C is token-major [M][HD]; stage the 64 x 64 tile as
        // rows of 16 pieces XOR-swizzled by row, then write whole rows with
        // the GELU and the window positions applied
        __syncthreads();
        float* stage = ring;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int q = (wn * 32 + 8 * g + 4 * (lane >> 5)) >> 2;
            *reinterpret_cast<float4*>(stage + m_l * BN + ((q ^ (m_l & 15)) << 2)) =
                make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        }
        __syncthreads();
        float* C = static_cast<float*>(a.Kc);
        auto gelu = [](float v) { return 0.5f * v * (1.f + erff(v * 0.70710678118654752f)); };
#pragma unroll 4
        for (int id = tid; id < BM * BN / 4; id += NT) {
            const int m = id >> 4, q = id & 15;
            if (m0 + m < a.M) {
                float4 v = *reinterpret_cast<const float4*>(stage + m * BN + ((q ^ (m & 15)) << 2));
                v = make_float4(gelu(v.x), gelu(v.y), gelu(v.z), gelu(v.w));
                const int col = n0 + 4 * q;
                if (a.pos) {
                    const float4 pv = *reinterpret_cast<const float4*>(
                        a.pos + (size_t)((m0 + m) % a.pos_rows) * HD + col);
                    v.x += pv.x;
                    v.y += pv.y;
                    v.z += pv.z;
                    v.w += pv.w;
                }
                *reinterpret_cast<float4*>(C + (size_t)(m0 + m) * HD + col) = v;
            }
        }
        return;
    }

    // epilogue: stage [head j][row m][D] with 16-byte pieces XOR-swizzled by row
    __syncthreads();
    float* stage = ring;
    const int lgD = __builtin_ctz(a.D);
    const int lgP = lgD - 2;                 // log2 of 16-byte pieces per row
    const int PD = 1 << lgP;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int n = wn * 32 + 8 * g + 4 * (lane >> 5);
        const int j = n >> lgD, d = n & (a.D - 1);
        const int off = ((j * BM + m_l) << lgD) + (((d >> 2) ^ (m_l & (PD - 1))) << 2);
        *reinterpret_cast<float4*>(stage + off) = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2],
                                                              acc[4 * g + 3]);
    }
    __syncthreads();
    const int l = p < a.L ? p : p - a.L;
    float* C = static_cast<float*>(p < a.L ? a.Kc : a.Vc);
    const size_t TD = (size_t)a.T * a.D;
    const int h0 = col0 >> lgD;
    const int b0 = m0 / a.T, t0 = m0 - b0 * a.T;
#pragma unroll 4
    for (int id = tid; id < BM * BN / 4; id += NT) {
        const int q = id & (PD - 1);
        const int m = (id >> lgP) & (BM - 1);
        const int j = id >> (lgP + 6);       // BM == 64 rows per head block
        if (m0 + m < a.M) {
            int t = t0 + m, b = b0;
            if (t >= a.T) {
                if (a.T >= BM) { t -= a.T; b += 1; }
                else { b += t / a.T; t -= (t / a.T) * a.T; }
            }
            const float4 v = *reinterpret_cast<const float4*>(stage + ((j * BM + m) << lgD) +
                                                              ((q ^ (m & (PD - 1))) << 2));
            const size_t idx = ((size_t)(l * a.B + b) * a.H + h0 + j) * TD + (size_t)t * a.D + q * 4;
            *reinterpret_cast<float4*>(C + idx) = v;
        }
    }
}

template <int NSLOT, int BK>
hipError_t launch_f32_dma(const GemmArgs& g, hipStream_t st) {
    const int HD = g.H * g.D;
    const int num_m = (g.M + 63) / 64;
    const int num_n = 2 * g.L * HD / 64;
    const int ntiles = num_m * num_n;
    const int grid = ((ntiles + 7) / 8) * 8;
    hipLaunchKernelGGL((populate_f32_dma_kernel<NSLOT, BK>), dim3(grid), dim3(256), 0, st, g, num_m, num_n);
    return hipGetLastError();
}

template <int BM, int BN, int NSLOT, bool FP8>
hipError_t launch_bf16_w4(const GemmArgs& g, hipStream_t st) {
    const int HD = g.H * g.D;
    const int num_m = (g.M + BM - 1) / BM;
    const int num_n = 2 * g.L * HD / BN;
    const int ntiles = num_m * num_n;
    const int grid = ((ntiles + 7) / 8) * 8;
    if (g.D == 64)   // the common head size: staging offsets fold at compile time
        hipLaunchKernelGGL((populate_bf16_w4_kernel<BM, BN, NSLOT, FP8, 64>), dim3(grid), dim3(256), 0, st,
                           g, num_m, num_n);
    else
        hipLaunchKernelGGL((populate_bf16_w4_kernel<BM, BN, NSLOT, FP8>), dim3(grid), dim3(256), 0, st, g,
                           num_m, num_n);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN>
hipError_t launch_bf16_big(const GemmArgs& g, hipStream_t st) {
    const int HD = g.H * g.D;
    const int num_m = (g.M + BM - 1) / BM;
    const int num_n = 2 * g.L * HD / BN;
    const int ntiles = num_m * num_n;
    const int grid = ((ntiles + 7) / 8) * 8;
    hipLaunchKernelGGL((populate_bf16_big_kernel<BM, BN, BK, WGM, WGN>), dim3(grid),
                       dim3(WGM * WGN * 64), 0, st, g, num_m, num_n);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN>
hipError_t launch_f32x3(const GemmArgs& g, hipStream_t st) {
    const int HD = g.H * g.D;
    const int num_m = (g.M + BM - 1) / BM;
    const int num_n = 2 * g.L * HD / BN;
    const int ntiles = num_m * num_n;
    const int grid = ((ntiles + 7) / 8) * 8;
    hipLaunchKernelGGL((populate_f32x3_kernel<BM, BN, BK, WGM, WGN>), dim3(grid), dim3(WGM * WGN * 64), 0,
                       st, g, num_m, num_n);
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_cfg(const GemmArgs& g, bool bf16, hipStream_t st) {
    const int HD = g.H * g.D;
    dim3 grid((g.M + BM - 1) / BM, 2 * g.L * HD / BN);
    if (bf16)
        hipLaunchKernelGGL((populate_bf16_kernel<BM, BN, WGM, WGN>), grid, dim3(256), 0, st, g);
    else
        hipLaunchKernelGGL((populate_f32_kernel<BM, BN, WGM, WGN>), grid, dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace

// Projector memory lift: out = gelu(x . W) (+ positions), fp32, one weight,
// N = n columns, with a token-major epilogue. Inputs at least 1024 wide run as
// three bf16 products on 128 x 64 tiles (the Q-Former's 1500 x 4096 x 2048:
// 204 us, max error 3e-5, against 248 us on the fp32 kernel; 128 x 128 tiles,
// only 192 of them for 256 compute units, took 257 us). Narrower inputs stay on
// the fp32 DMA kernel, where splitting the operands costs more than it saves.
namespace {
template <int BM, int BN>
hipError_t launch_lift_x3(const GemmArgs& g, int n, hipStream_t st) {
    const int num_m = (g.M + BM - 1) / BM, num_n = n / BN;
    const int grid = ((num_m * num_n + 7) / 8) * 8;
    hipLaunchKernelGGL((populate_f32x3_kernel<BM, BN, 32, 2, 2, true>), dim3(grid), dim3(256), 0, st, g,
                       num_m, num_n);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_lift(const LiftLaunch& a, hipStream_t st) {
    if (a.rows < 1 || a.k_in % 32 != 0 || a.n % 64 != 0 || (a.pos && a.pos_rows < 1))
        return hipErrorInvalidValue;
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.E = a.x;
    g.wt.w[0] = a.w;
    g.Kc = a.out;
    g.M = a.rows;
    g.dm = a.k_in;
    g.T = a.rows;
    g.L = 1;
    g.B = 1;
    g.H = a.n / 64;
    g.D = 64;
    g.pos = a.pos;
    g.pos_rows = a.pos_rows;
    if (a.k_in >= 1024) return launch_lift_x3<128, 64>(g, a.n, st);   // n % 64 == 0 checked above
    const int num_m = (a.rows + 63) / 64, num_n = a.n / 64;
    const int ntiles = num_m * num_n;
    const int grid = ((ntiles + 7) / 8) * 8;
    hipLaunchKernelGGL((populate_f32_dma_kernel<3, 32, true>), dim3(grid), dim3(256), 0, st, g, num_m,
                       num_n);
    return hipGetLastError();
}

namespace {

// Planes workspace: E (or x) hi and lo planes, [M][K] each, then from the
// next 256-byte boundary n_mat weight plane pairs [N][K].
size_t planes_w_offset(long long M, int K) { return ((size_t)(2 * M * K * 2) + 255) / 256 * 256; }

size_t planes_bytes(long long M, int K, int n_mat, int N) {
    return planes_w_offset(M, K) + (size_t)n_mat * 2 * N * K * 2;
}

bool planes_shape_ok(int K, int N) { return K % 64 == 0 && N % 128 == 0; }

#ifndef CKE_PLANES_MIN_BIG_TILES
#define CKE_PLANES_MIN_BIG_TILES 128
#endif


// the rows of E (or x) split into hi and lo planes at Ep: [2][M][K]
hipError_t launch_split_rows(const float* E, long long M, int K, uint16_t* Ep, hipStream_t st) {
    const size_t n8 = (size_t)M * K / 8;
    const size_t blocks = (n8 + 255) / 256;
    const dim3 sgrid((unsigned)(blocks < 4096 ? blocks : 4096));
    hipLaunchKernelGGL(split_rows_kernel, sgrid, dim3(256), 0, st, E, n8, Ep, Ep + (size_t)M * K);
    return hipGetLastError();
}

// A memory lift too small to give most compute units a 192 x 256 tile is
// split over k into 4 or 2 slices of at least 256 each, so that tiles x
// slices stays within one workgroup per compute unit; lift_reduce_kernel
// then adds the slices in order and applies the GELU and the positions.
int lift_splits(long long M, int K, int N) {
    if (N % 256 != 0) return 1;
    const long long tiles = ((M + 191) / 192) * (N / 256);
    if (tiles >= CKE_PLANES_MIN_BIG_TILES) return 1;
    if (tiles * 4 <= 256 && K % 256 == 0 && K / 4 >= 256) return 4;
    if (tiles * 2 <= 256 && K % 128 == 0 && K / 2 >= 256) return 2;
    return 1;
}

size_t lift_partial_bytes(long long M, int K, int N) {
    const int S = lift_splits(M, K, N);
    return S > 1 ? ((size_t)S * M * N * 4 + 255) / 256 * 256 : 0;
}

// the product over split planes: E planes at Ep, weight planes at Wp; a
// split lift's slices go to `part` (lift_partial_bytes)
hipError_t launch_planes_product(GemmArgs g, int K, int N_per_mat, int n_total, bool lift,
                                 const uint16_t* Ep, const uint16_t* Wp, float* part, hipStream_t st) {
    const int S = lift ? lift_splits(g.M, K, n_total) : 1;
    // 192 x 256 tiles stream fewer operand bytes per product, but only pay
    // while they still give most compute units a tile
    const long long tiles_big = (long long)((g.M + 191) / 192) * (n_total / 256);
    const bool big = S > 1 || (N_per_mat % 256 == 0 && tiles_big >= CKE_PLANES_MIN_BIG_TILES);
    const int bm = big ? 192 : 128, bn = big ? 256 : 128;
    const int num_m = (g.M + bm - 1) / bm;
    const int num_n = n_total / bn;
    const int ntiles = num_m * num_n;
    const int grid = ((ntiles * S + 7) / 8) * 8;
    float* p = S > 1 ? part : nullptr;
    if (big) {
        if (lift)
            hipLaunchKernelGGL((populate_planes_x3_kernel<192, 256, 16, 4, true>), dim3(grid),
                               dim3(256), 0, st, g, Ep, Wp, K, num_m, num_n, S, p);
        else
            hipLaunchKernelGGL((populate_planes_x3_kernel<192, 256, 16, 4, false>), dim3(grid),
                               dim3(256), 0, st, g, Ep, Wp, K, num_m, num_n, 1, nullptr);
    } else {
        if (lift)
            hipLaunchKernelGGL((populate_planes_x3_kernel<128, 128, 32, 4, true>), dim3(grid), dim3(256), 0, st,
                               g, Ep, Wp, K, num_m, num_n, 1, nullptr);
        else
            hipLaunchKernelGGL((populate_planes_x3_kernel<128, 128, 32, 4, false>), dim3(grid), dim3(256), 0, st,
                               g, Ep, Wp, K, num_m, num_n, 1, nullptr);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    const size_t n4 = (size_t)g.M * n_total / 4;
    const size_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(lift_reduce_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, st,
                       part, S, g.M, n_total, g.pos, g.pos_rows, static_cast<float*>(g.Kc));
    return hipGetLastError();
}

// split prologue (E rows, then every weight transposed) and the product
hipError_t launch_planes(GemmArgs g, int K, int N_per_mat, int n_mat, int n_total, bool lift,
                         void* ws, hipStream_t st) {
    uint16_t* Ep = static_cast<uint16_t*>(ws);
    uint16_t* Wp = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + planes_w_offset(g.M, K));
    hipError_t e = launch_split_rows(static_cast<const float*>(g.E), g.M, K, Ep, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(split_transpose_kernel, dim3(N_per_mat / 64, K / 64, n_mat), dim3(256), 0, st,
                       g.wt, K, N_per_mat, Wp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + planes_bytes(g.M, K, n_mat, N_per_mat));
    return launch_planes_product(g, K, N_per_mat, n_total, lift, Ep, Wp, part, st);
}

}  // namespace

size_t populate_planes_bytes(const PopulateLaunch& a) {
    if (a.bf16 || a.fp8 || !planes_shape_ok(a.dm, a.H * a.D)) return 0;
    return planes_bytes((long long)a.B * a.T, a.dm, 2 * a.L, a.H * a.D);
}

size_t lift_planes_bytes(const LiftLaunch& a) {
    if (!planes_shape_ok(a.k_in, a.n)) return 0;
    return planes_bytes(a.rows, a.k_in, 1, a.n) + lift_partial_bytes(a.rows, a.k_in, a.n);
}

size_t lift_rows_bytes(const LiftLaunch& a) {
    if (a.rows < 1 || !planes_shape_ok(a.k_in, a.n)) return 0;
    return planes_w_offset(a.rows, a.k_in) + lift_partial_bytes(a.rows, a.k_in, a.n);
}

namespace {

GemmArgs populate_gemm_args(const PopulateLaunch& a) {
    GemmArgs g;
    g.pos = nullptr;
    g.pos_rows = 0;
    g.E = a.E;
    g.wt = a.wt;
    g.Kc = a.Kc;
    g.Vc = a.Vc;
    g.M = a.B * a.T;
    g.dm = a.dm;
    g.T = a.T;
    g.L = a.L;
    g.B = a.B;
    g.H = a.H;
    g.D = a.D;
    return g;
}

GemmArgs lift_gemm_args(const LiftLaunch& a) {
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.E = a.x;
    g.wt.w[0] = a.w;
    g.Kc = a.out;
    g.M = a.rows;
    g.dm = a.k_in;
    g.T = a.rows;
    g.L = 1;
    g.B = 1;
    g.H = a.n / 64;
    g.D = 64;
    g.pos = a.pos;
    g.pos_rows = a.pos_rows;
    return g;
}

}  // namespace

hipError_t launch_populate_planes(const PopulateLaunch& a, void* ws, hipStream_t st) {
    const int HD = a.H * a.D;
    return launch_planes(populate_gemm_args(a), a.dm, HD, 2 * a.L, 2 * a.L * HD, false, ws, st);
}

hipError_t launch_lift_planes(const LiftLaunch& a, void* ws, hipStream_t st) {
    return launch_planes(lift_gemm_args(a), a.k_in, a.n, 1, a.n, true, ws, st);
}

size_t weight_planes_bytes(int n_mat, int K, int N) {
    if (n_mat < 1 || n_mat > 2 * kMaxLayers || K < 1 || N < 1 || !planes_shape_ok(K, N)) return 0;
    return (size_t)n_mat * 2 * N * K * 2;
}

size_t row_planes_bytes(long long M, int K) {
    if (M < 1 || K < 1 || K % 64 != 0) return 0;
    return planes_w_offset(M, K);
}

hipError_t launch_weight_planes(const WeightTable& wt, int n_mat, int K, int N, void* planes,
                                hipStream_t st) {
    hipLaunchKernelGGL(split_transpose_kernel, dim3(N / 64, K / 64, n_mat), dim3(256), 0, st, wt, K, N,
                       static_cast<uint16_t*>(planes));
    return hipGetLastError();
}

hipError_t launch_populate_from_planes(const PopulateLaunch& a, const void* w_planes, void* e_ws,
                                       hipStream_t st) {
    const GemmArgs g = populate_gemm_args(a);
    uint16_t* Ep = static_cast<uint16_t*>(e_ws);
    hipError_t e = launch_split_rows(static_cast<const float*>(a.E), g.M, a.dm, Ep, st);
    if (e != hipSuccess) return e;
    const int HD = a.H * a.D;
    return launch_planes_product(g, a.dm, HD, 2 * a.L * HD, false, Ep,
                                 static_cast<const uint16_t*>(w_planes), nullptr, st);
}

hipError_t launch_lift_from_planes(const LiftLaunch& a, const void* w_planes, void* e_ws, hipStream_t st) {
    const GemmArgs g = lift_gemm_args(a);
    uint16_t* Ep = static_cast<uint16_t*>(e_ws);
    hipError_t e = launch_split_rows(a.x, g.M, a.k_in, Ep, st);
    if (e != hipSuccess) return e;
    float* part = reinterpret_cast<float*>(static_cast<char*>(e_ws) + planes_w_offset(g.M, a.k_in));
    return launch_planes_product(g, a.k_in, a.n, a.n, true, Ep, static_cast<const uint16_t*>(w_planes),
                                 part, st);
}

hipError_t launch_populate(const PopulateLaunch& a, hipStream_t st) {
    GemmArgs g;
    g.pos = nullptr;
    g.pos_rows = 0;
    g.E = a.E;
    g.wt = a.wt;
    g.Kc = a.Kc;
    g.Vc = a.Vc;
    g.M = a.B * a.T;
    g.dm = a.dm;
    g.T = a.T;
    g.L = a.L;
    g.B = a.B;
    g.H = a.H;
    g.D = a.D;
    const int HD = a.H * a.D;
#ifndef CKE_POP_W4_SLOTS
#define CKE_POP_W4_SLOTS 4
#endif
    if (a.fp8) {   // only the 256x256 kernel has an fp8 epilogue
        if (HD % 256 == 0 && a.dm % 32 == 0) return launch_bf16_w4<256, 256, CKE_POP_W4_SLOTS, true>(g, st);
        return hipErrorInvalidValue;
    }
    if (a.bf16 && HD % 256 == 0 && a.dm % 32 == 0) return launch_bf16_w4<256, 256, CKE_POP_W4_SLOTS, false>(g, st);
    if (a.bf16 && HD % 128 == 0 && a.dm % 64 == 0) return launch_bf16_big<128, 128, 64, 2, 2>(g, st);
#ifndef CKE_POP_F32X3
#define CKE_POP_F32X3 1
#endif
#ifndef CKE_POP_X3_BM
#define CKE_POP_X3_BM 128
#endif
#ifndef CKE_POP_X3_BK
#define CKE_POP_X3_BK 32
#endif
    if (CKE_POP_F32X3 && !a.bf16 && HD % CKE_POP_X3_BM == 0 && a.dm % CKE_POP_X3_BK == 0)
        return launch_f32x3<CKE_POP_X3_BM, CKE_POP_X3_BM, CKE_POP_X3_BK, 2, 2>(g, st);
#ifndef CKE_POP_F32_DMA
#define CKE_POP_F32_DMA 3
#endif
#ifndef CKE_POP_F32_DMA_BK
#define CKE_POP_F32_DMA_BK 32
#endif
    if (!a.bf16 && HD % 64 == 0 && a.D <= 64 && 64 % a.D == 0 && a.dm % CKE_POP_F32_DMA_BK == 0)
        return launch_f32_dma<CKE_POP_F32_DMA, CKE_POP_F32_DMA_BK>(g, st);
    if (HD % 64 == 0) return launch_cfg<64, 64, 2, 2>(g, a.bf16, st);
    return launch_cfg<128, 32, 4, 1>(g, a.bf16, st);
}

}  // namespace cke
