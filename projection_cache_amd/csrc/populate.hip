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

namespace cke {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct GemmArgs {
    const void* E;
    WeightTable wt;
    void* Kc;
    void* Vc;
    int M, dm, T, L, B, H, D;
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
    TOUT* C = static_cast<TOUT*>(p < a.L ? a.Kc : a.Vc);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = col0 + wn * WTN + nb * 32 + (lane & 31);
            const int h = col / a.D, d = col - (col / a.D) * a.D;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WTM + mb * 32 + acc_row(lane, r);
                if (row < a.M) {
                    const int b = row / a.T, t = row - (row / a.T) * a.T;
                    const size_t idx = ((((size_t)l * a.B + b) * a.H + h) * a.T + t) * a.D + d;
                    store_out<TOUT>(C, idx, acc[mb][nb][r]);
                }
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
            const int blk = tid + i * NT;                 // block: n-chunk fastest
            if (blk < B_BLOCKS) {
                const int nb8 = blk % (BN / 8), kb8 = blk / (BN / 8);
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
                const int nb8 = blk % (BN / 8), kb8 = blk / (BN / 8);
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
// bf16 kernel: both tiles staged k-major in LDS (As[k][m] transposed while
// storing, Bs[k][n] as loaded) so a half-wave reads 32 consecutive floats per
// operand; the next k-tile is prefetched into registers during the MFMA loop
// into a second LDS buffer (one barrier per k-tile); same tile order.
template <int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void populate_f32_big_kernel(GemmArgs a, int num_m, int num_n)
{
    constexpr int NT = WGM * WGN * 64;
    constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 32, NB = WTN / 32;
    constexpr int A_VEC = BM * BK / 4 / NT;   // float4 pieces per thread
    constexpr int B_VEC = BK * BN / 4 / NT;
    constexpr int LDM = BM + 4, LDN = BN + 4;
    constexpr int GROUP_M = 8;
    static_assert(MB >= 1 && NB >= 1 && A_VEC >= 1 && B_VEC >= 1, "tile");
    static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "tile");
    __shared__ __attribute__((aligned(16))) float As[2][BK * LDM];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDN];

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

    float4 ra[A_VEC], rb[B_VEC];
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
        for (int i = 0; i < B_VEC; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BN / 4), c4 = (idx % (BN / 4)) * 4;
            rb[i] = *reinterpret_cast<const float4*>(W + (size_t)(k0 + r) * HD + col0 + c4);
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 4), c4 = (idx % (BK / 4)) * 4;
            As[buf][(c4 + 0) * LDM + r] = ra[i].x;
            As[buf][(c4 + 1) * LDM + r] = ra[i].y;
            As[buf][(c4 + 2) * LDM + r] = ra[i].z;
            As[buf][(c4 + 3) * LDM + r] = ra[i].w;
        }
#pragma unroll
        for (int i = 0; i < B_VEC; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BN / 4), c4 = (idx % (BN / 4)) * 4;
            *reinterpret_cast<float4*>(&Bs[buf][r * LDN + c4]) = rb[i];
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
        for (int kk = 0; kk < BK; kk += 2) {
            float av[MB], bv[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                av[mb] = As[buf][(kk + (lane >> 5)) * LDM + wm * WTM + mb * 32 + (lane & 31)];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                bv[nb] = Bs[buf][(kk + (lane >> 5)) * LDN + wn * WTN + nb * 32 + (lane & 31)];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }
    epilogue<BM, BN, WGM, WGN, float>(a, acc, m0, p, col0);
}

template <int BM, int BN, int BK, int WGM, int WGN>
hipError_t launch_f32_big(const GemmArgs& g, hipStream_t st) {
    const int HD = g.H * g.D;
    const int num_m = (g.M + BM - 1) / BM;
    const int num_n = 2 * g.L * HD / BN;
    const int ntiles = num_m * num_n;
    const int grid = ((ntiles + 7) / 8) * 8;
    hipLaunchKernelGGL((populate_f32_big_kernel<BM, BN, BK, WGM, WGN>), dim3(grid),
                       dim3(WGM * WGN * 64), 0, st, g, num_m, num_n);
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

hipError_t launch_populate(const PopulateLaunch& a, hipStream_t st) {
    GemmArgs g;
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
#ifndef CKE_POP_BF16_BM
#define CKE_POP_BF16_BM 256
#endif
#ifndef CKE_POP_BF16_BN
#define CKE_POP_BF16_BN 256
#endif
#ifndef CKE_POP_BF16_BK
#define CKE_POP_BF16_BK 64
#endif
#ifndef CKE_POP_BF16_WGM
#define CKE_POP_BF16_WGM 4
#endif
#ifndef CKE_POP_BF16_WGN
#define CKE_POP_BF16_WGN 2
#endif
    if (a.bf16 && HD % CKE_POP_BF16_BN == 0 && a.dm % CKE_POP_BF16_BK == 0)
        return launch_bf16_big<CKE_POP_BF16_BM, CKE_POP_BF16_BN, CKE_POP_BF16_BK, CKE_POP_BF16_WGM,
                               CKE_POP_BF16_WGN>(g, st);
    if (a.bf16 && HD % 128 == 0 && a.dm % 64 == 0) return launch_bf16_big<128, 128, 64, 2, 2>(g, st);
#ifndef CKE_POP_F32_BM
#define CKE_POP_F32_BM 64
#endif
#ifndef CKE_POP_F32_BN
#define CKE_POP_F32_BN 64
#endif
#ifndef CKE_POP_F32_BK
#define CKE_POP_F32_BK 16
#endif
#ifndef CKE_POP_F32_WGM
#define CKE_POP_F32_WGM 2
#endif
#ifndef CKE_POP_F32_WGN
#define CKE_POP_F32_WGN 2
#endif
    if (!a.bf16 && HD % CKE_POP_F32_BN == 0 && a.dm % CKE_POP_F32_BK == 0)
        return launch_f32_big<CKE_POP_F32_BM, CKE_POP_F32_BN, CKE_POP_F32_BK, CKE_POP_F32_WGM,
                              CKE_POP_F32_WGN>(g, st);
    if (HD % 128 == 0) return launch_cfg<128, 128, 2, 2>(g, a.bf16, st);
    if (HD % 64 == 0) return launch_cfg<64, 64, 2, 2>(g, a.bf16, st);
    return launch_cfg<128, 32, 4, 1>(g, a.bf16, st);
}

}  // namespace cke
