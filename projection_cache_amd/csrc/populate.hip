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
    if (HD % 128 == 0) return launch_cfg<128, 128, 2, 2>(g, a.bf16, st);
    if (HD % 64 == 0) return launch_cfg<64, 64, 2, 2>(g, a.bf16, st);
    return launch_cfg<128, 32, 4, 1>(g, a.bf16, st);
}

}  // namespace cke
