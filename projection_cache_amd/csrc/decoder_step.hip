// Skinny products of the decoder-layer step on gfx950:
//   Y[s][n] = R[s][n] + sum_k X[s][k] W[k][n]      (R optional)
// for the few rows s of one decode token (one per sequence), with fp32 X, Y, R
// and fp32 or bf16 weights W [K][N] in the y = x.W orientation. One launch
// takes up to three weights that share X (the self-attention Q, K and V
// projections of C-Kernel-Engine's decoder body, "The concept").
//
// These products read every weight element once for a handful of rows
// (0.5-16 FLOP per weight byte), so they are bound by the weight stream, not
// by arithmetic: plain fp32 FMAs on the vector units, no matrix cores.
//
// Work split: a workgroup (8 waves) owns NB = G x 4 columns (G lanes of 4
// columns: 16 bytes of fp32 or 8 bytes of bf16 per lane) of every weight
// row, and all K rows. Its 512/G row groups stride over the rows, each lane
// holding up to 16 rows (12 of fp32) in registers; the first rows are
// requested before X is staged, so
// the two latencies overlap. X (a chunk of SB sequences) is staged in LDS as
// it lies in memory, [s][k], with 16-byte stores; the 4 lanes of a row group
// read it as broadcasts. Row-group partial sums are reduced inside each 16-lane row
// with DPP rotations and across rows and waves through LDS (reusing the X
// space), in a fixed order (deterministic). Column blocks are assigned
// XCD by XCD, so the two 64-byte halves of a 128-byte weight line are read by
// workgroups of one XCD and share its L2.
#include <type_traits>

#include "cke_device.h"
#include "cke_internal.h"

namespace cke {
namespace {

#ifndef CKE_GEMV_G
#define CKE_GEMV_G 4
#endif
constexpr int kGemvG = CKE_GEMV_G;   // lanes across one weight row's column block
constexpr int kGemvThreads = 512;
// weight rows held in registers per lane (fp32 pieces take twice the registers)
template <typename TW> constexpr int gemv_rows() { return sizeof(TW) == 4 ? 12 : 16; }

template <typename TW, int SB>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const float* __restrict__ X,
                                                            GemvOut o0, GemvOut o1, GemvOut o2,
                                                            int S, int K, int N, int nblk)
{
    constexpr int CV = 4;                     // columns per lane (16 B fp32, 8 B bf16)
    constexpr int G = kGemvG;
    constexpr int NB = G * CV;                // columns per workgroup
    constexpr int NT = kGemvThreads;
    constexpr int RG = NT / G;                // row groups per workgroup
    constexpr int NW = NT / 64;
    extern __shared__ float smem[];           // xs [SB][K], later red [4*NW][SB][NB]
    static_assert(G == 1 || G == 2 || G == 4, "row groups are reduced inside 16-lane rows");

    const int per_xcd = (nblk + 7) / 8;
    const int blk = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (blk >= nblk) return;                  // whole workgroup, before any barrier
    const GemvOut o = blockIdx.y == 0 ? o0 : (blockIdx.y == 1 ? o1 : o2);
    const TW* __restrict__ Wc = static_cast<const TW*>(o.W) + (size_t)blk * NB +
                                (threadIdx.x % G) * CV;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = threadIdx.x % G, rg = threadIdx.x / G;
    float* xs = smem;
    float* red = smem;

    // a lane's 4 columns of one weight row: 16 bytes of fp32 or 8 of bf16
    using Piece = typename std::conditional<sizeof(TW) == 4, uint4, uint2>::type;
    constexpr int ROWS = gemv_rows<TW>();
    Piece w[ROWS];
    auto load_rows = [&](int kb) {
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int k = kb + rg + u * RG;
            if (k < K) w[u] = *reinterpret_cast<const Piece*>(Wc + (size_t)k * N);
        }
    };

    for (int s0 = 0; s0 < S; s0 += SB) {
        const int sn = min(SB, S - s0);
        // the first rows of weights do not depend on X: in flight while X is staged
        load_rows(0);
        __syncthreads();   // readers of the previous chunk's LDS are done
        {
            // rows s0.. of X are contiguous: 16-byte loads and stores, up to
            // 16 in flight per thread (K is a multiple of 4); rows past S are
            // zero
            const float4* X4 = reinterpret_cast<const float4*>(X + (size_t)s0 * K);
            float4* xs4 = reinterpret_cast<float4*>(xs);
            const int n4 = sn * K / 4, tot4 = SB * K / 4;
            for (int i0 = threadIdx.x; i0 < tot4; i0 += NT * 16) {
                float4 v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int i = i0 + u * NT;
                    v[u] = i < n4 ? X4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (i0 + u * NT < tot4) xs4[i0 + u * NT] = v[u];
            }
        }
        __syncthreads();
        float acc[SB][CV];
#pragma unroll
        for (int s = 0; s < SB; ++s)
#pragma unroll
            for (int c = 0; c < CV; ++c) acc[s][c] = 0.f;
        for (int kb = 0; kb < K; kb += RG * ROWS) {
            if (kb > 0) load_rows(kb);
#pragma unroll
            for (int u = 0; u < ROWS; ++u) {
                const int k = kb + rg + u * RG;
                if (k < K) {
                    float xv[SB];   // broadcast reads: the 4 lanes of a row group share k
#pragma unroll
                    for (int j = 0; j < SB; ++j) xv[j] = xs[j * K + k];
#pragma unroll
                    for (int c = 0; c < CV; ++c) {
                        float wv;
                        if constexpr (sizeof(TW) == 4) {
                            wv = elem<float>(w[u], c);
                        } else {
                            const uint32_t h = c < 2 ? w[u].x : w[u].y;
                            wv = (c & 1) ? bf16_hi(h) : bf16_lo(h);
                        }
#pragma unroll
                        for (int s = 0; s < SB; ++s) acc[s][c] = fmaf(xv[s], wv, acc[s][c]);
                    }
                }
            }
        }
        __syncthreads();   // every read of xs is done before red reuses the space
        // The 16/G row groups inside each 16-lane row are summed with DPP row
        // rotations by G, 2G, .. 8 lanes, which keep a lane's column group;
        // the 4*NW row sums of the workgroup then go through LDS.
#pragma unroll
        for (int s = 0; s < SB; ++s)
#pragma unroll
            for (int c = 0; c < CV; ++c) {
                float v = acc[s][c];
                if constexpr (G <= 1) v += dpp<0x121>(v);   // row_ror:1
                if constexpr (G <= 2) v += dpp<0x122>(v);   // row_ror:2
                v += dpp<0x124>(v);                         // row_ror:4
                v += dpp<0x128>(v);                         // row_ror:8
                acc[s][c] = v;
            }
        if ((lane & 15) < G) {
            const int row = wave * 4 + (lane >> 4);
#pragma unroll
            for (int s = 0; s < SB; ++s)
#pragma unroll
                for (int c = 0; c < CV; ++c) red[(row * SB + s) * NB + g * CV + c] = acc[s][c];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < sn * NB; i += NT) {
            const int s = i / NB, col = i - s * NB;
            float v = red[s * NB + col];
#pragma unroll
            for (int r = 1; r < 4 * NW; ++r) v += red[(r * SB + s) * NB + col];
            const size_t idx = (size_t)(s0 + s) * N + (size_t)blk * NB + col;
            if (o.R) v += o.R[idx];
            o.Y[idx] = v;
        }
    }
}

template <typename TW, int SB>
hipError_t launch_gemv_sb(const GemvLaunch& a, hipStream_t st) {
    const int nblk = a.N / gemv_cols_per_block(a.bf16);
    const int grid = ((nblk + 7) / 8) * 8;
    const size_t lds = gemv_lds_bytes(SB, a.K, a.bf16);
    hipLaunchKernelGGL((gemv_kernel<TW, SB>), dim3(grid, a.n_out), dim3(kGemvThreads), lds, st, a.X, a.o[0],
                       a.o[1], a.o[2], a.S, a.K, a.N, nblk);
    return hipGetLastError();
}

template <typename TW>
hipError_t launch_gemv_t(const GemvLaunch& a, hipStream_t st) {
    switch (gemv_rows_per_pass(a.S, a.K, a.bf16)) {
        case 1: return launch_gemv_sb<TW, 1>(a, st);
        case 2: return launch_gemv_sb<TW, 2>(a, st);
        case 4: return launch_gemv_sb<TW, 4>(a, st);
        case 8: return launch_gemv_sb<TW, 8>(a, st);
        case 16: return launch_gemv_sb<TW, 16>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int gemv_cols_per_block(bool) { return kGemvG * 4; }

size_t gemv_lds_bytes(int sb, int K, bool bf16) {
    const size_t xs = (size_t)K * sb;
    const size_t red = (size_t)4 * (kGemvThreads / 64) * sb * gemv_cols_per_block(bf16);
    return (xs > red ? xs : red) * sizeof(float);
}

// LDS a workgroup may take on the current device (the smaller of
// kGemvMaxLds and what the runtime reports).
static size_t gemv_lds_limit() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v <= 0)
        return 64 * 1024;
    return (size_t)v < kGemvMaxLds ? (size_t)v : kGemvMaxLds;
}

// Sequences per pass over the weights: the smallest power of two covering S,
// at most 16, and small enough for the staged X chunk and the reduction
// buffer to fit the LDS limit; 0 if not even one row fits.
int gemv_rows_per_pass(int S, int K, bool bf16) {
    const size_t lim = gemv_lds_limit();
    int sb = 1;
    while (sb < S && sb < 16) sb *= 2;
    while (sb >= 1 && gemv_lds_bytes(sb, K, bf16) > lim) sb /= 2;
    return sb;
}

hipError_t launch_gemv(const GemvLaunch& a, hipStream_t st) {
    if (a.n_out < 1 || a.n_out > 3 || a.N % gemv_cols_per_block(a.bf16) != 0 ||
        gemv_rows_per_pass(a.S, a.K, a.bf16) < 1)
        return hipErrorInvalidValue;
    return a.bf16 ? launch_gemv_t<uint16_t>(a, st) : launch_gemv_t<float>(a, st);
}

}  // namespace cke
