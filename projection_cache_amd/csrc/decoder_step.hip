// Skinny products of the decoder-layer step on gfx950:
//   Y[s][n] = R[s][n] + sum_k X[s][k] W[n][k]      (R optional)
// for the few rows s of one decode token (one per sequence), with fp32 X, Y, R
// and fp32 or bf16 weights W [N][K] stored output-major (row n holds output
// n's K input weights, the nn.Linear layout). One launch takes up to three
// weights that share X (the self-attention Q, K and V projections of
// C-Kernel-Engine's decoder body, "The concept").
//
// The products are done on the matrix cores with the sequences as the 16 rows
// of one MFMA tile: v_mfma_f32_16x16x32_bf16 for bf16 weights, with X split
// into two bf16 terms (x = hi + lo, |x - hi - lo| <= 2^-17 |x|, so the sum
// keeps about 16 significant bits of X against bf16's 8), and
// v_mfma_f32_16x16x4_f32 for fp32 weights (exact fp32 products). On the vector
// units the 16 rows x K x N multiply-adds of the largest workload kept each
// workgroup busy for microseconds; here they are a few dozen MFMAs.
//
// Work split: a workgroup (8 waves) owns 16 output columns (one MFMA tile
// wide) and all K; its waves split K. Because row n of W is contiguous in k,
// lane l of an MFMA (column l % 16, k-group l / 16) loads 16 contiguous bytes
// of W (8 bf16 or 4 fp32 k values) and the matching 8 or 4 contiguous values
// of its X row straight from memory, with no LDS staging; the k values a
// lane group holds are the same for both operands, which is all the product
// needs. Every load of a wave is issued before its first MFMA. The 8 waves'
// 16 x 16 partial tiles are summed through LDS in wave order (deterministic)
// and the first 16 x 16 threads add the residual and store. (Measured: two or
// four tiles per workgroup, sharing the X loads, were slower, and 4 or 16
// waves no better than 8.)
#include "cke_device.h"
#include "cke_internal.h"

namespace cke {
namespace {

#ifndef CKE_GEMV_WAVES
#define CKE_GEMV_WAVES 8
#endif
constexpr int kGemvWaves = CKE_GEMV_WAVES;   // waves per workgroup, splitting K
constexpr int kGemvCols = 16;   // output columns per workgroup (one MFMA tile)
constexpr int kGemvRowsMax = 16;
constexpr int kGemvBatch = 8;   // 16-byte W pieces in flight per lane

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename TW>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_kernel(const float* __restrict__ X,
                                                               GemvOut o0, GemvOut o1,
                                                               GemvOut o2, int S, int K, int N)
{
    constexpr int CKV = 16 / sizeof(TW);   // k values per lane per 16-byte piece
    constexpr int CK = 4 * CKV;            // k values per chunk (4 lane groups)
    __shared__ float red[kGemvWaves][kGemvRowsMax * kGemvCols];

    const GemvOut o = blockIdx.y == 0 ? o0 : (blockIdx.y == 1 ? o1 : o2);
    // Workgroups i and i + 8 run on one XCD. With the column blocks a
    // multiple of 8, class x (workgroups x, x + 8, ...) takes the contiguous
    // x-th eighth of the columns, so for eight heads the columns of head h
    // come out of one XCD, the class the attention calls that read them give
    // head h (its self-attention workgroup and its cross-attention splits);
    // it is the same XCD when the dispatches start their rounds of XCDs
    // alike, which varies.
    const int nblk = gridDim.x;
    const int blk = nblk % 8 == 0 ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
    const int n0 = blk * kGemvCols;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int nch = K / CK;
    const int cpw = (nch + kGemvWaves - 1) / kGemvWaves;
    const int c0 = wave * cpw, c1 = min(nch, c0 + cpw);
    const TW* __restrict__ Wr = static_cast<const TW*>(o.W) + (size_t)(n0 + i) * K + g * CKV;

    for (int s0 = 0; s0 < S; s0 += kGemvRowsMax) {
        const bool row_ok = s0 + i < S;
        const float* __restrict__ Xr = X + (size_t)(s0 + i) * K + g * CKV;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int cb = c0; cb < c1; cb += kGemvBatch) {
            uint4 w[kGemvBatch];
            float4 x[kGemvBatch][CKV / 4];
#pragma unroll
            for (int u = 0; u < kGemvBatch; ++u) {
                const int c = cb + u;
                if (c < c1) {
                    w[u] = load16(Wr + (size_t)c * CK);
#pragma unroll
                    for (int h = 0; h < CKV / 4; ++h)
                        x[u][h] = row_ok ? *reinterpret_cast<const float4*>(Xr + (size_t)c * CK + 4 * h)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int u = 0; u < kGemvBatch; ++u) {
                if (cb + u < c1) {
                    if constexpr (sizeof(TW) == 2) {
                        const float xv[8] = {x[u][0].x, x[u][0].y, x[u][0].z, x[u][0].w,
                                             x[u][1].x, x[u][1].y, x[u][1].z, x[u][1].w};
                        bf16x8 hi, lo;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const __bf16 h = (__bf16)xv[e];
                            hi[e] = h;
                            lo[e] = (__bf16)(xv[e] - (float)h);
                        }
                        const bf16x8 b = __builtin_bit_cast(bf16x8, w[u]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc, 0, 0, 0);
                    } else {
                        const float xv[4] = {x[u][0].x, x[u][0].y, x[u][0].z, x[u][0].w};
                        const float wv[4] = {__uint_as_float(w[u].x), __uint_as_float(w[u].y),
                                             __uint_as_float(w[u].z), __uint_as_float(w[u].w)};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j], wv[j], acc, 0, 0, 0);
                    }
                }
            }
        }
        // lane l holds tile rows 4*(l/16) + r, column l % 16
        __syncthreads();   // the previous pass's readers of red are done
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][(4 * g + r) * kGemvCols + i] = acc[r];
        __syncthreads();
        for (int e = threadIdx.x; e < kGemvRowsMax * kGemvCols; e += kGemvWaves * 64) {   // one pass
            const int s = e / kGemvCols, col = e % kGemvCols;
            if (s0 + s < S) {
                float v = red[0][e];
#pragma unroll
                for (int wv = 1; wv < kGemvWaves; ++wv) v += red[wv][e];
                const size_t idx = (size_t)(s0 + s) * N + n0 + col;
                if (o.R) v += o.R[idx];
                o.Y[idx] = v;
            }
        }
    }
}

template <typename TW>
hipError_t launch_gemv_t(const GemvLaunch& a, hipStream_t st) {
    hipLaunchKernelGGL((gemv_kernel<TW>), dim3(a.N / kGemvCols, a.n_out), dim3(kGemvWaves * 64), 0,
                       st, a.X, a.o[0], a.o[1], a.o[2], a.S, a.K, a.N);
    return hipGetLastError();
}

}  // namespace

bool gemv_shape_ok(int K, int N) { return K > 0 && N > 0 && K % 32 == 0 && N % kGemvCols == 0; }

hipError_t launch_gemv(const GemvLaunch& a, hipStream_t st) {
    if (a.n_out < 1 || a.n_out > 3 || a.S < 1 || !gemv_shape_ok(a.K, a.N)) return hipErrorInvalidValue;
    return a.bf16 ? launch_gemv_t<uint16_t>(a, st) : launch_gemv_t<float>(a, st);
}

}  // namespace cke
