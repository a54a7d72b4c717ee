// Decode-time attention kernels for gfx950:
//   * cross-attention of one query token (per stream, up to NQ of them)
//     against one layer slab of the projection cache, split over the memory
//     rows and merged by the last workgroup to finish (C-Kernel-Engine,
//     "Whisper: Trace One Encoder Tensor into Every Decoder Layer", "View 2":
//     query_tokens = 1 against all key_tokens rows, head-major K/V);
//   * fused scatter-append + causal attention over a self-attention KV cache
//     ("Recurrence as feeds", "What it opened": the cache is an explicit input
//     and output and the new row is written with scatter).
//
// Both are HBM-bound streaming kernels (0.5-2.5 FLOP per byte). Each lane
// reads 16 contiguous bytes of a K row and of a V row, a wave reads whole
// rows, and every load of a tile is issued before the arithmetic that uses it.
#include "cke_device.h"
#include "cke_internal.h"

namespace cke {

// ----------------------------------------------------------------- cross
// Grid: (nsplit, H, B). Workgroup `split` covers memory rows
// [split*chunk, min(T, (split+1)*chunk)) of head h of stream b, for all nq
// queries of that stream. With nsplit > 1 each workgroup writes its partial
// (max, sum, acc[D]) per query to `part` and the last one to finish (an
// atomic counter per (b, h)) merges the nsplit partials in ascending split
// order, writes `out` and resets the counter to zero.
template <int D, typename TE, int NQ, int NW, int NP>
__global__ __launch_bounds__(NW * 64) void xattn_decode_kernel(
    const float* __restrict__ q, const TE* __restrict__ Kl, const TE* __restrict__ Vl,
    float* __restrict__ out, float* __restrict__ part, unsigned* __restrict__ counters,
    int nq, int max_q, int H, int T, int nsplit, int chunk, float sl2)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    __shared__ float wm[NW * NQ], wl[NW * NQ], wa[NW * NQ * D];
    __shared__ float sM[NQ], sL[NQ], sA[NQ * D];
    __shared__ int is_last;

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t bh = (size_t)b * H + h;
    const TE* K = Kl + bh * (size_t)T * D;
    const TE* V = Vl + bh * (size_t)T * D;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane % LPK;

    float qr[NQ][VEC];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            qr[i][j] = (i < nq) ? q[(((size_t)b * nq + i) * H + h) * D + sub * VEC + j] : 0.f;
    }

    const int c0 = split * chunk;
    const int c1 = min(T, c0 + chunk);
    const int per_wave = ((c1 - c0 + NW * KPW - 1) / (NW * KPW)) * KPW;
    const int r0 = min(c1, c0 + w * per_wave);
    const int r1 = min(c1, r0 + per_wave);

    WaveState<NQ, VEC> st;
    st.init();
    wave_attend<D, TE, NQ, NP>(K, V, r0, r1, qr, nq, sl2, -1, nullptr, nullptr, st);
    wg_merge<D, TE, NQ, NW>(st, nq, wm, wl, wa, sM, sL, sA);

    if (nsplit == 1) {
        for (int idx = threadIdx.x; idx < nq * D; idx += NW * 64) {
            const int i = idx / D, d = idx % D;
            out[(((size_t)b * nq + i) * H + h) * D + d] = sA[i * D + d] / sL[i];
        }
        return;
    }

    // partial layout [B][max_q][H][nsplit][D+2]: M, L, acc[0..D)
    auto pslot = [&](int i, int s) -> float* {
        return part + ((((size_t)b * max_q + i) * H + h) * nsplit + s) * (D + 2);
    };
    for (int idx = threadIdx.x; idx < nq * D; idx += NW * 64) {
        const int i = idx / D, d = idx % D;
        float* p = pslot(i, split);
        p[2 + d] = sA[i * D + d];
        if (d == 0) { p[0] = sM[i]; p[1] = sL[i]; }
    }
    __threadfence();  // release: partials visible device-wide (all XCD L2s)
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(&counters[bh], 1u);
        is_last = (prev == (unsigned)(nsplit - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();  // acquire: see every other workgroup's partials

    for (int idx = threadIdx.x; idx < nq * D; idx += NW * 64) {
        const int i = idx / D, d = idx % D;
        float M = -INFINITY;
        for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pslot(i, s)[0]);
        float L = 0.f, A = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float* p = pslot(i, s);
            const float f = fast_exp2(p[0] - M);
            L = fmaf(p[1], f, L);
            A = fmaf(p[2 + d], f, A);
        }
        out[(((size_t)b * nq + i) * H + h) * D + d] = A / L;
    }
    if (threadIdx.x == 0) atomicExch(&counters[bh], 0u);
}

// ------------------------------------------------------------------ self
// Grid: (H, S). One workgroup per (sequence, head) owns rows 0..pos of that
// head's cache: it writes row pos from k_new / v_new (rounded to the storage
// type) and attends over rows 0..pos, taking row pos from the fp32 inputs
// rounded the same way rather than re-reading it, so no workgroup ever reads a
// row another one writes. Rows > pos are neither read nor written.
template <int D, typename TE, int NW, int NP>
__global__ __launch_bounds__(NW * 64) void selfattn_append_kernel(
    const float* __restrict__ q, const float* __restrict__ k_new,
    const float* __restrict__ v_new, TE* __restrict__ Kc, TE* __restrict__ Vc,
    float* __restrict__ out, int H, int max_pos, int pos, float sl2)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    __shared__ float wm[NW], wl[NW], wa[NW * D];
    __shared__ float sM[1], sL[1], sA[D];

    const int h = blockIdx.x, s = blockIdx.y;
    const size_t bh = (size_t)s * H + h;
    TE* K = Kc + bh * (size_t)max_pos * D;
    TE* V = Vc + bh * (size_t)max_pos * D;
    const float* kn = k_new + bh * D;
    const float* vn = v_new + bh * D;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane % LPK;

    // scatter the new row
    for (int d = threadIdx.x; d < D; d += NW * 64) {
        if constexpr (sizeof(TE) == 2) {
            K[(size_t)pos * D + d] = to_bf16_bits(kn[d]);
            V[(size_t)pos * D + d] = to_bf16_bits(vn[d]);
        } else {
            K[(size_t)pos * D + d] = kn[d];
            V[(size_t)pos * D + d] = vn[d];
        }
    }

    float qr[1][VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) qr[0][j] = q[bh * D + sub * VEC + j];

    const int n = pos + 1;
    const int per_wave = ((n + NW * KPW - 1) / (NW * KPW)) * KPW;
    const int r0 = min(n, w * per_wave);
    const int r1 = min(n, r0 + per_wave);

    WaveState<1, VEC> st;
    st.init();
    wave_attend<D, TE, 1, NP>(K, V, r0, r1, qr, 1, sl2, pos, kn, vn, st);
    wg_merge<D, TE, 1, NW>(st, 1, wm, wl, wa, sM, sL, sA);
    for (int d = threadIdx.x; d < D; d += NW * 64) out[bh * D + d] = sA[d] / sL[0];
}

// ------------------------------------------------------------- launchers
namespace {

constexpr int kCrossWaves = 4;
constexpr int kSelfWaves = 16;

template <int D, typename TE, int NQ>
hipError_t launch_cross_nq(const XattnLaunch& a, hipStream_t st) {
    constexpr int NP = (sizeof(TE) == 4) ? 4 : 4;
    dim3 grid(a.nsplit, a.H, a.B);
    hipLaunchKernelGGL((xattn_decode_kernel<D, TE, NQ, kCrossWaves, NP>), grid,
                       dim3(kCrossWaves * 64), 0, st, a.q,
                       static_cast<const TE*>(a.K), static_cast<const TE*>(a.V), a.out,
                       a.part, a.counters, a.nq, a.max_q, a.H, a.T, a.nsplit, a.chunk,
                       a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, typename TE>
hipError_t launch_cross_d(const XattnLaunch& a, hipStream_t st) {
    if (a.nq <= 1) return launch_cross_nq<D, TE, 1>(a, st);
    if (a.nq <= 2) return launch_cross_nq<D, TE, 2>(a, st);
    if (a.nq <= 4) return launch_cross_nq<D, TE, 4>(a, st);
    return launch_cross_nq<D, TE, 8>(a, st);
}

template <typename TE>
hipError_t launch_cross_t(const XattnLaunch& a, hipStream_t st) {
    switch (a.D) {
        case 32: return launch_cross_d<32, TE>(a, st);
        case 64: return launch_cross_d<64, TE>(a, st);
        case 128: return launch_cross_d<128, TE>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int D, typename TE>
hipError_t launch_self_d(const SelfLaunch& a, hipStream_t st) {
    dim3 grid(a.H, a.S);
    hipLaunchKernelGGL((selfattn_append_kernel<D, TE, kSelfWaves, 2>), grid,
                       dim3(kSelfWaves * 64), 0, st, a.q, a.k_new, a.v_new,
                       static_cast<TE*>(a.K), static_cast<TE*>(a.V), a.out, a.H,
                       a.max_pos, a.pos, a.scale * kLog2e);
    return hipGetLastError();
}

template <typename TE>
hipError_t launch_self_t(const SelfLaunch& a, hipStream_t st) {
    switch (a.D) {
        case 32: return launch_self_d<32, TE>(a, st);
        case 64: return launch_self_d<64, TE>(a, st);
        case 128: return launch_self_d<128, TE>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int cross_keys_per_pass(int D, int elem_bytes) {
    const int lpk = D * elem_bytes / 16;
    return (64 / lpk) * kCrossWaves;
}

hipError_t launch_xattn_decode(const XattnLaunch& a, hipStream_t st) {
    return a.bf16 ? launch_cross_t<uint16_t>(a, st) : launch_cross_t<float>(a, st);
}

hipError_t launch_selfattn_append(const SelfLaunch& a, hipStream_t st) {
    return a.bf16 ? launch_self_t<uint16_t>(a, st) : launch_self_t<float>(a, st);
}

}  // namespace cke
