// Internal launch descriptors shared by the C-ABI layer and the kernel files.
// Host-visible only; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cke {

constexpr int kMaxLayers = 128;

struct XattnLaunch {
    const float* q;
    const void* K;       // layer slab base, [B][H][T][D]
    const void* V;
    float* out;
    float* part;         // workspace: split partials [B][max_q][H][nsplit][D+2]
    int B, H, T, D, nq, max_q, nsplit, chunk;
    int n_whole;         // (stream, head) pairs 0 .. n_whole-1 run unsplit, one workgroup each
                         // (a multiple of 8); the rest are split nsplit ways
    float scale;
    int dtype;           // CKE_F32, CKE_BF16 or CKE_FP8
    bool stream_rows;    // whole cross cache far larger than the MALL: non-temporal row loads
    float* stats;        // nullptr, or fp32 [B][max_q][H][2]: each head's final (max, sum), base 2
    unsigned* tickets;   // nullptr (merge by a second kernel), or B*H zeroed counters of
                         // kTicketBytes each: the split kernel merges in the same launch
};

// One arrival counter per head, each in a 128-byte line of its own.
constexpr size_t kTicketBytes = 128;
#ifndef CKE_CROSS_WAVES
#define CKE_CROSS_WAVES 4
#endif
constexpr int kCrossWaves = CKE_CROSS_WAVES;  // waves per cross-decode workgroup
#ifndef CKE_CROSS_NP_BF16
#define CKE_CROSS_NP_BF16 3
#endif
constexpr int kCrossNP16Rows = CKE_CROSS_NP_BF16;  // row passes per load tile: bf16 rows, one query

// Most split-kernel workgroups the split plan puts on one compute unit when
// there are at least as many (stream, head) pairs as units: as many as a unit
// holds at once, so no workgroup waits for another to finish. Register-limited
// as compiled (4 waves per workgroup, 512 VGPRs per SIMD lane): bf16 rows with
// one query take 80 VGPRs (3-pass tiles), so 6 fit; fp8 rows take 115, so 4.
// Other cases keep 4 (fp32 and multi-query geometries with that many pairs
// were not measured).
inline int cross_units_cap(int elem_bytes, int max_q) {
    return (elem_bytes == 2 && max_q == 1 && kCrossNP16Rows <= 3) ? 6 : 4;
}

// Merge of split partials: merge_lanes(nsplit) lanes (1, 2, 4 or 8) share one
// output, each folding at most kMergePer splits (nsplit <= 64).
constexpr int kMergePer = 8;
inline __host__ __device__ int merge_lanes(int nsplit) {
    return nsplit <= 8 ? 1 : (nsplit <= 16 ? 2 : (nsplit <= 32 ? 4 : 8));
}
// Whether a split decode may merge in its own launch: one pass of the split
// kernel's threads covers every (output, lane) pair, and the partials stay
// under 2 GB (32-bit buffer offsets). Otherwise a second kernel merges.
inline bool merge_in_launch_fits(int nq, int D, int nsplit, long long n_bh, int max_q) {
    return nsplit > 1 && nq * D * merge_lanes(nsplit) <= kCrossWaves * 64 &&
           (size_t)n_bh * max_q * nsplit * (D + 2) * sizeof(float) < ((size_t)1 << 31) - 16;
}

struct SelfLaunch {
    const float* q;
    const float* k_new;
    const float* v_new;
    void* K;             // [S][H][max_pos][D]
    void* V;
    float* out;
    int S, H, D, max_pos, pos;
    float scale;
    bool bf16;
};

// Selected heads for attention-weight output (at most kMaxWeightHeads).
constexpr int kMaxWeightHeads = 32;
struct HeadList {
    int n;
    int h[kMaxWeightHeads];
};

struct WeightsLaunch {
    const float* q;      // [B][nq][H][D]
    const void* K;       // layer slab base, [B][H][T][D]
    const float* stats;  // [B][max_q][H][2] from the decode of the same call
    float* weights;      // [B][nq][T]
    HeadList heads;
    int B, H, T, D, nq, max_q;
    float scale;
    int dtype;           // CKE_F32, CKE_BF16 or CKE_FP8
};

struct PrefillLaunch {
    const float* q;      // [S][n_new][Hq][D]
    const float* k_new;  // [S][n_new][Hkv][D]
    const float* v_new;
    void* K;             // [S][Hkv][max_pos][D]
    void* V;
    float* out;          // [S][n_new][Hq][D]
    int S, Hkv, Hq, D, max_pos, pos, n_new;
    float scale;
    bool bf16;
};

// Pointer table of the 2*L weight matrices: entries [0, L) are WK_0..WK_{L-1},
// entries [L, 2L) are WV_0..WV_{L-1}. Passed by value as a kernel argument.
struct WeightTable {
    const void* w[2 * kMaxLayers];
};

// Memories of at most this many rows are decoded one wave per head, unsplit.
constexpr int kShortMemRows = 64;

// Largest number of key splits a decode call may use.
constexpr int kMaxSplits = 64;
static_assert(kMaxSplits <= 8 * kMergePer, "a merge covers at most 8 lanes of kMergePer splits");

struct PopulateLaunch {
    const void* E;       // [B*T][d_model]
    WeightTable wt;
    void* Kc;            // [L][B][H][T][D]
    void* Vc;
    int L, B, T, dm, H, D;
    bool bf16;           // bf16 E and W (else fp32)
    bool fp8;            // bf16 inputs, fp8 E4M3 cache
};

// Rows of K/V one decode workgroup covers per pass of all its waves.
// Decoder-step products Y = R + X.W^T (decoder_step.hip): up to three
// weights sharing X, each with its own output and optional residual.
struct GemvOut {
    const void* W;       // [N][K] (output-major), fp32 or bf16
    float* Y;            // [S][N]
    const float* R;      // nullptr or [S][N]
};
struct GemvLaunch {
    const float* X;      // [S][K]
    GemvOut o[3];
    int n_out, S, K, N;
    bool bf16;
};
bool gemv_shape_ok(int K, int N);   // K a multiple of 32, N of 16
hipError_t launch_gemv(const GemvLaunch& a, hipStream_t st);

int cross_keys_per_pass(int D, int elem_bytes);

hipError_t launch_xattn_decode(const XattnLaunch& a, hipStream_t st);
// Zero n 32-bit words (a kernel, so that it can sit inside a captured graph).
hipError_t launch_zero_words(unsigned* p, size_t n, hipStream_t st);
// Whether workgroups i and i + 8 of a launch always run on the same XCD on
// the current device (a probe launch on a private stream, synchronised).
// false on any HIP error.
bool probe_xcd_placement();

hipError_t launch_selfattn_append(const SelfLaunch& a, hipStream_t st);
hipError_t launch_selfattn_prefill(const PrefillLaunch& a, hipStream_t st);
hipError_t launch_xattn_weights(const WeightsLaunch& a, hipStream_t st);
hipError_t launch_populate(const PopulateLaunch& a, hipStream_t st);

// Projector memory lift: out[r][j] = gelu(sum_c x[r][c] w[c][j]) + pos[r % pos_rows][j].
struct LiftLaunch {
    const float* x;      // [rows][k_in]
    const float* w;      // [k_in][n]
    const float* pos;    // nullptr or [pos_rows][n]
    float* out;          // [rows][n]
    int rows, k_in, n, pos_rows;
};
hipError_t launch_lift(const LiftLaunch& a, hipStream_t st);

// fp32 products as three bf16 products over operands split once into bf16
// hi/lo planes in caller workspace (a prologue), for widths the planes kernel
// takes (K a multiple of 64, output columns per weight of 128); 0 bytes means
// the shape does not use planes.
size_t populate_planes_bytes(const PopulateLaunch& a);
size_t lift_planes_bytes(const LiftLaunch& a);
hipError_t launch_populate_planes(const PopulateLaunch& a, void* ws, hipStream_t st);
hipError_t launch_lift_planes(const LiftLaunch& a, void* ws, hipStream_t st);

// The same products with the weights split ahead of time: weight planes are
// [n_mat][hi, lo][N][K] bf16 (each fp32 [K][N] weight transposed), the rows
// of E or x are split per call into [hi, lo][M][K] at e_ws. 0 bytes means the
// shape does not use planes.
size_t weight_planes_bytes(int n_mat, int K, int N);
// workspace of launch_lift_from_planes: x's planes, then (a memory lift split
// over k) its partial sums
size_t lift_rows_bytes(const LiftLaunch& a);
size_t row_planes_bytes(long long M, int K);
hipError_t launch_weight_planes(const WeightTable& wt, int n_mat, int K, int N, void* planes,
                                hipStream_t st);
hipError_t launch_populate_from_planes(const PopulateLaunch& a, const void* w_planes, void* e_ws,
                                       hipStream_t st);
hipError_t launch_lift_from_planes(const LiftLaunch& a, const void* w_planes, void* e_ws, hipStream_t st);

}  // namespace cke
