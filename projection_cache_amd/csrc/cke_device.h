// Device-side building blocks shared by the decode kernels (gfx950, wave64).
//
// Attention of one query row against a run of cached K/V rows, computed by a
// single wavefront with a running max and running sum (the online softmax of
// Rabe & Staats, which the WhisperKit case study, section 3, lists as the
// SplitKV attention variant: key chunks keep a running max/sum and are merged).
// Several wavefronts' partial states are merged through LDS, and several
// workgroups' partial states through a workspace (the cross-block merge).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cke {

// exp(x) = 2^(x * log2 e); scores are kept in the base-2 domain so the
// hardware exp2 (v_exp_f32) applies directly.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element storage types: float (fp32), bf16 held as raw uint16_t bits, or
// fp8 E4M3 held as raw uint8_t bits (projection caches only).
template <typename TE> struct ElemTraits;
template <> struct ElemTraits<float> {
    static constexpr int kVec = 4;  // elements per 16-byte lane load
};
template <> struct ElemTraits<uint16_t> {
    static constexpr int kVec = 8;
};
template <> struct ElemTraits<uint8_t> {
    static constexpr int kVec = 16;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest-even bf16 (hardware v_cvt_pk_bf16_f32) and return the bits.
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float round_to_bf16(float x) { return (float)(__bf16)x; }

// A lane's 16-byte share of a cached row is kept packed in registers (4 fp32,
// 8 bf16 or 16 fp8 values) and widened to fp32 only where it is used, so bf16 rows
// cost half the registers of fp32 ones. With STREAM the load is marked
// non-temporal (load_tile issues such rows as buffer loads, see there).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool STREAM = false>
__device__ __forceinline__ uint4 load16(const void* __restrict__ p) {
    if constexpr (STREAM) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

template <typename TE> __device__ __forceinline__ float elem(const uint4& r, int j);
template <> __device__ __forceinline__ float elem<float>(const uint4& r, int j) {
    const uint32_t w = j == 0 ? r.x : (j == 1 ? r.y : (j == 2 ? r.z : r.w));
    return __uint_as_float(w);
}
template <> __device__ __forceinline__ float elem<uint16_t>(const uint4& r, int j) {
    const uint32_t w = (j >> 1) == 0 ? r.x : ((j >> 1) == 1 ? r.y : ((j >> 1) == 2 ? r.z : r.w));
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}
// fp8: the hardware converts the two values of one 16-bit half of a word at
// once (v_cvt_pk_f32_fp8, OCP E4M3 on gfx950); j is a constant after
// unrolling, so the half select is an immediate and the converted pair is
// shared by j and j ^ 1.
template <> __device__ __forceinline__ float elem<uint8_t>(const uint4& r, int j) {
    const int wi = j >> 2;
    const int w = (int)(wi == 0 ? r.x : (wi == 1 ? r.y : (wi == 2 ? r.z : r.w)));
    const auto pr = (j & 2) ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true)
                            : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    return (j & 1) ? pr[1] : pr[0];
}

// fp32 -> fp8 E4M3, nearest-even, after clamping to the largest finite value
// (the hardware conversion turns out-of-range values into NaN). Two values go
// into the low (HI = false) or high 16 bits of `old`.
constexpr float kFp8Max = 448.f;
template <bool HI>
__device__ __forceinline__ int pack2_fp8(float a, float b, int old) {
    a = fminf(fmaxf(a, -kFp8Max), kFp8Max);
    b = fminf(fmaxf(b, -kFp8Max), kFp8Max);
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    return (uint32_t)pack2_fp8<true>(c, d, pack2_fp8<false>(a, b, 0));
}

// The same 16-byte share of the row a self-attention call appends, from its
// fp32 source: load_cur reads the source (16 / sizeof(TE) floats) and
// pack_cur rounds it to the storage type, since attention reads the value as
// stored. Separate steps, so that a kernel can issue the source loads first
// and round the values only after its cache-row loads.
template <typename TE> struct CurRow { float4 f[16 / sizeof(TE) / 4]; };
template <typename TE>
__device__ __forceinline__ CurRow<TE> load_cur(const float* __restrict__ p) {
    CurRow<TE> r;
#pragma unroll
    for (int k = 0; k < (int)(16 / sizeof(TE) / 4); ++k) r.f[k] = reinterpret_cast<const float4*>(p)[k];
    return r;
}
// An empty statement that takes r's registers as in/out operands and clobbers
// memory. Placed after a kernel's cache-row loads it keeps the rounding of r
// below them: the compiler would otherwise hoist that pure arithmetic up to
// the source loads and wait for them there, before any cache-row load.
template <typename TE>
__device__ __forceinline__ void keep_below(CurRow<TE>& r) {
#pragma unroll
    for (int k = 0; k < (int)(16 / sizeof(TE) / 4); ++k)
        asm volatile("" : "+v"(r.f[k].x), "+v"(r.f[k].y), "+v"(r.f[k].z), "+v"(r.f[k].w) : : "memory");
}
template <typename TE> __device__ __forceinline__ uint4 pack_cur(const CurRow<TE>& r);
template <> __device__ __forceinline__ uint4 pack_cur<float>(const CurRow<float>& r) {
    const float4 a = r.f[0];
    return make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w));
}
template <> __device__ __forceinline__ uint4 pack_cur<uint16_t>(const CurRow<uint16_t>& r) {
    const float4 a = r.f[0], b = r.f[1];
    auto pk = [](float lo, float hi) {
        return (uint32_t)to_bf16_bits(lo) | ((uint32_t)to_bf16_bits(hi) << 16);
    };
    return make_uint4(pk(a.x, a.y), pk(a.z, a.w), pk(b.x, b.y), pk(b.z, b.w));
}
template <> __device__ __forceinline__ uint4 pack_cur<uint8_t>(const CurRow<uint8_t>& r) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack4_fp8(r.f[k].x, r.f[k].y, r.f[k].z, r.f[k].w);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Sum over aligned groups of N lanes (N = 1..32) using DPP lane permutes for
// the steps inside a 16-lane row (quad_perm xor 1, xor 2; half-row mirror;
// row mirror) and a bpermute for the step across rows. After the in-row
// steps every lane of a group holds the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group size");
    if constexpr (N >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (N >= 16) v += dpp<0x140>(v); // row_mirror
    if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
    return v;
}

// Butterfly reductions over lane groups of a wave64.
template <int FROM, int TO>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
    for (int m = FROM; m < TO; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}
template <int FROM, int TO>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
    for (int m = FROM; m < TO; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// Geometry of the lane -> (row, dims) mapping for head_dim D and element TE.
// A row of D elements is read by LPK lanes, 16 bytes each; a wave covers KPW
// consecutive rows per pass.
template <int D, typename TE>
struct RowMap {
    static constexpr int kVec = ElemTraits<TE>::kVec;
    static constexpr int kLPK = D / kVec;   // lanes per row
    static constexpr int kKPW = 64 / kLPK;  // rows per wave pass
    static_assert(kLPK >= 1 && kLPK <= 64 && (64 % kLPK) == 0, "bad head_dim");
};

// Running softmax state of one lane group (the LPK lanes sharing a row slot)
// for up to NQ queries: m is the group's running max in the base-2 domain
// (scores pre-multiplied by scale*log2 e), l and acc the sums relative to it.
// wg_share() and wg_combine() combine the groups of a wave and then the waves.
template <int NQ, int VEC>
struct WaveState {
    float m[NQ];
    float l[NQ];
    float acc[NQ][VEC];
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            m[i] = -INFINITY;
            l[i] = 0.f;
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[i][j] = 0.f;
        }
    }
};

// Load NP row passes of K and V starting at row `base` into packed
// registers. Branch-free, so a whole tile is in flight at once: every row
// index is clamped to r_safe (the last row this wave may read from memory);
// rows past it are masked or replaced in compute_tile.
template <int D, typename TE, int NP, bool STREAM = false>
__device__ __forceinline__ void load_tile(const TE* __restrict__ K, const TE* __restrict__ V,
                                          int base, int r_safe, int grp, int sub,
                                          uint4 (&kb)[NP], uint4 (&vb)[NP])
{
    using RM = RowMap<D, TE>;
    if constexpr (STREAM && sizeof(TE) != 2) {
        // fp32 and fp8 rows: buffer loads from the wave-uniform K and V bases,
        // with 32-bit byte offsets (the caller keeps a head's slab under 2 GB),
        // marked non-temporal. Measured on the cross-attention call,
        // alternating on one box: Whisper Base 6.47 us against 6.74 with
        // normal global loads (fp32 rows that stay in the MALL between decode
        // steps; non-temporal global loads had been slower still), Large over
        // an fp8 cache 16.23 against 16.33 us with non-temporal global loads.
        // bf16 rows keep those global loads (the branch below): Large 24.46
        // against 24.73 us with buffer loads.
        constexpr int kPolicyNT = 2;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)K, (short)0, 0x7ffffff0, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)V, (short)0, 0x7ffffff0, 0x00020000);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = min(base + p * RM::kKPW + grp, r_safe);
            const int off = (row * D + sub * RM::kVec) * (int)sizeof(TE);
            const auto k4 = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kPolicyNT);
            const auto v4 = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kPolicyNT);
            kb[p] = make_uint4(k4[0], k4[1], k4[2], k4[3]);
            vb[p] = make_uint4(v4[0], v4[1], v4[2], v4[3]);
        }
    } else {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = min(base + p * RM::kKPW + grp, r_safe);
            const size_t off = (size_t)row * D + sub * RM::kVec;
            kb[p] = load16<STREAM>(K + off);
            vb[p] = load16<STREAM>(V + off);
        }
    }
}

// Fold one loaded tile into the lane group's running softmax state. Each
// group of LPK lanes (one row slot) keeps its own running max, so a tile
// needs no communication across groups; groups are merged once, in
// wave_merge_groups. Lanes of a group hold identical scores and max. Rows past r1 get
// score -inf and a zero V share (their loaded bytes may be anything); the
// row equal to cur_row uses the values ck/cv instead of the loaded ones.
template <int D, typename TE, int NQ, int NP>
__device__ __forceinline__ void compute_tile(int base, int r1, int cur_row, bool has_cur,
                                             const uint4& ck, const uint4& cv, int grp,
                                             const float (&q)[NQ][RowMap<D, TE>::kVec], int nq,
                                             float sl2, const uint4 (&kb)[NP],
                                             const uint4 (&vb)[NP],
                                             WaveState<NQ, RowMap<D, TE>::kVec>& st)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    // every one of the NQ queries is computed, also those past nq (their
    // query vector is zero and their state unused): one straight-line block,
    // so the compiler interleaves the queries' independent reduction and
    // softmax chains instead of running them one after another
    (void)nq;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        {
            float s[NP];
            float mt = -INFINITY;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int row = base + p * KPW + grp;
                const uint4 kr = (has_cur && row == cur_row) ? ck : kb[p];
                float d = 0.f;
#pragma unroll
                for (int j = 0; j < VEC; ++j) d = fmaf(q[i][j], elem<TE>(kr, j), d);
                d = group_sum<LPK>(d);
                s[p] = row < r1 ? d * sl2 : -INFINITY;
                mt = fmaxf(mt, s[p]);
            }
            const float mn = fmaxf(st.m[i], mt);
            const float alpha = mn == -INFINITY ? 1.f : fast_exp2(st.m[i] - mn);
            st.l[i] *= alpha;
#pragma unroll
            for (int j = 0; j < VEC; ++j) st.acc[i][j] *= alpha;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int row = base + p * KPW + grp;
                const uint4 vr = row < r1 ? ((has_cur && row == cur_row) ? cv : vb[p]) : zero;
                const float e = s[p] == -INFINITY ? 0.f : fast_exp2(s[p] - mn);
                st.l[i] += e;
#pragma unroll
                for (int j = 0; j < VEC; ++j) st.acc[i][j] = fmaf(e, elem<TE>(vr, j), st.acc[i][j]);
            }
            st.m[i] = mn;
        }
    }
}

// One wave attends its queries over rows [r0, r1) of K/V (rows D elements
// apart; r0, r1 wave-uniform). Rows are read in tiles of NP passes; the
// loads of the next tile are issued before the current tile is computed
// (register double buffering), so each wave keeps up to 2*NP 16-byte loads
// per operand in flight.
template <int D, typename TE, int NQ, int NP, bool STREAM = false>
__device__ __forceinline__ void wave_attend(
    const TE* __restrict__ K, const TE* __restrict__ V, int r0, int r1,
    const float (&q)[NQ][RowMap<D, TE>::kVec], int nq, float sl2,
    WaveState<NQ, RowMap<D, TE>::kVec>& st)
{
    using RM = RowMap<D, TE>;
    constexpr int LPK = RM::kLPK, KPW = RM::kKPW;
    constexpr int TILE = NP * KPW;
    const int lane = threadIdx.x & 63;
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    if (r0 >= r1) return;

    const uint4 none = make_uint4(0u, 0u, 0u, 0u);
    const int r_safe = r1 - 1;   // last row that may be read
    uint4 ka[NP], va[NP], kb2[NP], vb2[NP];
    load_tile<D, TE, NP, STREAM>(K, V, r0, r_safe, grp, sub, ka, va);
    for (int base = r0; base < r1; base += 2 * TILE) {
        const bool more = base + TILE < r1;
        if (more) load_tile<D, TE, NP, STREAM>(K, V, base + TILE, r_safe, grp, sub, kb2, vb2);
        compute_tile<D, TE, NQ, NP>(base, r1, -1, false, none, none, grp, q, nq, sl2, ka, va, st);
        if (!more) break;
        if (base + 2 * TILE < r1) load_tile<D, TE, NP, STREAM>(K, V, base + 2 * TILE, r_safe, grp, sub, ka, va);
        compute_tile<D, TE, NQ, NP>(base + TILE, r1, -1, false, none, none, grp, q, nq, sl2, kb2, vb2, st);
    }
}

// Fold one row held in registers (ck, cv: this lane's 16-byte shares) into
// the running state, as the row `row` of a one-pass tile whose other rows
// are masked: lane group 0 takes it, every other group sees only masked rows.
template <int D, typename TE, int NQ>
__device__ __forceinline__ void fold_row(int row, const uint4& ck, const uint4& cv, int grp,
                                         const float (&q)[NQ][RowMap<D, TE>::kVec], int nq, float sl2,
                                         WaveState<NQ, RowMap<D, TE>::kVec>& st)
{
    const uint4 zero[1] = {make_uint4(0u, 0u, 0u, 0u)};
    compute_tile<D, TE, NQ, 1>(row, row + 1, row, true, ck, cv, grp, q, nq, sl2, zero, zero, st);
}

// compute_tile for causal groups of queries: query i only sees rows below
// lim[i] (its own causal limit); rows at or past it score -inf for that
// query. Every row of the tile was loaded from [0, max lim) (the caller
// clamps loads there), so a masked row's V share is finite and its weight 0.
template <int D, typename TE, int NQ, int NP>
__device__ __forceinline__ void compute_tile_causal(int base, const int (&lim)[NQ], int grp,
                                                    const float (&q)[NQ][RowMap<D, TE>::kVec],
                                                    int nq, float sl2, const uint4 (&kb)[NP],
                                                    const uint4 (&vb)[NP],
                                                    WaveState<NQ, RowMap<D, TE>::kVec>& st)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    // all NQ queries in straight-line code, as in compute_tile (the caller
    // gives queries past nq a copy of the last query and its limit)
    (void)nq;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        {
            float s[NP];
            float mt = -INFINITY;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int row = base + p * KPW + grp;
                float d = 0.f;
#pragma unroll
                for (int j = 0; j < VEC; ++j) d = fmaf(q[i][j], elem<TE>(kb[p], j), d);
                d = group_sum<LPK>(d);
                s[p] = row < lim[i] ? d * sl2 : -INFINITY;
                mt = fmaxf(mt, s[p]);
            }
            const float mn = fmaxf(st.m[i], mt);
            const float alpha = mn == -INFINITY ? 1.f : fast_exp2(st.m[i] - mn);
            st.l[i] *= alpha;
#pragma unroll
            for (int j = 0; j < VEC; ++j) st.acc[i][j] *= alpha;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float e = s[p] == -INFINITY ? 0.f : fast_exp2(s[p] - mn);
                st.l[i] += e;
#pragma unroll
                for (int j = 0; j < VEC; ++j) st.acc[i][j] = fmaf(e, elem<TE>(vb[p], j), st.acc[i][j]);
            }
            st.m[i] = mn;
        }
    }
}

// One wave attends a causal group of queries over rows [0, max lim): the rows
// are read once for the whole group (register double buffering as in
// wave_attend); query i sees rows below lim[i]. lim is non-decreasing and
// lim[nq-1] is the largest.
template <int D, typename TE, int NQ, int NP>
__device__ __forceinline__ void wave_attend_causal(
    const TE* __restrict__ K, const TE* __restrict__ V, const int (&lim)[NQ],
    const float (&q)[NQ][RowMap<D, TE>::kVec], int nq, float sl2,
    WaveState<NQ, RowMap<D, TE>::kVec>& st)
{
    using RM = RowMap<D, TE>;
    constexpr int LPK = RM::kLPK, KPW = RM::kKPW;
    constexpr int TILE = NP * KPW;
    const int lane = threadIdx.x & 63;
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    int r1 = lim[0];
#pragma unroll
    for (int i = 1; i < NQ; ++i)
        if (i < nq) r1 = max(r1, lim[i]);
    if (r1 <= 0) return;
    const int r_safe = r1 - 1;
    uint4 ka[NP], va[NP], kb2[NP], vb2[NP];
    load_tile<D, TE, NP>(K, V, 0, r_safe, grp, sub, ka, va);
    for (int base = 0; base < r1; base += 2 * TILE) {
        const bool more = base + TILE < r1;
        if (more) load_tile<D, TE, NP>(K, V, base + TILE, r_safe, grp, sub, kb2, vb2);
        compute_tile_causal<D, TE, NQ, NP>(base, lim, grp, q, nq, sl2, ka, va, st);
        if (!more) break;
        if (base + 2 * TILE < r1) load_tile<D, TE, NP>(K, V, base + 2 * TILE, r_safe, grp, sub, ka, va);
        compute_tile_causal<D, TE, NQ, NP>(base + TILE, lim, grp, q, nq, sl2, kb2, vb2, st);
    }
}

// One wave attends a causal group of queries over rows [r0, r1) of a
// self-attention cache during prefill: rows below `pos` come from the cache
// K/V, rows from `pos` on from the fp32 new rows (row pos + i at kn, vn +
// i * new_stride), rounded to the storage type exactly as they are stored, so
// the wave never reads a cache row that this launch writes. Query i sees rows
// below lim[i]; the caller clamps lim to r1. Each part is read in tiles of NP
// passes; the cache part with register double buffering as in wave_attend.
template <int D, typename TE, int NQ, int NP>
__device__ __forceinline__ void wave_attend_causal_span(
    const TE* __restrict__ K, const TE* __restrict__ V, const float* __restrict__ kn,
    const float* __restrict__ vn, size_t new_stride, int pos, int r0, int r1, const int (&lim)[NQ],
    const float (&q)[NQ][RowMap<D, TE>::kVec], int nq, float sl2,
    WaveState<NQ, RowMap<D, TE>::kVec>& st)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    constexpr int TILE = NP * KPW;
    const int lane = threadIdx.x & 63;
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    if (r0 >= r1) return;
    // cache rows [r0, c1): rows at or past c1 in the last tile are masked
    const int c1 = min(r1, pos);
    if (r0 < c1) {
        int lim_c[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) lim_c[i] = min(lim[i], c1);
        const int r_safe = c1 - 1;
        uint4 ka[NP], va[NP], kb2[NP], vb2[NP];
        load_tile<D, TE, NP>(K, V, r0, r_safe, grp, sub, ka, va);
        for (int base = r0; base < c1; base += 2 * TILE) {
            const bool more = base + TILE < c1;
            if (more) load_tile<D, TE, NP>(K, V, base + TILE, r_safe, grp, sub, kb2, vb2);
            compute_tile_causal<D, TE, NQ, NP>(base, lim_c, grp, q, nq, sl2, ka, va, st);
            if (!more) break;
            if (base + 2 * TILE < c1) load_tile<D, TE, NP>(K, V, base + 2 * TILE, r_safe, grp, sub, ka, va);
            compute_tile_causal<D, TE, NQ, NP>(base + TILE, lim_c, grp, q, nq, sl2, kb2, vb2, st);
        }
    }
    // new rows [max(r0, pos), r1), from the fp32 inputs
    for (int base = max(r0, pos); base < r1; base += TILE) {
        uint4 kb[NP], vb[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const size_t i = (size_t)(min(base + p * KPW + grp, r1 - 1) - pos);
            kb[p] = pack_cur<TE>(load_cur<TE>(kn + i * new_stride + sub * VEC));
            vb[p] = pack_cur<TE>(load_cur<TE>(vn + i * new_stride + sub * VEC));
        }
        compute_tile_causal<D, TE, NQ, NP>(base, lim, grp, q, nq, sl2, kb, vb, st);
    }
}

// Merge the row groups of one wave: afterwards every lane holds the wave's
// (max, sum) per query and the wave's unnormalised output for its own dims.
template <int D, typename TE, int NQ>
__device__ __forceinline__ void wave_merge_groups(WaveState<NQ, RowMap<D, TE>::kVec>& st, int nq)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK;
    (void)nq;   // all NQ, as in compute_tile: straight-line code
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        {
            const float M = xor_max<LPK, 64>(st.m[i]);
            const float f = M == -INFINITY ? 0.f : fast_exp2(st.m[i] - M);
            st.m[i] = M;
            st.l[i] = xor_sum<LPK, 64>(st.l[i] * f);
#pragma unroll
            for (int j = 0; j < VEC; ++j) st.acc[i][j] = xor_sum<LPK, 64>(st.acc[i][j] * f);
        }
    }
}

// Merge the NW waves of a workgroup, in two parts. wg_share merges the row
// groups of each wave, leaves every wave's (max, sum, unnormalised output) in
// LDS (wm, wl [NW*NQ], wa [NW*NQ*D]) and ends with a barrier. wg_combine then
// forms, for one query i and dim d,
//   M = max_w m_w,  L = sum_w l_w 2^(m_w - M),  A = sum_w a_w[d] 2^(m_w - M)
// over the waves in ascending order. Each thread that writes (i, d) forms M
// and L itself, so the results leave with no second barrier, and any two
// threads form the same M and L bit for bit.
template <int D, typename TE, int NQ, int NW>
__device__ __forceinline__ void wg_share(WaveState<NQ, RowMap<D, TE>::kVec>& st, int nq,
                                         float* wm, float* wl, float* wa)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    wave_merge_groups<D, TE, NQ>(st, nq);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        if (lane < LPK) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) wa[(w * NQ + i) * D + lane * VEC + j] = st.acc[i][j];
        }
        if (lane == 0) {
            wm[w * NQ + i] = st.m[i];
            wl[w * NQ + i] = st.l[i];
        }
    }
    __syncthreads();
}

template <int D, int NQ, int NW>
__device__ __forceinline__ void wg_combine(const float* wm, const float* wl, const float* wa, int i,
                                           int d, float& M, float& L, float& A)
{
    M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, wm[v * NQ + i]);
    L = 0.f;
    A = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const float f = fast_exp2(wm[v * NQ + i] - M);
        L = fmaf(wl[v * NQ + i], f, L);
        A = fmaf(wa[(v * NQ + i) * D + d], f, A);
    }
}

}  // namespace cke
