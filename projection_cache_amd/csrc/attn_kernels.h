#pragma once
// Decode-time attention kernels and their launch templates, included by the
// per-element-type translation units attn_f32.hip, attn_bf16.hip and
// attn_fp8.hip (each instantiates its own type, so the three build in
// parallel) and by attn_decode.hip (the type dispatch). Everything here has
// internal linkage: each translation unit owns its instantiations.
//
// Decode-time attention kernels for gfx950:
//   * cross-attention of one query token (per stream, up to NQ of them)
//     against one layer slab of the projection cache, split over the memory
//     rows (xattn_partial_kernel) and merged by a second, small kernel
//     (xattn_merge_kernel), or one wave per head for short memories
//     (xattn_short_kernel) (C-Kernel-Engine, "Whisper: Trace One Encoder
//     Tensor into Every Decoder Layer", "View 2": query_tokens = 1 against all
//     key_tokens rows, head-major K/V);
//   * the softmax weights of selected heads from the decode's own statistics
//     (xattn_weights_kernel; WhisperKit case study, section 6);
//   * fused scatter-append + causal attention over a self-attention KV cache,
//     one row (selfattn_append_kernel) or several rows with grouped kv heads
//     (selfattn_prefill_kernel) ("Recurrence as feeds", "What it opened": the
//     cache is an explicit input and output and the new rows are written with
//     scatter; WhisperKit case study, sections 3 and 4).
//
// All are HBM-bound streaming kernels (0.5-2.5 FLOP per byte). Each lane
// reads 16 contiguous bytes of a K row and of a V row (4 fp32, 8 bf16 or 16
// fp8 values), a wave reads whole rows, and every load of a tile is issued
// before the arithmetic that uses it.
#include "../../include/cke_xattn.h"
#include "cke_device.h"
#include "cke_internal.h"

namespace cke {
namespace {

// ----------------------------------------------------------------- cross
// Combines the nsplit partials of each (query, dim) of head (b, h):
//   M = max_s M_s,  L = sum_s L_s 2^(M_s - M),  out = sum_s A_s 2^(M_s - M) / L
// GL = merge_lanes(nsplit) adjacent lanes share one output o = (query, dim);
// lane g of them takes splits s = g, g+GL, ... (at most kMergePer). It loads
// (M_s, L_s, A_s[d]) of all its splits at once -- clamped, branch-free
// addresses, so the loads cost one memory round trip -- takes their max
// first, so that the exponentials are independent of each other (no chain of
// running-max updates), and sums L_s and A_s scaled by them in ascending s.
// The GL lanes then combine in rounds of lane permutes (DPP), with no LDS and
// no barrier; lane g = 0 writes. The same arithmetic in the
// same order whichever kernel runs it, so both merges give identical bits.
// L2 = true when the partials were written during this same launch by other
// workgroups of this XCD: they are then read with the L1 bypassed (buffer
// loads with sc0), from the XCD's L2. Every lane of a wave runs the loop the
// same number of times (the shuffles need them all).
template <int D, bool L2>
__device__ __forceinline__ void merge_head(const float* __restrict__ part, float* __restrict__ out,
                                           float* __restrict__ stats, int nq, int max_q, int H,
                                           int nsplit, int b, int h, int tid, int nthreads)
{
    const int GL = merge_lanes(nsplit);
    const int total = nq * D * GL;
    const int lane = tid & 63;
    constexpr int kPolicySC0 = 1;
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc((void*)part, (short)0, 0x7ffffff0, 0x00020000);
    for (int base = tid - lane; base < total; base += nthreads) {
        const bool live = base + lane < total;
        const int idx = min(base + lane, total - 1);
        const int o = idx / GL, g = idx % GL;
        const int i = o / D, d = o % D;
        const size_t p0 = (((size_t)b * max_q + i) * H + h) * (size_t)nsplit * (D + 2);
        float pm[kMergePer], pl[kMergePer], pa[kMergePer];
#pragma unroll
        for (int j = 0; j < kMergePer; ++j) {
            const int s = min(g + j * GL, nsplit - 1);
            const size_t w = p0 + (size_t)s * (D + 2);
            if constexpr (L2) {
                const int off = (int)(w * sizeof(float));   // the caller keeps partials under 2 GB
                pm[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, kPolicySC0));
                pl[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, off + 4, 0, kPolicySC0));
                pa[j] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rp, off + (2 + d) * 4, 0, kPolicySC0));
            } else {
                pm[j] = part[w];
                pl[j] = part[w + 1];
                pa[j] = part[w + 2 + d];
            }
        }
        // every lane has split g < GL <= nsplit, and every split has at least
        // one row, so m is finite
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMergePer; ++j)
            if (g + j * GL < nsplit) m = fmaxf(m, pm[j]);
        float l = 0.f, a = 0.f;
#pragma unroll
        for (int j = 0; j < kMergePer; ++j) {
            const float e = (g + j * GL < nsplit) ? fast_exp2(pm[j] - m) : 0.f;
            l = fmaf(pl[j], e, l);
            a = fmaf(pa[j], e, a);
        }
        // combine with the partner lane's (m, l, a): DPP quad permutes for
        // lane distances 1 and 2, the half-row mirror (lane i with 7 - i) to
        // join the two quads of an 8-lane group
        auto join = [&](float m2, float l2, float a2) {
            const float mn = fmaxf(m, m2);
            const float e1 = fast_exp2(m - mn), e2 = fast_exp2(m2 - mn);
            l = fmaf(l, e1, l2 * e2);
            a = fmaf(a, e1, a2 * e2);
            m = mn;
        };
        if (GL >= 2) join(dpp<0xB1>(m), dpp<0xB1>(l), dpp<0xB1>(a));
        if (GL >= 4) join(dpp<0x4E>(m), dpp<0x4E>(l), dpp<0x4E>(a));
        if (GL >= 8) join(dpp<0x141>(m), dpp<0x141>(l), dpp<0x141>(a));
        if (live && g == 0) {
            out[(((size_t)b * nq + i) * H + h) * D + d] = a / l;
            if (stats && d == 0) {
                float* st2 = stats + (((size_t)b * max_q + i) * H + h) * 2;
                st2[0] = m;
                st2[1] = l;
            }
        }
    }
}

// The second launch of a split decode: merges every head from the partials
// the first kernel left in memory. Z workgroups per head each take a
// contiguous share of its (output, lane) pairs; one-dimensional grid of
// 8 * Z * ceil(B*H / 8) workgroups placed like the split kernel's, so that
// the workgroups of head hb share an XCD (the one that wrote that head's
// partials when the two dispatches start their rounds of XCDs alike).
template <int D>
__global__ __launch_bounds__(256) void xattn_merge_kernel(
    const float* __restrict__ part, float* __restrict__ out, float* __restrict__ stats, int nq,
    int max_q, int H, int nsplit, int n_bh, int Z, int n_whole)
{
    const int xcd = blockIdx.x % 8, k_on_xcd = blockIdx.x / 8;
    const int head_slot = k_on_xcd / Z;
    const int z = k_on_xcd - head_slot * Z;
    const int hb = n_whole + xcd + 8 * head_slot;
    if (hb >= n_bh) return;
    merge_head<D, false>(part, out, stats, nq, max_q, H, nsplit, hb / H, hb % H,
                         z * blockDim.x + threadIdx.x, Z * blockDim.x);
}

// Grid: 8 * nsplit * ceil(B*H / 8) workgroups in one dimension. Workgroups i
// and i + 8 run on the same XCD (the dispatcher deals workgroups to the eight
// XCDs in turn; which XCD it starts a dispatch on varies), and every split of
// head hb = b*H + h is placed in class hb % 8, so all splits of a head share
// an XCD. Split s of head hb covers memory rows [s*chunk, min(T, (s+1)*chunk))
// for all nq queries of stream b, so the queries of one stream share every
// K/V read.
// With nsplit == 1 it writes `out` directly; otherwise it writes its partial
// (max, sum, acc[D]) per query to `part`, and the partials are merged:
//
//   * tickets != nullptr: by the last workgroup of the head to finish, in
//     this launch. All splits of a head share one XCD, hence one L2, which is
//     where they meet: each workgroup waits until L2 has acknowledged its
//     partial stores (s_waitcnt vmcnt(0)), then takes a ticket with an atomic
//     add that executes in that L2 (no device-scope bit); the workgroup that
//     draws ticket nsplit-1 resets the counter to 0 for the next call and
//     merges, reading the partials past its L1 (sc0) from the same L2. No
//     workgroup waits for another, and nothing crosses XCDs. This relies on
//     the dispatcher's placement (workgroups i and i + 8 share an XCD), which
//     the host verifies once per device before it passes tickets.
//   * tickets == nullptr: by xattn_merge_kernel, launched next on the same
//     stream, whose workgroups of head hb share an XCD as well (Whisper Base:
//     6.73 against 7.05 us per call with the splits spread over all XCDs).
//     That is not always the XCD that wrote the partials, since each dispatch
//     starts its round of XCDs elsewhere; they cross a kernel boundary and
//     are read correctly either way.
//
// Both merges run merge_head, so they give identical bits. Device-scope
// variants of the in-launch merge were slower than the second launch: a
// release/acquire pair per workgroup is a whole-L2 writeback + invalidate on
// gfx950 (54 us per Whisper Base call), and tagged 64-bit partial words with
// device-scope atomics and a device-scope ticket paid memory round trips on
// the ticket (32 adds serialised where the counter lives) and on the merge's
// loads (8.2 against 6.9 us).
template <int D, typename TE, int NQ, int NW, int NP, bool STREAM>
__global__ __launch_bounds__(NW * 64) void xattn_partial_kernel(
    const float* __restrict__ q, const TE* __restrict__ Kl, const TE* __restrict__ Vl,
    float* __restrict__ out, float* __restrict__ part, float* __restrict__ stats,
    unsigned* __restrict__ tickets, int nq, int max_q, int H, int T, int nsplit, int chunk,
    int n_bh, int n_whole, float sl2)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    __shared__ float wm[NW * NQ], wl[NW * NQ], wa[NW * NQ * D];

    // workgroups 0 .. n_whole-1: pairs 0 .. n_whole-1 whole; then the split
    // pairs, placed by class as above (n_whole is a multiple of 8)
    const int j = (int)blockIdx.x - n_whole;
    const bool whole = j < 0;
    const int xcd = j & 7, k_on_xcd = j >> 3;
    const int head_slot = whole ? 0 : k_on_xcd / nsplit;
    const int split = whole ? 0 : k_on_xcd - head_slot * nsplit;
    const int hb = whole ? (int)blockIdx.x : n_whole + xcd + 8 * head_slot;
    const int ns = whole ? 1 : nsplit;   // splits of this pair
    if (hb >= n_bh) return;   // B*H not a multiple of 8: this XCD has one head fewer
    const int h = hb % H, b = hb / H;
    const size_t bh = (size_t)hb;
    const TE* K = Kl + bh * (size_t)T * D;
    const TE* V = Vl + bh * (size_t)T * D;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int sub = lane % LPK;

    float qr[NQ][VEC];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            qr[i][j] = (i < nq) ? q[(((size_t)b * nq + i) * H + h) * D + sub * VEC + j] : 0.f;
    }

    const int c0 = split * chunk;
    const int c1 = whole ? T : min(T, c0 + chunk);
    const int per_wave = ((c1 - c0 + NW * KPW - 1) / (NW * KPW)) * KPW;
    const int r0 = min(c1, c0 + w * per_wave);
    const int r1 = min(c1, r0 + per_wave);

    WaveState<NQ, VEC> st;
    st.init();
    wave_attend<D, TE, NQ, NP, STREAM>(K, V, r0, r1, qr, nq, sl2, st);
    wg_share<D, TE, NQ, NW>(st, nq, wm, wl, wa);

    // one thread per (query, dim) writes the output (one split) or the
    // partial, layout [B][max_q][H][nsplit][D+2]: M, L, acc[0..D); the
    // thread of dim 0 adds M and L
    for (int idx = threadIdx.x; idx < nq * D; idx += NW * 64) {
        const int i = idx / D, d = idx % D;
        float M, L, A;
        wg_combine<D, NQ, NW>(wm, wl, wa, i, d, M, L, A);
        if (ns == 1) {
            out[(((size_t)b * nq + i) * H + h) * D + d] = A / L;
            if (stats && d == 0) {
                float* st2 = stats + (((size_t)b * max_q + i) * H + h) * 2;
                st2[0] = M;
                st2[1] = L;
            }
        } else {
            float* p = part + ((((size_t)b * max_q + i) * H + h) * nsplit + split) * (D + 2);
            p[2 + d] = A;
            if (d == 0) {
                p[0] = M;
                p[1] = L;
            }
        }
    }
    if (ns == 1 || !tickets) return;
    // this thread's partial stores acknowledged by L2 (the clobber keeps the
    // compiler from moving any store below the wait)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0) {
        unsigned* t = tickets + (size_t)hb * (kTicketBytes / sizeof(unsigned));
        const unsigned n = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int last = n == (unsigned)nsplit - 1u;
        if (last) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    merge_head<D, true>(part, out, stats, nq, max_q, H, nsplit, b, h, threadIdx.x, NW * 64);
}

// Short memories (e.g. 15-frame blocks): one wave per (stream, head), NW of
// them per workgroup, each attending over all T rows on its own, so no
// cross-wave merge and no split. Grid: ceil(B*H / NW).
template <int D, typename TE, int NQ, int NW, int NP>
__global__ __launch_bounds__(NW * 64) void xattn_short_kernel(
    const float* __restrict__ q, const TE* __restrict__ Kl, const TE* __restrict__ Vl,
    float* __restrict__ out, float* __restrict__ stats, int nq, int max_q, int H, int T, int n_bh,
    float sl2)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int bh = blockIdx.x * NW + w;
    if (bh >= n_bh) return;   // whole wave; this kernel has no barrier
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63, sub = lane % LPK;
    const TE* K = Kl + (size_t)bh * T * D;
    const TE* V = Vl + (size_t)bh * T * D;
    float qr[NQ][VEC];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            qr[i][j] = (i < nq) ? q[(((size_t)b * nq + i) * H + h) * D + sub * VEC + j] : 0.f;
    }
    WaveState<NQ, VEC> st;
    st.init();
    wave_attend<D, TE, NQ, NP>(K, V, 0, T, qr, nq, sl2, st);
    wave_merge_groups<D, TE, NQ>(st, nq);
    if (lane < LPK) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            if (i < nq) {
                float* o = out + (((size_t)b * nq + i) * H + h) * D + sub * VEC;
#pragma unroll
                for (int j = 0; j < VEC; ++j) o[j] = st.acc[i][j] / st.l[i];
                if (stats && lane == 0) {
                    float* st2 = stats + (((size_t)b * max_q + i) * H + h) * 2;
                    st2[0] = st.m[i];
                    st2[1] = st.l[i];
                }
            }
        }
    }
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

    const int h = blockIdx.x, s = blockIdx.y;
    const size_t bh = (size_t)s * H + h;
    TE* K = Kc + bh * (size_t)max_pos * D;
    TE* V = Vc + bh * (size_t)max_pos * D;
    const float* kn = k_new + bh * D;
    const float* vn = v_new + bh * D;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int sub = lane % LPK;

    const int n = pos + 1;
    const int per_wave = ((n + NW * KPW - 1) / (NW * KPW)) * KPW;
    const int r0 = min(n, w * per_wave);
    const int r1 = min(n, r0 + per_wave);
    const bool has_cur = r0 <= pos && pos < r1;   // this wave's range ends with row pos

    // Loads first: the new row's fp32 source (only the wave that owns row pos),
    // the query, then the cache rows 0..pos-1 inside wave_attend; the new row
    // is rounded and folded in after them, so no load waits for another.
    CurRow<TE> ckr{}, cvr{};
    if (has_cur) {
        ckr = load_cur<TE>(kn + sub * VEC);
        cvr = load_cur<TE>(vn + sub * VEC);
    }
    float qr[1][VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) qr[0][j] = q[bh * D + sub * VEC + j];

    WaveState<1, VEC> st;
    st.init();
    wave_attend<D, TE, 1, NP>(K, V, r0, min(r1, pos), qr, 1, sl2, st);
    uint4 ck = make_uint4(0u, 0u, 0u, 0u), cv = ck;
    if (has_cur) {
        keep_below(ckr);
        keep_below(cvr);
        ck = pack_cur<TE>(ckr);
        cv = pack_cur<TE>(cvr);
        fold_row<D, TE, 1>(pos, ck, cv, lane / LPK, qr, 1, sl2, st);
    }
    if constexpr (NW == 1) {
        // one wave holds every row: no cross-wave merge, no barrier
        wave_merge_groups<D, TE, 1>(st, 1);
        if (lane < LPK) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) out[bh * D + sub * VEC + j] = st.acc[0][j] / st.l[0];
        }
    } else {
        wg_share<D, TE, 1, NW>(st, 1, wm, wl, wa);
        for (int d = threadIdx.x; d < D; d += NW * 64) {
            float M, L, A;
            wg_combine<D, 1, NW>(wm, wl, wa, 0, d, M, L, A);
            out[bh * D + d] = A / L;
        }
    }
    // Scatter the new row last, from its owner's registers (the values it
    // folded in). No wave reads it from memory. Stored before the cache-row
    // loads it would delay them, and stored before the merge the barrier
    // would wait for the stores.
    if (has_cur && lane < LPK) {
        *reinterpret_cast<uint4*>(K + (size_t)pos * D + sub * VEC) = ck;
        *reinterpret_cast<uint4*>(V + (size_t)pos * D + sub * VEC) = cv;
    }
}

// ----------------------------------------------------- attention weights
// Grid: (ceil(T / (4 * KPW)), B), 4 waves. Rows map to lanes as in the decode
// kernels: a group of LPK lanes reads one row, 16 bytes per lane, so a wave
// covers KPW consecutive rows with coalesced loads. For every query i the
// group re-forms the row's score under each selected head,
// s = scale log2(e) q.K[b][h][t] (dot reduced across the group with DPP),
// weights it with that head's final (max, sum) in the base-2 domain left in
// `stats` by the decode of the same call, p = 2^(s - max) / sum, and the
// group's first lane writes the mean over the selected heads, summed in list
// order (deterministic).
template <int D, typename TE>
__global__ __launch_bounds__(256) void xattn_weights_kernel(
    const float* __restrict__ q, const TE* __restrict__ Kl, const float* __restrict__ stats,
    float* __restrict__ weights, HeadList heads, int H, int T, int nq, int max_q, float sl2)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int grp = lane / LPK, sub = lane % LPK;
    const int t = (blockIdx.x * 4 + w) * KPW + grp;
    const int tr = min(t, T - 1);   // rows past T load row T-1 and write nothing
    const int n_sel = heads.n;
    for (int i = 0; i < nq; ++i) {
        float acc = 0.f;
        for (int k = 0; k < n_sel; ++k) {
            const int h = heads.h[k];
            const uint4 r = load16(Kl + (((size_t)b * H + h) * T + tr) * D + sub * VEC);
            const float* qv = q + (((size_t)b * nq + i) * H + h) * D + sub * VEC;
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < VEC; ++j) dot = fmaf(qv[j], elem<TE>(r, j), dot);
            dot = group_sum<LPK>(dot);
            const float* st2 = stats + (((size_t)b * max_q + i) * H + h) * 2;
            acc += fast_exp2(dot * sl2 - st2[0]) / st2[1];
        }
        if (sub == 0 && t < T) weights[((size_t)b * nq + i) * T + t] = acc / n_sel;
    }
}

// --------------------------------------------------------- self prefill
// Grid: (Hkv, S). One workgroup per (sequence, kv head) writes that kv head's
// rows pos .. pos+n_new-1 (rounded to the storage type), passes a workgroup
// barrier -- whose workgroup-scope release/acquire makes those stores visible
// to its own waves -- and then its waves take groups of up to QB consecutive
// tokens of one query head of the kv head's group (group j: head
// h = kv*G + j % G, tokens QB*(j / G) ..), reading rows 0 .. pos+i once per
// group with each token i masked to its own causal limit pos+i+1. Rows past
// pos+n_new-1 are neither read nor written, and no workgroup touches another
// one's rows.
template <int D, typename TE, int NW, int NP, int QB>
__global__ __launch_bounds__(NW * 64) void selfattn_prefill_kernel(
    const float* __restrict__ q, const float* __restrict__ k_new,
    const float* __restrict__ v_new, TE* __restrict__ Kc, TE* __restrict__ Vc,
    float* __restrict__ out, int Hkv, int Hq, int max_pos, int pos, int n_new, float sl2)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK;
    const int hk = blockIdx.x, s = blockIdx.y;
    const size_t skv = (size_t)s * Hkv + hk;
    TE* K = Kc + skv * (size_t)max_pos * D;
    TE* V = Vc + skv * (size_t)max_pos * D;
    const int G = Hq / Hkv;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int sub = lane % LPK;

    for (int x = threadIdx.x; x < n_new * D; x += NW * 64) {
        const int i = x / D, d = x % D;
        const size_t src = (((size_t)s * n_new + i) * Hkv + hk) * D + d;
        const size_t dst = (size_t)(pos + i) * D + d;
        if constexpr (sizeof(TE) == 2) {
            K[dst] = to_bf16_bits(k_new[src]);
            V[dst] = to_bf16_bits(v_new[src]);
        } else {
            K[dst] = k_new[src];
            V[dst] = v_new[src];
        }
    }
    __syncthreads();

    const int blocks = (n_new + QB - 1) / QB;
    for (int j = w; j < blocks * G; j += NW) {
        const int h = hk * G + j % G, i0 = QB * (j / G);
        const int nq = min(QB, n_new - i0);
        float qr[QB][VEC];
        int lim[QB];
#pragma unroll
        for (int k = 0; k < QB; ++k) {
            const int i = min(i0 + k, n_new - 1);
            lim[k] = pos + i + 1;
            const size_t qo = (((size_t)s * n_new + i) * Hq + h) * D;
#pragma unroll
            for (int e = 0; e < VEC; ++e) qr[k][e] = q[qo + sub * VEC + e];
        }
        WaveState<QB, VEC> st;
        st.init();
        wave_attend_causal<D, TE, QB, NP>(K, V, lim, qr, nq, sl2, st);
        wave_merge_groups<D, TE, QB>(st, nq);
        if (lane < LPK) {
#pragma unroll
            for (int k = 0; k < QB; ++k) {
                if (k < nq) {
                    const size_t qo = (((size_t)s * n_new + i0 + k) * Hq + h) * D;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) out[qo + sub * VEC + e] = st.acc[k][e] / st.l[k];
                }
            }
        }
    }
}

// Grid: (Hkv * Z, S), Z = ceil(n_new / QB) * G groups per kv head. One
// workgroup per group of up to QB consecutive tokens of one query head (group
// j of kv head hk: head h = hk*G + j % G, tokens QB*(j / G) ..), its NW waves
// taking contiguous shares of the rows the group reads, 0 .. pos+i for token
// i, merged through LDS. Rows below pos come from the cache, the new rows
// from k_new / v_new rounded as they are stored; the group's own new rows are
// written to the cache by its first head's workgroup (j % G == 0), which no
// workgroup of this launch reads. So no workgroup depends on another, and the
// rows of a kv head spread over Z workgroups instead of one. Rows past
// pos+n_new-1 are neither read nor written.
template <int D, typename TE, int NW, int NP, int QB>
__global__ __launch_bounds__(NW * 64) void selfattn_prefill_groups_kernel(
    const float* __restrict__ q, const float* __restrict__ k_new,
    const float* __restrict__ v_new, TE* __restrict__ Kc, TE* __restrict__ Vc,
    float* __restrict__ out, int Hkv, int Hq, int max_pos, int pos, int n_new, int Z, float sl2)
{
    using RM = RowMap<D, TE>;
    constexpr int VEC = RM::kVec, LPK = RM::kLPK, KPW = RM::kKPW;
    __shared__ float wm[NW * QB], wl[NW * QB], wa[NW * QB * D];
    const int s = blockIdx.y;
    const int hk = blockIdx.x / Z, j = blockIdx.x - hk * Z;
    const int G = Hq / Hkv;
    const size_t skv = (size_t)s * Hkv + hk;
    TE* K = Kc + skv * (size_t)max_pos * D;
    TE* V = Vc + skv * (size_t)max_pos * D;
    // token i of this sequence and kv head: k_new[(s * n_new + i) * Hkv + hk]
    const float* kn = k_new + ((size_t)s * n_new * Hkv + hk) * D;
    const float* vn = v_new + ((size_t)s * n_new * Hkv + hk) * D;
    const size_t new_stride = (size_t)Hkv * D;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int sub = lane % LPK;
    const int h = hk * G + j % G, i0 = QB * (j / G);
    const int nq = min(QB, n_new - i0);

    if (j % G == 0) {   // this token block's new rows, once per kv head
        for (int x = threadIdx.x; x < nq * D; x += NW * 64) {
            const int i = i0 + x / D, d = x % D;
            const size_t src = (size_t)i * new_stride + d;
            const size_t dst = (size_t)(pos + i) * D + d;
            if constexpr (sizeof(TE) == 2) {
                K[dst] = to_bf16_bits(kn[src]);
                V[dst] = to_bf16_bits(vn[src]);
            } else {
                K[dst] = kn[src];
                V[dst] = vn[src];
            }
        }
    }

    float qr[QB][VEC];
    int lim[QB];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        const int i = min(i0 + k, n_new - 1);
        lim[k] = pos + i + 1;
        const size_t qo = (((size_t)s * n_new + i) * Hq + h) * D;
#pragma unroll
        for (int e = 0; e < VEC; ++e) qr[k][e] = q[qo + sub * VEC + e];
    }
    const int R = pos + i0 + nq;   // rows the group reads: 0 .. R-1
    const int per_wave = ((R + NW * KPW - 1) / (NW * KPW)) * KPW;
    const int r0 = min(R, w * per_wave);
    const int r1 = min(R, r0 + per_wave);
    int lim_w[QB];
#pragma unroll
    for (int k = 0; k < QB; ++k) lim_w[k] = min(lim[k], r1);
    WaveState<QB, VEC> st;
    st.init();
    wave_attend_causal_span<D, TE, QB, NP>(K, V, kn, vn, new_stride, pos, r0, r1, lim_w, qr, nq, sl2, st);
    wg_share<D, TE, QB, NW>(st, nq, wm, wl, wa);
    for (int x = threadIdx.x; x < nq * D; x += NW * 64) {
        const int k = x / D, d = x % D;
        float M, L, A;
        wg_combine<D, QB, NW>(wm, wl, wa, k, d, M, L, A);
        out[(((size_t)s * n_new + i0 + k) * Hq + h) * D + d] = A / L;
    }
}

// ------------------------------------------------------------- launchers

#ifndef CKE_CROSS_NP
#define CKE_CROSS_NP 4
#endif
#ifndef CKE_CROSS_NP_F32
#define CKE_CROSS_NP_F32 3
#endif
#ifndef CKE_SELF_WAVES
#define CKE_SELF_WAVES 8
#endif
#ifndef CKE_SELF_NP
#define CKE_SELF_NP 2
#endif
constexpr int kCrossNP = CKE_CROSS_NP;        // row passes per load tile (16- and 8-bit rows)
constexpr int kCrossNPf32 = CKE_CROSS_NP_F32; // row passes per load tile (fp32 rows)
constexpr int kCrossNP16 = kCrossNP16Rows;    // bf16 rows, one query
constexpr int kSelfWaves = CKE_SELF_WAVES;
constexpr int kSelfNP = CKE_SELF_NP;

// Memories this short go to xattn_short_kernel.
constexpr int kShortRows = kShortMemRows;
#ifndef CKE_SHORT_NP
#define CKE_SHORT_NP 4
#endif
constexpr int kShortNP = CKE_SHORT_NP;  // passes per tile: 16 fp32 rows of 64 in one tile

template <int D, typename TE, int NQ>
hipError_t launch_cross_nq(const XattnLaunch& a, hipStream_t st) {
    if (a.T <= kShortRows) {
        constexpr int NW = 4;
        const int n_bh = a.B * a.H;
        hipLaunchKernelGGL((xattn_short_kernel<D, TE, NQ, NW, kShortNP>), dim3((n_bh + NW - 1) / NW),
                           dim3(NW * 64), 0, st, a.q, static_cast<const TE*>(a.K),
                           static_cast<const TE*>(a.V), a.out, a.stats, a.nq, a.max_q, a.H, a.T,
                           n_bh, a.scale * kLog2e);
        return hipGetLastError();
    }
    // Row passes per load tile. fp32 rows (4 values per lane): 3 at any query
    // count (Whisper Base 5.26 against 5.34 us per call with 4, Beam 8.64
    // against 8.83; 2 and 6 slower; before the in-launch merge, 4 passes had
    // taken Beam from 11.75 to 11.3 us against 2). bf16 and fp8 rows (8 or 16
    // values per lane): 4 (over fp8 16.17 against 16.35 us with 3), but 2
    // with more than two queries: long tiles cost registers (fp8 spills from
    // four queries on). bf16 rows and one query: 3, whose 80 VGPRs let a
    // compute unit hold 6 of these workgroups (4 at the 97 VGPRs of 4 passes),
    // so the 4-way split of Large's 320 heads, 5 per unit, is resident at
    // once: 22.97 against 23.98 us per call (4 passes, 3 splits).
    constexpr int NP = sizeof(TE) == 4
                           ? kCrossNPf32
                           : ((sizeof(TE) == 2 && NQ == 1) ? kCrossNP16
                                                           : ((NQ > 2 && kCrossNP > 2) ? 2 : kCrossNP));
    const int n_bh = a.B * a.H;
    dim3 grid(a.n_whole + 8 * a.nsplit * ((n_bh - a.n_whole + 7) / 8));
    unsigned* tickets =
        (a.tickets && merge_in_launch_fits(a.nq, D, a.nsplit, n_bh, a.max_q)) ? a.tickets : nullptr;
    // non-temporal buffer loads for fp32 caches and for 16- and 8-bit caches
    // far larger than the MALL; normal loads otherwise, and for a head slab
    // of 2 GB or more (buffer offsets are 32-bit)
    const bool slab_ok = (size_t)a.T * a.D * sizeof(TE) < ((size_t)1 << 31) - 16;
    if (slab_ok && (sizeof(TE) == 4 || a.stream_rows))
        hipLaunchKernelGGL((xattn_partial_kernel<D, TE, NQ, kCrossWaves, NP, true>), grid,
                           dim3(kCrossWaves * 64), 0, st, a.q,
                           static_cast<const TE*>(a.K), static_cast<const TE*>(a.V), a.out,
                           a.part, a.stats, tickets, a.nq, a.max_q, a.H, a.T, a.nsplit, a.chunk,
                           n_bh, a.n_whole, a.scale * kLog2e);
    else
        hipLaunchKernelGGL((xattn_partial_kernel<D, TE, NQ, kCrossWaves, NP, false>), grid,
                           dim3(kCrossWaves * 64), 0, st, a.q,
                           static_cast<const TE*>(a.K), static_cast<const TE*>(a.V), a.out,
                           a.part, a.stats, tickets, a.nq, a.max_q, a.H, a.T, a.nsplit, a.chunk,
                           n_bh, a.n_whole, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1 || tickets) return e;
    const int lanes = a.nq * D * merge_lanes(a.nsplit);
    const int threads = lanes >= 256 ? 256 : ((lanes + 63) / 64) * 64;
    const int Z = (lanes + threads - 1) / threads;
    hipLaunchKernelGGL((xattn_merge_kernel<D>), dim3(8 * Z * ((n_bh - a.n_whole + 7) / 8)), dim3(threads), 0,
                       st, a.part, a.out, a.stats, a.nq, a.max_q, a.H, a.nsplit, n_bh, Z, a.n_whole);
    return hipGetLastError();
}

template <int D, typename TE>
hipError_t launch_cross_d(const XattnLaunch& a, hipStream_t st) {
    switch (a.nq) {
        case 1: return launch_cross_nq<D, TE, 1>(a, st);
        case 2: return launch_cross_nq<D, TE, 2>(a, st);
        case 3: return launch_cross_nq<D, TE, 3>(a, st);
        case 4: return launch_cross_nq<D, TE, 4>(a, st);
        case 5: return launch_cross_nq<D, TE, 5>(a, st);
    }
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

template <int D, typename TE, int NW>
hipError_t launch_self_nw(const SelfLaunch& a, hipStream_t st) {
    dim3 grid(a.H, a.S);
    hipLaunchKernelGGL((selfattn_append_kernel<D, TE, NW, kSelfNP>), grid, dim3(NW * 64), 0, st,
                       a.q, a.k_new, a.v_new, static_cast<TE*>(a.K), static_cast<TE*>(a.V), a.out,
                       a.H, a.max_pos, a.pos, a.scale * kLog2e);
    return hipGetLastError();
}

// Waves per workgroup grow with the rows attended (pos + 1): each wave gets
// at least one full load tile, so short caches skip the cross-wave merge.
template <int D, typename TE>
hipError_t launch_self_d(const SelfLaunch& a, hipStream_t st) {
    constexpr int rows_per_tile = RowMap<D, TE>::kKPW * kSelfNP;
    const int tiles = (a.pos + 1 + rows_per_tile - 1) / rows_per_tile;
    if (tiles <= 1 || kSelfWaves == 1) return launch_self_nw<D, TE, 1>(a, st);
    if (tiles <= 2 || kSelfWaves == 2) return launch_self_nw<D, TE, 2>(a, st);
    if (tiles <= 4 || kSelfWaves == 4) return launch_self_nw<D, TE, 4>(a, st);
    return launch_self_nw<D, TE, kSelfWaves>(a, st);
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

constexpr int kPrefillQB = 8;   // tokens of one head sharing a wave's row reads
constexpr int kPrefillNP = 2;
constexpr long long kPrefillWaves = 2048;   // waves a grouped prefill launch aims to keep within

template <int D, typename TE, int NW, int QB>
hipError_t launch_prefill_nw(const PrefillLaunch& a, hipStream_t st) {
    hipLaunchKernelGGL((selfattn_prefill_kernel<D, TE, NW, QB == 1 ? kSelfNP : kPrefillNP, QB>),
                       dim3(a.Hkv, a.S), dim3(NW * 64), 0,
                       st, a.q, a.k_new, a.v_new, static_cast<TE*>(a.K), static_cast<TE*>(a.V), a.out,
                       a.Hkv, a.Hq, a.max_pos, a.pos, a.n_new, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, typename TE, int NW>
hipError_t launch_prefill_groups(const PrefillLaunch& a, int Z, hipStream_t st) {
    hipLaunchKernelGGL((selfattn_prefill_groups_kernel<D, TE, NW, kPrefillNP, kPrefillQB>),
                       dim3(a.Hkv * Z, a.S), dim3(NW * 64), 0, st, a.q, a.k_new, a.v_new,
                       static_cast<TE*>(a.K), static_cast<TE*>(a.V), a.out, a.Hkv, a.Hq, a.max_pos, a.pos,
                       a.n_new, Z, a.scale * kLog2e);
    return hipGetLastError();
}

// A kv head with at most 8 queries gives each query a wave of its own, in
// one workgroup per kv head (short, latency-bound calls such as a few prefix
// rows). With more, selfattn_prefill_groups_kernel: one workgroup per
// kPrefillQB tokens of one head (reading their rows once), up to 8 waves
// sharing those rows.
template <int D, typename TE>
hipError_t launch_prefill_d(const PrefillLaunch& a, hipStream_t st) {
    const long long G = a.Hq / a.Hkv;
    if ((long long)a.n_new * G <= 8) {
        const long long queries = (long long)a.n_new * G;
        if (queries <= 1) return launch_prefill_nw<D, TE, 1, 1>(a, st);
        if (queries <= 2) return launch_prefill_nw<D, TE, 2, 1>(a, st);
        if (queries <= 4) return launch_prefill_nw<D, TE, 4, 1>(a, st);
        return launch_prefill_nw<D, TE, 8, 1>(a, st);
    }
    // one workgroup per group of kPrefillQB tokens of one head, with waves
    // enough for a load tile each over the rows its last token reads, but no
    // more than keep the launch within about kPrefillWaves waves (8 per
    // compute unit) so that every workgroup is resident at once: Whisper
    // Base's 64-row chunk (64 groups) takes 8 waves per group, 8.75 against
    // 29.2 us with one workgroup per kv head; Large's (2,560 groups) one.
    const int Z = ((a.n_new + kPrefillQB - 1) / kPrefillQB) * (int)G;
    constexpr int rows_per_tile = RowMap<D, TE>::kKPW * kPrefillNP;
    const long long tiles = ((long long)a.pos + a.n_new + rows_per_tile - 1) / rows_per_tile;
    const long long wgs = (long long)a.Hkv * Z * a.S;
    const long long fit = kPrefillWaves / wgs;
    const long long nw = tiles < fit ? tiles : fit;
    if (nw <= 1) return launch_prefill_groups<D, TE, 1>(a, Z, st);
    if (nw < 4) return launch_prefill_groups<D, TE, 2>(a, Z, st);
    if (nw < 8) return launch_prefill_groups<D, TE, 4>(a, Z, st);
    return launch_prefill_groups<D, TE, 8>(a, Z, st);
}

template <typename TE>
hipError_t launch_prefill_t(const PrefillLaunch& a, hipStream_t st) {
    switch (a.D) {
        case 32: return launch_prefill_d<32, TE>(a, st);
        case 64: return launch_prefill_d<64, TE>(a, st);
        case 128: return launch_prefill_d<128, TE>(a, st);
    }
    return hipErrorInvalidValue;
}

// One workgroup of 4 waves per 4*KPW memory rows of one stream.
template <int D, typename TE>
hipError_t launch_weights_d(const WeightsLaunch& a, hipStream_t st) {
    constexpr int rows = 4 * RowMap<D, TE>::kKPW;
    hipLaunchKernelGGL((xattn_weights_kernel<D, TE>), dim3((a.T + rows - 1) / rows, a.B), dim3(256),
                       0, st, a.q, static_cast<const TE*>(a.K), a.stats, a.weights, a.heads, a.H,
                       a.T, a.nq, a.max_q, a.scale * kLog2e);
    return hipGetLastError();
}

template <typename TE>
hipError_t launch_weights_t(const WeightsLaunch& a, hipStream_t st) {
    switch (a.D) {
        case 32: return launch_weights_d<32, TE>(a, st);
        case 64: return launch_weights_d<64, TE>(a, st);
        case 128: return launch_weights_d<128, TE>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Per-type entry points, defined in attn_f32.hip, attn_bf16.hip, attn_fp8.hip.
hipError_t launch_cross_f32(const XattnLaunch& a, hipStream_t st);
hipError_t launch_weights_f32(const WeightsLaunch& a, hipStream_t st);
hipError_t launch_cross_bf16(const XattnLaunch& a, hipStream_t st);
hipError_t launch_weights_bf16(const WeightsLaunch& a, hipStream_t st);
hipError_t launch_cross_fp8(const XattnLaunch& a, hipStream_t st);
hipError_t launch_weights_fp8(const WeightsLaunch& a, hipStream_t st);
hipError_t launch_self_f32(const SelfLaunch& a, hipStream_t st);
hipError_t launch_prefill_f32(const PrefillLaunch& a, hipStream_t st);
hipError_t launch_self_bf16(const SelfLaunch& a, hipStream_t st);
hipError_t launch_prefill_bf16(const PrefillLaunch& a, hipStream_t st);

}  // namespace cke
