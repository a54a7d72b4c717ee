// C ABI of libcke_xattn.so: host-side validation, the cache handle with its
// ready flag, launch planning and error reporting. Kernels live in
// populate.hip and attn_decode.hip.
//
// The ready flag follows C-Kernel-Engine, "Whisper: Trace One Encoder Tensor
// into Every Decoder Layer", "View 3": new encoder memory clears it, decode
// refuses with -2 until prefill has repopulated the cache. Geometry errors are
// fail-closed (same section): a non-positive encoder memory length or
// num_heads * head_dim != embed_dim is an error, never a default.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/cke_xattn.h"
#include "cke_internal.h"

struct cke_xattn_cache {
    cke_xattn_geom g;
    void* k;
    void* v;
    void* ws;
    int ready;
    int nsplit;
    int chunk;
    int n_whole;           // pairs 0 .. n_whole-1 decoded unsplit (split_plan)
    int merge_in_launch;   // split decode merges in its own launch (device placement verified)
};

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int elem_bytes(int dtype) { return dtype == CKE_FP8 ? 1 : (dtype == CKE_BF16 ? 2 : 4); }

bool dtype_ok(int dtype) { return dtype == CKE_F32 || dtype == CKE_BF16; }
bool cache_dtype_ok(int dtype) { return dtype_ok(dtype) || dtype == CKE_FP8; }

bool head_dim_ok(int D) { return D == 32 || D == 64 || D == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validate a geometry; returns CKE_OK or an error (message set).
int check_geom(const cke_xattn_geom* g) {
    if (!g) return fail(CKE_EINVAL, "geometry is NULL");
    if (g->mem_len <= 0)
        return fail(CKE_EINVAL, "encoder memory length must be positive (got %d)", g->mem_len);
    if (g->n_layers < 1 || g->n_layers > cke::kMaxLayers)
        return fail(CKE_EINVAL, "n_layers must be in [1, %d] (got %d)", cke::kMaxLayers, g->n_layers);
    if (g->n_streams < 1 || g->n_streams > 65535)
        return fail(CKE_EINVAL, "n_streams must be in [1, 65535] (got %d)", g->n_streams);
    if (g->n_heads < 1 || g->n_heads > 65535)
        return fail(CKE_EINVAL, "n_heads must be in [1, 65535] (got %d)", g->n_heads);
    if (!head_dim_ok(g->head_dim))
        return fail(CKE_EINVAL, "head_dim must be 32, 64 or 128 (got %d)", g->head_dim);
    if ((long long)g->n_heads * g->head_dim != g->d_model)
        return fail(CKE_EINVAL, "num_heads * head_dim (%d * %d) must equal d_model (%d)",
                    g->n_heads, g->head_dim, g->d_model);
    if (g->d_model % 32 != 0)
        return fail(CKE_EINVAL, "d_model must be a multiple of 32 (got %d)", g->d_model);
    if (g->max_q < 1 || g->max_q > 8) return fail(CKE_EINVAL, "max_q must be in [1, 8] (got %d)", g->max_q);
    if (!cache_dtype_ok(g->cache_dtype)) return fail(CKE_EINVAL, "unknown cache dtype %d", g->cache_dtype);
    const long long rows = (long long)g->n_streams * g->mem_len;
    if (rows > (1ll << 31) - 1) return fail(CKE_EINVAL, "n_streams * mem_len too large");
    const long long grid_y = 2ll * g->n_layers * g->d_model / 32;
    if (grid_y > 65535) return fail(CKE_EINVAL, "2 * n_layers * d_model too large");
    return CKE_OK;
}

// Whole cross caches (K + V, all layers) above this size are streamed past
// the caches by decode (twice the MALL; Whisper Base's 37 MB and Q-Former's
// 49 MB stay resident between calls, Large's 3.9 GB cannot).
constexpr size_t kStreamCacheBytes = size_t(512) << 20;

size_t region_elems(const cke_xattn_geom* g) {
    return (size_t)g->n_layers * g->n_streams * g->n_heads * (size_t)g->mem_len * g->head_dim;
}

#ifndef CKE_TARGET_WGS
#define CKE_TARGET_WGS 256
#endif
#ifndef CKE_MAX_SPLITS
#define CKE_MAX_SPLITS 64
#endif
static_assert(CKE_MAX_LAYERS == cke::kMaxLayers, "layer cap of the header and the kernels");
static_assert(CKE_MAX_SPLITS >= 1 && CKE_MAX_SPLITS <= cke::kMaxSplits, "split cap");

// Split of the T memory rows of one (stream, head) across workgroups. Fixed
// per geometry so that decode results are reproducible run to run.
//  * Fewer (stream, head) pairs than CKE_TARGET_WGS (one workgroup per
//    compute unit): split each head into about CKE_TARGET_WGS / (B*H) pieces,
//    but never fewer rows per workgroup than one pass of its waves. The call
//    is latency-bound; every compute unit gets a share.
//  * At least that many pairs: the unsplit grid already covers every compute
//    unit, but B*H workgroups over 256 units leave some units one workgroup
//    more than others (Large: 320 heads, 64 units with two), and each unit
//    streams at a capped rate, so the busiest units set the call's time.
//    Split into s pieces (2 <= s <= 8, at least 256 rows each, at most
//    cross_units_cap workgroups per compute unit, so that every workgroup is
//    resident at once) when that evens out the workgroups per unit: s
//    minimises ceil(B*H*s / 256) * 256 / (B*H*s), ties to the smaller s.
//    Large (bf16 cache): 4 splits, 5 workgroups on every unit, 22.97 against
//    26.3 us per call unsplit (3 splits, the best while a unit held only 4 of
//    these workgroups: 24.0); over its fp8 cache 3 splits, 16.2 against 16.7
//    us (2 splits 16.3; 4 splits 18.3: five workgroups per unit do not all
//    fit).
//  * Where B*H = 256k + R with R a multiple of 8 that divides 256 (or 512),
//    whole pairs plus one split group instead (cke_xattn_whole_pairs):
//    Large's 320 pairs as 256 whole and 64 split in 8 (two pieces per unit;
//    over fp8 in 4, one per unit). A uniform split ends with every head's
//    merge after the last rows are streamed; here the split pairs finish
//    early and merge while the whole pairs still stream, and whole pairs need
//    no merge: Large 21.96 against 23.04 us per call (4 uniform splits), over
//    fp8 15.48 against 15.95 (3 splits).
double unit_imbalance(long long wgs) {
    const long long units = CKE_TARGET_WGS;
    return (double)((wgs + units - 1) / units) * units / (double)wgs;
}

void split_plan(const cke_xattn_geom* g, int* nsplit, int* chunk, int* n_whole = nullptr) {
    int whole = 0;
    if (n_whole) *n_whole = 0;
    if (g->mem_len <= cke::kShortMemRows) {  // one wave per head, no split
        *nsplit = 1;
        *chunk = g->mem_len;
        return;
    }
    const int kpp = cke::cross_keys_per_pass(g->head_dim, elem_bytes(g->cache_dtype));
    const long long bh = (long long)g->n_streams * g->n_heads;
    const int max_by_rows = (g->mem_len + kpp - 1) / kpp;
    int s = 1;
    if (bh < CKE_TARGET_WGS) {
        long long want = (CKE_TARGET_WGS + bh - 1) / bh;
        if (want > CKE_MAX_SPLITS) want = CKE_MAX_SPLITS;
        s = (int)(want < max_by_rows ? want : max_by_rows);
        if (s < 1) s = 1;
    } else {
        double best = unit_imbalance(bh);
        for (int t = 2; t <= 8 && t <= max_by_rows && bh * t <= (long long)cke::cross_units_cap(elem_bytes(g->cache_dtype), g->max_q) * CKE_TARGET_WGS &&
                        g->mem_len >= 256LL * t; ++t) {
            const double im = unit_imbalance(bh * t);
            if (im < best - 1e-9) {
                best = im;
                s = t;
            }
        }
        // B*H = 256k + R, R a multiple of 8: the first 256k pairs whole (k
        // per unit) and the last R split into u*256/R pieces (u per unit), so
        // every unit streams the same rows and the split pairs, done early,
        // merge while whole pairs still stream. u = 2 for single-query bf16
        // rows where it fits (Large 21.82 against 21.93 us per call with
        // u = 1), else 1 (over fp8 u = 2 took 15.80 against 15.49 us).
        const long long R = bh % CKE_TARGET_WGS;
        const int cap = cke::cross_units_cap(elem_bytes(g->cache_dtype), g->max_q);
        const int u_max = (elem_bytes(g->cache_dtype) == 2 && g->max_q == 1) ? 2 : 1;
        for (int u = u_max; u >= 1 && R > 0 && R % 8 == 0 && whole == 0; --u) {
            if ((u * CKE_TARGET_WGS) % R != 0) continue;
            const long long t = u * CKE_TARGET_WGS / R;
            if (t >= 2 && t <= 8 && t <= max_by_rows && g->mem_len >= 128LL * t &&
                bh / CKE_TARGET_WGS + u <= cap) {
                s = (int)t;
                whole = (int)(bh - R);
            }
        }
    }
    int c = (g->mem_len + s - 1) / s;
    c = ((c + kpp - 1) / kpp) * kpp;
    *chunk = c;
    *nsplit = (g->mem_len + c - 1) / c;
    if (n_whole) *n_whole = *nsplit > 1 ? whole : 0;
}

constexpr size_t kAlign = 256;

// Workspace: fp32 split partials [B][max_q][H][nsplit][D+2], then (256-byte
// aligned) fp32 per-head statistics [B][max_q][H][2] that a decode call
// writes only when attention weights are requested, then (256-byte aligned,
// split geometries only) one arrival counter per head, 128 bytes apart,
// which populate zeroes and every decode leaves at zero.
size_t partial_words(const cke_xattn_geom* g, int nsplit) {
    return (size_t)g->n_streams * g->max_q * g->n_heads * (size_t)nsplit * (g->head_dim + 2);
}
size_t stats_offset_bytes(const cke_xattn_geom* g, int nsplit) {
    return (partial_words(g, nsplit) * sizeof(float) + kAlign - 1) / kAlign * kAlign;
}
size_t stats_bytes(const cke_xattn_geom* g) {
    return (size_t)g->n_streams * g->max_q * g->n_heads * 2 * sizeof(float);
}
size_t tickets_offset_bytes(const cke_xattn_geom* g, int nsplit) {
    return (stats_offset_bytes(g, nsplit) + stats_bytes(g) + kAlign - 1) / kAlign * kAlign;
}
size_t tickets_bytes(const cke_xattn_geom* g, int nsplit) {
    return nsplit > 1 ? (size_t)g->n_streams * g->n_heads * cke::kTicketBytes : 0;
}
unsigned* tickets_of(const cke_xattn_cache* c) {
    return reinterpret_cast<unsigned*>(static_cast<char*>(c->ws) + tickets_offset_bytes(&c->g, c->nsplit));
}

// In-launch merge of split decodes: process-wide switch (1 = where the
// device allows, 0 = always the second kernel) and the per-device result of
// the placement probe (0 = not yet probed, 1 = fails, 2 = holds).
std::atomic<int> g_merge_mode{1};
constexpr int kProbeDevices = 64;
std::atomic<int> g_placement[kProbeDevices];
std::mutex g_placement_mu;

bool xcd_placement_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kProbeDevices) {
        (void)hipGetLastError();
        return false;
    }
    int st = g_placement[dev].load(std::memory_order_acquire);
    if (st) return st == 2;
    std::lock_guard<std::mutex> lock(g_placement_mu);
    st = g_placement[dev].load(std::memory_order_relaxed);
    if (!st) {
        st = cke::probe_xcd_placement() ? 2 : 1;
        g_placement[dev].store(st, std::memory_order_release);
    }
    return st == 2;
}

// Zero the arrival counters (after a populate, before the first decode).
hipError_t reset_tickets(const cke_xattn_cache* c, hipStream_t st) {
    if (!c->merge_in_launch) return hipSuccess;
    return cke::launch_zero_words(tickets_of(c), tickets_bytes(&c->g, c->nsplit) / sizeof(unsigned), st);
}

}  // namespace

extern "C" {

const char* cke_last_error(void) { return g_err; }

const char* cke_version(void) { return "cke_xattn 0.1 gfx950"; }

size_t cke_xattn_region_bytes(const cke_xattn_geom* g) {
    if (check_geom(g) != CKE_OK) return 0;
    return region_elems(g) * elem_bytes(g->cache_dtype);
}

size_t cke_xattn_layer_offset_bytes(const cke_xattn_geom* g, int layer) {
    if (check_geom(g) != CKE_OK) return (size_t)-1;
    if (layer < 0 || layer >= g->n_layers) {
        fail(CKE_ERANGE, "layer %d outside [0, %d)", layer, g->n_layers);
        return (size_t)-1;
    }
    return region_elems(g) / g->n_layers * layer * elem_bytes(g->cache_dtype);
}

int cke_xattn_num_splits(const cke_xattn_geom* g) {
    if (check_geom(g) != CKE_OK) return 0;
    int s, c;
    split_plan(g, &s, &c);
    return s;
}

int cke_xattn_whole_pairs(const cke_xattn_geom* g) {
    if (check_geom(g) != CKE_OK) return 0;
    int s, c, w;
    split_plan(g, &s, &c, &w);
    return w;
}

size_t cke_xattn_workspace_bytes(const cke_xattn_geom* g) {
    if (check_geom(g) != CKE_OK) return 0;
    int s, c;
    split_plan(g, &s, &c);
    const size_t b = tickets_offset_bytes(g, s) + tickets_bytes(g, s);
    return b < kAlign ? kAlign : b;
}

int cke_xattn_cache_create(const cke_xattn_geom* g, void* k_dev, void* v_dev, void* ws_dev,
                           cke_xattn_cache** out) {
    if (!out) return fail(CKE_EINVAL, "out handle pointer is NULL");
    *out = nullptr;
    int rc = check_geom(g);
    if (rc != CKE_OK) return rc;
    if (!k_dev || !v_dev || !ws_dev) return fail(CKE_EINVAL, "k, v and workspace pointers must be non-NULL");
    if (!aligned16(k_dev) || !aligned16(v_dev))
        return fail(CKE_EINVAL, "cache regions must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(ws_dev) & (kAlign - 1)) != 0)
        return fail(CKE_EINVAL, "workspace must be 256-byte aligned");
    cke_xattn_cache* c = new (std::nothrow) cke_xattn_cache;
    if (!c) return fail(CKE_EINVAL, "out of host memory");
    c->g = *g;
    c->k = k_dev;
    c->v = v_dev;
    c->ws = ws_dev;
    c->ready = 0;
    split_plan(g, &c->nsplit, &c->chunk, &c->n_whole);
    // split geometries: verify (once per device) that the dispatcher keeps
    // workgroups i and i + 8 on one XCD, which the in-launch merge relies on
    c->merge_in_launch = c->nsplit > 1 && xcd_placement_ok();
    *out = c;
    return CKE_OK;
}

void cke_xattn_cache_destroy(cke_xattn_cache* c) { delete c; }

int cke_xattn_invalidate(cke_xattn_cache* c) {
    if (!c) return fail(CKE_EINVAL, "cache handle is NULL");
    c->ready = 0;
    return CKE_OK;
}

int cke_xattn_is_ready(const cke_xattn_cache* c) { return c ? c->ready : 0; }

int cke_xattn_set_merge_mode(int mode) {
    if (mode != 0 && mode != 1) return fail(CKE_EINVAL, "merge mode must be 0 or 1 (got %d)", mode);
    return g_merge_mode.exchange(mode);
}

int cke_xattn_merges_in_launch(const cke_xattn_cache* c, int n_q) {
    if (!c || !c->merge_in_launch || !g_merge_mode.load(std::memory_order_relaxed)) return 0;
    if (n_q < 1 || n_q > c->g.max_q) return 0;
    return cke::merge_in_launch_fits(n_q, c->g.head_dim, c->nsplit,
                                     (long long)c->g.n_streams * c->g.n_heads, c->g.max_q) ? 1 : 0;
}

}  // extern "C"

namespace {

// Geometry part of a populate launch descriptor (no weights).
void populate_geom(const cke_xattn_cache* c, const void* E, cke::PopulateLaunch* a) {
    const cke_xattn_geom& g = c->g;
    std::memset(a, 0, sizeof(*a));
    a->E = E;
    a->Kc = c->k;
    a->Vc = c->v;
    a->L = g.n_layers;
    a->B = g.n_streams;
    a->T = g.mem_len;
    a->dm = g.d_model;
    a->H = g.n_heads;
    a->D = g.head_dim;
}

// Checks shared by the populate calls; fills the launch descriptor.
int populate_args(const cke_xattn_cache* c, const void* E, int e_dtype, const void* const* WK,
                  const void* const* WV, int w_dtype, cke::PopulateLaunch* a) {
    if (!c) return fail(CKE_EINVAL, "cache handle is NULL");
    if (!E || !WK || !WV) return fail(CKE_EINVAL, "E, WK and WV must be non-NULL");
    const cke_xattn_geom& g = c->g;
    const bool f32 = e_dtype == CKE_F32 && w_dtype == CKE_F32 && g.cache_dtype == CKE_F32;
    const bool bf16 = e_dtype == CKE_BF16 && w_dtype == CKE_BF16 && g.cache_dtype == CKE_BF16;
    const bool fp8 = e_dtype == CKE_BF16 && w_dtype == CKE_BF16 && g.cache_dtype == CKE_FP8;
    if (!f32 && !bf16 && !fp8)
        return fail(CKE_EINVAL,
                    "unsupported dtypes (E %d, W %d, cache %d): need all fp32, all bf16, or bf16 "
                    "inputs with an fp8 cache", e_dtype, w_dtype, g.cache_dtype);
    if (fp8 && (g.n_heads * g.head_dim) % 256 != 0)
        return fail(CKE_EINVAL, "an fp8 cache needs n_heads * head_dim to be a multiple of 256");
    if (!aligned16(E)) return fail(CKE_EINVAL, "E must be 16-byte aligned");
    populate_geom(c, E, a);
    for (int l = 0; l < g.n_layers; ++l) {
        if (!WK[l] || !WV[l]) return fail(CKE_EINVAL, "weight pointer of layer %d is NULL", l);
        if (!aligned16(WK[l]) || !aligned16(WV[l]))
            return fail(CKE_EINVAL, "weights of layer %d must be 16-byte aligned", l);
        a->wt.w[l] = WK[l];
        a->wt.w[g.n_layers + l] = WV[l];
    }
    a->bf16 = bf16 || fp8;
    a->fp8 = fp8;
    return CKE_OK;
}

int populate_impl(cke_xattn_cache* c, const void* E, int e_dtype, const void* const* WK,
                  const void* const* WV, int w_dtype, void* ws, size_t ws_bytes, bool with_ws,
                  void* stream) {
    cke::PopulateLaunch a;
    const int rc = populate_args(c, E, e_dtype, WK, WV, w_dtype, &a);
    if (rc != CKE_OK) return rc;
    const size_t need = with_ws ? cke::populate_planes_bytes(a) : 0;
    if (need) {
        if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
            return fail(CKE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
        if (ws_bytes < need)
            return fail(CKE_EINVAL, "workspace holds %zu bytes; populate needs %zu", ws_bytes, need);
    }
    c->ready = 0;
    hipError_t e = need ? cke::launch_populate_planes(a, ws, static_cast<hipStream_t>(stream))
                        : cke::launch_populate(a, static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = reset_tickets(c, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "populate launch failed: %s", hipGetErrorString(e));
    c->ready = 1;
    return CKE_OK;
}

}  // namespace

extern "C" {

int cke_xattn_populate(cke_xattn_cache* c, const void* E, int e_dtype, const void* const* WK,
                       const void* const* WV, int w_dtype, void* stream) {
    return populate_impl(c, E, e_dtype, WK, WV, w_dtype, nullptr, 0, false, stream);
}

size_t cke_xattn_populate_workspace_bytes(const cke_xattn_geom* g, int e_dtype, int w_dtype) {
    if (check_geom(g) != CKE_OK) return 0;
    if (e_dtype != CKE_F32 || w_dtype != CKE_F32 || g->cache_dtype != CKE_F32) return 0;
    cke::PopulateLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.L = g->n_layers;
    a.B = g->n_streams;
    a.T = g->mem_len;
    a.dm = g->d_model;
    a.H = g->n_heads;
    a.D = g->head_dim;
    return cke::populate_planes_bytes(a);
}

int cke_xattn_populate_ws(cke_xattn_cache* c, const void* E, int e_dtype, const void* const* WK,
                          const void* const* WV, int w_dtype, void* ws, size_t ws_bytes,
                          void* stream) {
    return populate_impl(c, E, e_dtype, WK, WV, w_dtype, ws, ws_bytes, true, stream);
}

size_t cke_weight_planes_bytes(int n_mat, int k, int n) { return cke::weight_planes_bytes(n_mat, k, n); }

size_t cke_row_planes_bytes(int rows, int k) { return cke::row_planes_bytes(rows, k); }

int cke_weight_planes(const float* const* W, int n_mat, int k, int n, void* planes, size_t bytes,
                      void* stream) {
    const size_t need = cke::weight_planes_bytes(n_mat, k, n);
    if (!need)
        return fail(CKE_EINVAL, "weight planes need 1..%d matrices, k a multiple of 64 and n of 128 "
                    "(got %d, %d, %d)", 2 * cke::kMaxLayers, n_mat, k, n);
    if (!W) return fail(CKE_EINVAL, "weight table is NULL");
    if (!planes || (reinterpret_cast<uintptr_t>(planes) & (kAlign - 1)) != 0)
        return fail(CKE_EINVAL, "planes must be non-NULL and 256-byte aligned");
    if (bytes < need) return fail(CKE_EINVAL, "planes hold %zu bytes; %zu needed", bytes, need);
    cke::WeightTable wt;
    std::memset(&wt, 0, sizeof(wt));
    for (int i = 0; i < n_mat; ++i) {
        if (!W[i] || !aligned16(W[i]))
            return fail(CKE_EINVAL, "weight %d must be non-NULL and 16-byte aligned", i);
        wt.w[i] = W[i];
    }
    hipError_t e = cke::launch_weight_planes(wt, n_mat, k, n, planes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "weight split launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}

int cke_xattn_populate_planes(cke_xattn_cache* c, const float* E, const void* w_planes,
                              size_t w_bytes, void* ws, size_t ws_bytes, void* stream) {
    if (!c) return fail(CKE_EINVAL, "cache handle is NULL");
    const cke_xattn_geom& g = c->g;
    if (g.cache_dtype != CKE_F32) return fail(CKE_EINVAL, "prepared weight planes serve fp32 caches only");
    const int HD = g.n_heads * g.head_dim;
    const size_t w_need = cke::weight_planes_bytes(2 * g.n_layers, g.d_model, HD);
    const size_t e_need = cke::row_planes_bytes((long long)g.n_streams * g.mem_len, g.d_model);
    if (!w_need || !e_need)
        return fail(CKE_EINVAL, "prepared weight planes need d_model a multiple of 64 and n_heads * "
                    "head_dim of 128 (got %d, %d)", g.d_model, HD);
    if (!E || !w_planes || !ws) return fail(CKE_EINVAL, "E, w_planes and ws must be non-NULL");
    if (!aligned16(E)) return fail(CKE_EINVAL, "E must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_planes) & (kAlign - 1)) != 0 ||
        (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(CKE_EINVAL, "w_planes and ws must be 256-byte aligned");
    if (w_bytes < w_need) return fail(CKE_EINVAL, "w_planes hold %zu bytes; %zu needed", w_bytes, w_need);
    if (ws_bytes < e_need) return fail(CKE_EINVAL, "workspace holds %zu bytes; %zu needed", ws_bytes, e_need);
    cke::PopulateLaunch a;
    populate_geom(c, E, &a);
    c->ready = 0;
    hipError_t e = cke::launch_populate_from_planes(a, w_planes, ws, static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = reset_tickets(c, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "populate launch failed: %s", hipGetErrorString(e));
    c->ready = 1;
    return CKE_OK;
}

}  // extern "C"

namespace {

// Checks and launch shared by the two cross-decode calls; `stats` is null
// unless attention weights follow.
int cross_decode(const float* q, int n_q, const cke_xattn_cache* c, int layer, float scale,
                 float* out, float* stats, void* stream);

}  // namespace

extern "C" {

int cke_xattn_decode(const float* q, int n_q, const cke_xattn_cache* c, int layer, float scale,
                     float* out, void* stream) {
    return cross_decode(q, n_q, c, layer, scale, out, nullptr, stream);
}

int cke_xattn_decode_weights(const float* q, int n_q, const cke_xattn_cache* c, int layer,
                             float scale, const int32_t* heads, int n_heads_sel, float* out,
                             float* weights, void* stream) {
    if (!c) return fail(CKE_EINVAL, "cache handle is NULL");
    const cke_xattn_geom& g = c->g;
    if (!heads || n_heads_sel < 1 || n_heads_sel > cke::kMaxWeightHeads)
        return fail(CKE_EINVAL, "heads must list 1..%d heads", cke::kMaxWeightHeads);
    for (int k = 0; k < n_heads_sel; ++k)
        if (heads[k] < 0 || heads[k] >= g.n_heads)
            return fail(CKE_ERANGE, "heads[%d] = %d outside [0, %d)", k, heads[k], g.n_heads);
    if (n_q > 0 && (!weights || !aligned16(weights)))
        return fail(CKE_EINVAL, "weights must be non-NULL and 16-byte aligned");
    float* stats = reinterpret_cast<float*>(static_cast<char*>(c->ws) + stats_offset_bytes(&g, c->nsplit));
    int rc = cross_decode(q, n_q, c, layer, scale, out, stats, stream);
    if (rc != CKE_OK || n_q == 0) return rc;
    cke::WeightsLaunch a;
    a.q = q;
    a.K = static_cast<const char*>(c->k) + region_elems(&g) / g.n_layers * layer * elem_bytes(g.cache_dtype);
    a.stats = stats;
    a.weights = weights;
    a.heads.n = n_heads_sel;
    for (int k = 0; k < cke::kMaxWeightHeads; ++k) a.heads.h[k] = k < n_heads_sel ? heads[k] : 0;
    a.B = g.n_streams;
    a.H = g.n_heads;
    a.T = g.mem_len;
    a.D = g.head_dim;
    a.nq = n_q;
    a.max_q = g.max_q;
    a.scale = scale;
    a.dtype = g.cache_dtype;
    hipError_t e = cke::launch_xattn_weights(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "attention-weight launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}

}  // extern "C"

namespace {

int cross_decode(const float* q, int n_q, const cke_xattn_cache* c, int layer, float scale,
                 float* out, float* stats, void* stream) {
    if (!c) return fail(CKE_EINVAL, "cache handle is NULL");
    const cke_xattn_geom& g = c->g;
    if (layer < 0 || layer >= g.n_layers)
        return fail(CKE_ERANGE, "layer %d outside [0, %d)", layer, g.n_layers);
    if (n_q < 0 || n_q > g.max_q) return fail(CKE_ERANGE, "n_q %d outside [0, %d]", n_q, g.max_q);
    if (!c->ready)
        return fail(CKE_ENOTREADY, "projection cache is not populated for the current encoder memory");
    if (n_q == 0) return CKE_OK;
    if (!q || !out) return fail(CKE_EINVAL, "q and out must be non-NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(CKE_EINVAL, "q and out must be 16-byte aligned");
    if (!(scale == scale)) return fail(CKE_EINVAL, "scale is NaN");
    const size_t off = region_elems(&g) / g.n_layers * layer * elem_bytes(g.cache_dtype);
    cke::XattnLaunch a;
    a.q = q;
    a.K = static_cast<const char*>(c->k) + off;
    a.V = static_cast<const char*>(c->v) + off;
    a.out = out;
    a.part = static_cast<float*>(c->ws);
    a.B = g.n_streams;
    a.H = g.n_heads;
    a.T = g.mem_len;
    a.D = g.head_dim;
    a.nq = n_q;
    a.max_q = g.max_q;
    a.nsplit = c->nsplit;
    a.chunk = c->chunk;
    a.n_whole = c->n_whole;
    a.scale = scale;
    a.dtype = g.cache_dtype;
    // K and V of every layer together: a cache this much larger than the
    // 256 MB MALL is never re-read from it, so its rows are streamed
    a.stream_rows = 2 * region_elems(&g) * elem_bytes(g.cache_dtype) > kStreamCacheBytes;
    a.stats = stats;
    a.tickets = c->merge_in_launch && g_merge_mode.load(std::memory_order_relaxed) ? tickets_of(c) : nullptr;
    hipError_t e = cke::launch_xattn_decode(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "decode launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}


// Checks shared by the self-attention calls, in the order they report.
int check_self_args(const float* q, const float* k_new, const float* v_new,
                    const cke_kv_layer* kv, const float* out, float scale) {
    if (!kv) return fail(CKE_EINVAL, "kv layer descriptor is NULL");
    if (!q || !k_new || !v_new || !out || !kv->k || !kv->v)
        return fail(CKE_EINVAL, "q, k_new, v_new, out, kv->k and kv->v must be non-NULL");
    if (kv->n_seqs < 1 || kv->n_heads < 1 || kv->max_pos < 1)
        return fail(CKE_EINVAL, "n_seqs, n_heads and max_pos must be >= 1");
    if (kv->n_heads > 65535 || kv->n_seqs > 65535) return fail(CKE_EINVAL, "n_seqs or n_heads too large");
    if (!head_dim_ok(kv->head_dim))
        return fail(CKE_EINVAL, "head_dim must be 32, 64 or 128 (got %d)", kv->head_dim);
    if (!dtype_ok(kv->dtype)) return fail(CKE_EINVAL, "unknown kv dtype %d", kv->dtype);
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) ||
        !aligned16(kv->k) || !aligned16(kv->v))
        return fail(CKE_EINVAL, "all tensors must be 16-byte aligned");
    if (!(scale == scale)) return fail(CKE_EINVAL, "scale is NaN");
    return CKE_OK;
}

}  // namespace

extern "C" {

int cke_selfattn_decode_append(const float* q, const float* k_new, const float* v_new,
                               const cke_kv_layer* kv, int pos, float scale, float* out,
                               void* stream) {
    const int rc = check_self_args(q, k_new, v_new, kv, out, scale);
    if (rc != CKE_OK) return rc;
    if (pos < 0 || pos >= kv->max_pos)
        return fail(CKE_ERANGE, "pos %d outside [0, %d)", pos, kv->max_pos);
    cke::SelfLaunch a;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.K = kv->k;
    a.V = kv->v;
    a.out = out;
    a.S = kv->n_seqs;
    a.H = kv->n_heads;
    a.D = kv->head_dim;
    a.max_pos = kv->max_pos;
    a.pos = pos;
    a.scale = scale;
    a.bf16 = kv->dtype == CKE_BF16;
    hipError_t e = cke::launch_selfattn_append(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "self-attention launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}

int cke_selfattn_prefill_append(const float* q, const float* k_new, const float* v_new,
                                const cke_kv_layer* kv, int pos, int n_new, int n_q_heads,
                                float scale, float* out, void* stream) {
    const int rc = check_self_args(q, k_new, v_new, kv, out, scale);
    if (rc != CKE_OK) return rc;
    if (n_q_heads < 1 || n_q_heads > 65535 || n_q_heads % kv->n_heads != 0)
        return fail(CKE_EINVAL, "n_q_heads %d must be a positive multiple of kv->n_heads %d (at most 65535)",
                    n_q_heads, kv->n_heads);
    if (n_new < 1 || pos < 0 || (long long)pos + n_new > kv->max_pos)
        return fail(CKE_ERANGE, "rows [%d, %lld) outside [0, %d) or n_new < 1", pos,
                    (long long)pos + n_new, kv->max_pos);
    cke::PrefillLaunch a;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.K = kv->k;
    a.V = kv->v;
    a.out = out;
    a.S = kv->n_seqs;
    a.Hkv = kv->n_heads;
    a.Hq = n_q_heads;
    a.D = kv->head_dim;
    a.max_pos = kv->max_pos;
    a.pos = pos;
    a.n_new = n_new;
    a.scale = scale;
    a.bf16 = kv->dtype == CKE_BF16;
    hipError_t e = cke::launch_selfattn_prefill(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "self-attention prefill launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}

}  // extern "C"

namespace {

// Decoder-step workspace: seven fp32 [S][d_model] buffers, each 256-byte
// aligned: self q, k, v, self output, hidden state after the self residual,
// cross q, cross output.
constexpr int kStepBuffers = 7;

size_t step_buffer_bytes(const cke_xattn_geom* g, int n_seqs) {
    const size_t b = (size_t)n_seqs * g->d_model * sizeof(float);
    return (b + kAlign - 1) / kAlign * kAlign;
}

hipError_t gemv(const float* X, int n_out, const void* const* W, float* const* Y,
                const float* const* R, int S, int dm, bool bf16, hipStream_t st) {
    cke::GemvLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.X = X;
    a.n_out = n_out;
    for (int i = 0; i < n_out; ++i) a.o[i] = cke::GemvOut{W[i], Y[i], R ? R[i] : nullptr};
    for (int i = n_out; i < 3; ++i) a.o[i] = a.o[0];
    a.S = S;
    a.K = dm;
    a.N = dm;
    a.bf16 = bf16;
    return cke::launch_gemv(a, st);
}

}  // namespace

extern "C" {

size_t cke_decoder_step_workspace_bytes(const cke_xattn_geom* g, int n_seqs) {
    if (check_geom(g) != CKE_OK) return 0;
    if (n_seqs < 1 || n_seqs > 65535) {
        fail(CKE_EINVAL, "n_seqs must be in [1, 65535] (got %d)", n_seqs);
        return 0;
    }
    return kStepBuffers * step_buffer_bytes(g, n_seqs);
}

}  // extern "C"

namespace {

// Checks and launches shared by the two decoder-step entry points. `ws` is
// the seven-buffer workspace (caller memory or the library's scratch array);
// `ws_cap` its capacity in bytes, or 0 when the caller vouches for the size.
int decoder_layer_step(float* x, const cke_decoder_layer* w, const cke_kv_layer* kv, int pos,
                       const cke_xattn_cache* c, int layer, float scale, void* ws, size_t ws_cap,
                       void* stream) {
    if (!c) return fail(CKE_EINVAL, "cache handle is NULL");
    const cke_xattn_geom& g = c->g;
    if (layer < 0 || layer >= g.n_layers)
        return fail(CKE_ERANGE, "layer %d outside [0, %d)", layer, g.n_layers);
    if (!c->ready)
        return fail(CKE_ENOTREADY, "projection cache is not populated for the current encoder memory");
    if (!w || !kv) return fail(CKE_EINVAL, "weights and kv layer descriptors must be non-NULL");
    const void* W[6] = {w->wq_self, w->wk_self, w->wv_self, w->wo_self, w->wq_cross, w->wo_cross};
    for (int i = 0; i < 6; ++i)
        if (!W[i] || !aligned16(W[i])) return fail(CKE_EINVAL, "weight %d is NULL or not 16-byte aligned", i);
    if (!dtype_ok(w->dtype)) return fail(CKE_EINVAL, "unknown weight dtype %d", w->dtype);
    if (!kv->k || !kv->v || !aligned16(kv->k) || !aligned16(kv->v))
        return fail(CKE_EINVAL, "kv->k and kv->v must be non-NULL and 16-byte aligned");
    if (!dtype_ok(kv->dtype)) return fail(CKE_EINVAL, "unknown kv dtype %d", kv->dtype);
    if (kv->n_heads != g.n_heads || kv->head_dim != g.head_dim)
        return fail(CKE_EINVAL, "kv heads x head_dim (%d x %d) must match the cache's (%d x %d)",
                    kv->n_heads, kv->head_dim, g.n_heads, g.head_dim);
    if (kv->n_seqs < 1 || kv->n_seqs > 65535 || kv->max_pos < 1)
        return fail(CKE_EINVAL, "n_seqs must be in [1, 65535] and max_pos >= 1");
    const int S = kv->n_seqs;
    if (S % g.n_streams != 0 || S / g.n_streams > g.max_q)
        return fail(CKE_ERANGE, "n_seqs %d must be n_streams (%d) x n_q with n_q <= max_q (%d)", S,
                    g.n_streams, g.max_q);
    if (pos < 0 || pos >= kv->max_pos) return fail(CKE_ERANGE, "pos %d outside [0, %d)", pos, kv->max_pos);
    if (!x || !aligned16(x)) return fail(CKE_EINVAL, "x must be non-NULL and 16-byte aligned");
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(CKE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
    if (ws_cap && kStepBuffers * step_buffer_bytes(&g, S) > ws_cap)
        return fail(CKE_EINVAL,
                    "n_seqs x d_model (%d x %d) needs %zu bytes of step buffers; the library's "
                    "scratch holds %zu", S, g.d_model, kStepBuffers * step_buffer_bytes(&g, S),
                    ws_cap);
    if (!(scale == scale)) return fail(CKE_EINVAL, "scale is NaN");
    const int dm = g.d_model;
    const bool wbf16 = w->dtype == CKE_BF16;
    if (!cke::gemv_shape_ok(dm, dm))
        return fail(CKE_EINVAL, "d_model %d must be a multiple of 32 for the decoder-step products", dm);

    const size_t stride = step_buffer_bytes(&g, S);
    float* buf[kStepBuffers];
    for (int i = 0; i < kStepBuffers; ++i)
        buf[i] = reinterpret_cast<float*>(static_cast<char*>(ws) + i * stride);
    float *qs = buf[0], *ks = buf[1], *vs = buf[2], *so = buf[3], *x1 = buf[4], *qc = buf[5],
          *co = buf[6];
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    // 1. self-attention projections, one launch for the three weights
    {
        float* Y[3] = {qs, ks, vs};
        e = gemv(x, 3, W, Y, nullptr, S, dm, wbf16, st);
        if (e != hipSuccess) return fail(CKE_EDEVICE, "decoder-step projection launch failed: %s", hipGetErrorString(e));
    }
    // 2. append row pos to the self cache and attend
    cke::SelfLaunch sa;
    sa.q = qs;
    sa.k_new = ks;
    sa.v_new = vs;
    sa.K = kv->k;
    sa.V = kv->v;
    sa.out = so;
    sa.S = S;
    sa.H = kv->n_heads;
    sa.D = kv->head_dim;
    sa.max_pos = kv->max_pos;
    sa.pos = pos;
    sa.scale = scale;
    sa.bf16 = kv->dtype == CKE_BF16;
    e = cke::launch_selfattn_append(sa, st);
    if (e != hipSuccess) return fail(CKE_EDEVICE, "self-attention launch failed: %s", hipGetErrorString(e));
    // 3. x1 = x + so . WOs   4. qc = x1 . WQ
    {
        const void* Wo[1] = {W[3]};
        float* Y[1] = {x1};
        const float* R[1] = {x};
        e = gemv(so, 1, Wo, Y, R, S, dm, wbf16, st);
        if (e != hipSuccess) return fail(CKE_EDEVICE, "decoder-step projection launch failed: %s", hipGetErrorString(e));
        const void* Wq[1] = {W[4]};
        float* Yq[1] = {qc};
        e = gemv(x1, 1, Wq, Yq, nullptr, S, dm, wbf16, st);
        if (e != hipSuccess) return fail(CKE_EDEVICE, "decoder-step projection launch failed: %s", hipGetErrorString(e));
    }
    // 5. cross-attention: sequence s is query s % n_q of stream s / n_q
    int rc = cross_decode(qc, S / g.n_streams, c, layer, scale, co, nullptr, stream);
    if (rc != CKE_OK) return rc;
    // 6. x = x1 + co . WO
    {
        const void* Wo[1] = {W[5]};
        float* Y[1] = {x};
        const float* R[1] = {x1};
        e = gemv(co, 1, Wo, Y, R, S, dm, wbf16, st);
        if (e != hipSuccess) return fail(CKE_EDEVICE, "decoder-step projection launch failed: %s", hipGetErrorString(e));
    }
    return CKE_OK;
}

// The allocation-free decoder step's buffers: one file-scope device array per
// GPU, alive until the process ends. In host code `scratch` names only a
// host-side stand-in; the device address of each GPU's copy comes from
// hipGetSymbolAddress with that GPU current and is kept per device.
constexpr size_t kStepScratchBytes = size_t(2) << 20;
static __device__ __align__(256) unsigned char scratch[kStepScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's scratch array (looked up once per
// device); nullptr with the message set on failure.
void* step_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(CKE_EDEVICE, "no current HIP device (or device index >= %d)", kMaxDevices);
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        fail(CKE_EDEVICE, "scratch address lookup failed on device %d: %s", dev, hipGetErrorString(e));
        return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

int cke_decoder_layer_step(float* x, const cke_decoder_layer* w, const cke_kv_layer* kv, int pos,
                           const cke_xattn_cache* c, int layer, float scale, void* ws,
                           void* stream) {
    return decoder_layer_step(x, w, kv, pos, c, layer, scale, ws, 0, stream);
}

size_t cke_decoder_step_scratch_bytes(void) { return kStepScratchBytes; }

int cke_decoder_layer_step_noalloc(float* x, const cke_decoder_layer* w, const cke_kv_layer* kv,
                                   int pos, const cke_xattn_cache* c, int layer, float scale,
                                   void* stream) {
    void* ws = step_scratch();
    if (!ws) return CKE_EDEVICE;
    return decoder_layer_step(x, w, kv, pos, c, layer, scale, ws, kStepScratchBytes, stream);
}

}  // extern "C"

extern "C" {

}  // extern "C"

namespace {

int lift_args(const float* x, int rows, int k_in, const float* w, int n, const float* pos,
              int pos_rows, float* out, cke::LiftLaunch* a) {
    if (!x || !w || !out) return fail(CKE_EINVAL, "x, w and out must be non-NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (pos && !aligned16(pos)))
        return fail(CKE_EINVAL, "x, w, pos and out must be 16-byte aligned");
    if (rows < 1 || k_in < 1 || n < 1)
        return fail(CKE_EINVAL, "rows, k_in and n must be positive (got %d, %d, %d)", rows, k_in, n);
    if (k_in % 32 != 0 || n % 64 != 0)
        return fail(CKE_EINVAL, "k_in must be a multiple of 32 and n of 64 (got %d, %d)", k_in, n);
    if ((long long)rows * k_in > (1ll << 31) - 1 || (long long)rows * n > (1ll << 31) - 1)
        return fail(CKE_EINVAL, "rows x k_in or rows x n too large");
    if (pos && pos_rows < 1) return fail(CKE_EINVAL, "pos_rows must be >= 1 when pos is given");
    a->x = x;
    a->w = w;
    a->pos = pos;
    a->out = out;
    a->rows = rows;
    a->k_in = k_in;
    a->n = n;
    a->pos_rows = pos ? pos_rows : 1;
    return CKE_OK;
}

}  // namespace

extern "C" {

int cke_memory_lift_gelu(const float* x, int rows, int k_in, const float* w, int n,
                         const float* pos, int pos_rows, float* out, void* stream) {
    cke::LiftLaunch a;
    const int rc = lift_args(x, rows, k_in, w, n, pos, pos_rows, out, &a);
    if (rc != CKE_OK) return rc;
    hipError_t e = cke::launch_lift(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "memory lift launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}

size_t cke_memory_lift_workspace_bytes(int rows, int k_in, int n) {
    if (rows < 1 || k_in < 1 || n < 1 || k_in % 32 != 0 || n % 64 != 0) return 0;
    if ((long long)rows * k_in > (1ll << 31) - 1 || (long long)rows * n > (1ll << 31) - 1) return 0;
    cke::LiftLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.rows = rows;
    a.k_in = k_in;
    a.n = n;
    return cke::lift_planes_bytes(a);
}

size_t cke_memory_lift_planes_workspace_bytes(int rows, int k_in, int n) {
    if (rows < 1 || k_in < 1 || n < 1) return 0;
    if ((long long)rows * k_in > (1ll << 31) - 1 || (long long)rows * n > (1ll << 31) - 1) return 0;
    cke::LiftLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.rows = rows;
    a.k_in = k_in;
    a.n = n;
    return cke::lift_rows_bytes(a);
}

int cke_memory_lift_gelu_planes(const float* x, int rows, int k_in, const void* w_planes,
                                size_t w_bytes, int n, const float* pos, int pos_rows, float* out,
                                void* ws, size_t ws_bytes, void* stream) {
    const size_t w_need = cke::weight_planes_bytes(1, k_in, n);
    const size_t e_need = cke_memory_lift_planes_workspace_bytes(rows, k_in, n);
    if (rows >= 1 && (!w_need || !e_need))
        return fail(CKE_EINVAL, "prepared weight planes need k_in a multiple of 64 and n of 128 "
                    "(got %d, %d)", k_in, n);
    cke::LiftLaunch a;
    // lift_args checks the weight argument for NULL and alignment only
    const int rc = lift_args(x, rows, k_in, static_cast<const float*>(w_planes), n, pos, pos_rows, out, &a);
    if (rc != CKE_OK) return rc;
    if (!ws) return fail(CKE_EINVAL, "ws must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(w_planes) & (kAlign - 1)) != 0 ||
        (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(CKE_EINVAL, "w_planes and ws must be 256-byte aligned");
    if (w_bytes < w_need) return fail(CKE_EINVAL, "w_planes hold %zu bytes; %zu needed", w_bytes, w_need);
    if (ws_bytes < e_need) return fail(CKE_EINVAL, "workspace holds %zu bytes; %zu needed", ws_bytes, e_need);
    a.w = nullptr;
    hipError_t e = cke::launch_lift_from_planes(a, w_planes, ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "memory lift launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}

int cke_memory_lift_gelu_ws(const float* x, int rows, int k_in, const float* w, int n,
                            const float* pos, int pos_rows, float* out, void* ws, size_t ws_bytes,
                            void* stream) {
    cke::LiftLaunch a;
    const int rc = lift_args(x, rows, k_in, w, n, pos, pos_rows, out, &a);
    if (rc != CKE_OK) return rc;
    const size_t need = cke::lift_planes_bytes(a);
    if (need) {
        if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
            return fail(CKE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
        if (ws_bytes < need)
            return fail(CKE_EINVAL, "workspace holds %zu bytes; the lift needs %zu", ws_bytes, need);
    }
    hipError_t e = need ? cke::launch_lift_planes(a, ws, static_cast<hipStream_t>(stream))
                        : cke::launch_lift(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CKE_EDEVICE, "memory lift launch failed: %s", hipGetErrorString(e));
    return CKE_OK;
}

}  // extern "C"
