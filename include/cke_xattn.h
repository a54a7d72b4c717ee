/*
 * cke_xattn.h -- C ABI of libcke_xattn.so: encoder-decoder cross-attention over
 * a projection cache, and one-token self-attention over an explicit KV cache,
 * on one AMD Instinct MI355X (gfx950).
 *
 * Operations and where the pages define them:
 *   populate  C-Kernel-Engine, "Whisper: Trace One Encoder Tensor into Every
 *             Decoder Layer", section "The concept": every decoder layer l
 *             projects the one encoder memory E with its own weights,
 *             K_l = E x WK_l and V_l = E x WV_l. Section "View 2" and the
 *             circuit's projection_cache declaration: the result is kept
 *             layer-major, head-major, one slab per layer.
 *   ready     same page, "View 3": installing new encoder memory clears a
 *             ready flag, and decode refuses with -2 until prefill has
 *             repopulated the cache.
 *   decode    same page, "View 2": one query token of layer l attends over
 *             all key_tokens rows of slab l (not causal) with an explicit
 *             scale.
 *   self      "Recurrence as feeds" (topos), "What it opened": the self-
 *             attention cache is an ordinary input and output; the new row is
 *             written with scatter, then the token attends.
 *
 * Conventions shared by every call
 *   - All tensors are device memory owned by the caller. The library never
 *     allocates or frees device memory and keeps no pointer beyond what a
 *     cache handle records at creation.
 *   - Row-major, innermost index last. Weights are [d_model][H*D] in the
 *     y = x . W orientation; head h owns columns [h*D, (h+1)*D).
 *   - Cache layout (K and V are separate regions of identical shape):
 *     [L][B][H][T][D], elements of cache_dtype. Layer l's slab starts
 *     l*B*H*T*D elements into the region (for Whisper Base, fp32, layer 5
 *     starts 15,360,000 bytes in).
 *   - Every compute call is asynchronous on the given HIP stream (a
 *     hipStream_t passed as void*; NULL is the default stream). Status codes
 *     report host-side validation and launch errors only.
 *   - Calls that share one cache handle (its workspace) must be ordered on
 *     one stream; concurrent calls on one handle race.
 *   - On a non-OK status nothing was launched and no output was written;
 *     cke_last_error() returns a message (thread-local).
 */
#ifndef CKE_XATTN_H
#define CKE_XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. CKE_ENOTREADY is the -2 refusal of a stale cache. */
enum {
    CKE_OK = 0,
    CKE_EINVAL = -1,     /* null pointer, bad geometry, unsupported dtype mix */
    CKE_ENOTREADY = -2,  /* decode on a cache that is not populated */
    CKE_ERANGE = -3,     /* layer, position or query count out of range */
    CKE_EDEVICE = -4     /* the HIP runtime reported an error at launch */
};

/* Element types. CKE_FP8 is the 8-bit float with 4 exponent and 3 mantissa
 * bits (OCP E4M3: largest finite 448, no infinities), for projection caches
 * only: the compressed cache. WhisperKit case study, section 9: compress
 * where bandwidth is the limit, as it is for decode, which then reads half
 * the bytes of a bf16 cache. */
enum { CKE_F32 = 0, CKE_BF16 = 1, CKE_FP8 = 2 };

/* Largest number of decoder layers one cache (and one populate) serves. */
enum { CKE_MAX_LAYERS = 128 };

/* Geometry of one projection cache. Fail-closed: mem_len must be positive and
 * n_heads*head_dim must equal d_model (C-Kernel-Engine page, "View 3": both
 * are hard errors, not defaults). head_dim must be 32, 64 or 128 and d_model
 * a multiple of 32. */
typedef struct cke_xattn_geom {
    int32_t n_layers;    /* L, 1 .. CKE_MAX_LAYERS */
    int32_t n_streams;   /* B: independent encoder memories, >= 1 */
    int32_t mem_len;     /* T: encoder memory rows per stream, >= 1 */
    int32_t d_model;     /* encoder width = n_heads * head_dim */
    int32_t n_heads;     /* H */
    int32_t head_dim;    /* D */
    int32_t max_q;       /* largest n_q a decode call may pass, 1..8 */
    int32_t cache_dtype; /* CKE_F32, CKE_BF16 or CKE_FP8 */
} cke_xattn_geom;

/* Opaque host-side handle: geometry, the caller's K/V/workspace pointers and
 * the ready flag. Not thread-safe; one handle per cache. */
typedef struct cke_xattn_cache cke_xattn_cache;

/* Bytes of ONE of the two cache regions (K or V): L*B*H*T*D*elem.
 * Returns 0 for an invalid geometry. */
size_t cke_xattn_region_bytes(const cke_xattn_geom* g);

/* Byte offset of layer `layer`'s slab inside a region. Returns (size_t)-1 for
 * an invalid geometry or layer. */
size_t cke_xattn_layer_offset_bytes(const cke_xattn_geom* g, int layer);

/* Bytes of device workspace a cache needs: split-key partial results, fp32
 * [B][max_q][H][splits][D+2], then (256-byte aligned) per-head softmax
 * statistics, fp32 [B][max_q][H][2], that only cke_xattn_decode_weights
 * writes, then (256-byte aligned, when splits > 1) one 32-bit arrival
 * counter per (stream, head), 128 bytes apart (at least 256 bytes in all).
 * The workspace needs no initialisation: populate zeroes the counters and
 * every decode leaves them at zero; it belongs to one cache handle. Returns 0
 * for an invalid geometry. */
size_t cke_xattn_workspace_bytes(const cke_xattn_geom* g);

/* Number of key splits a decode call of this geometry uses (fixed per
 * geometry, so results are run-to-run deterministic). 0 if invalid. */
int cke_xattn_num_splits(const cke_xattn_geom* g);

/* Number of leading (stream, head) pairs, b*H + h < this value, that a decode
 * call of this geometry runs unsplit, one workgroup each; the others use
 * cke_xattn_num_splits splits. Nonzero only when B*H = 256k + R with R a
 * multiple of 8 such that the last R pairs split into u*256/R pieces (u = 1,
 * or 2 for single-query bf16 caches; 2 to 8 pieces of at least 128 rows)
 * give each of the 256 compute units k whole pairs and u pieces; the split
 * pairs, finished early, merge while whole pairs still stream. A plan choice
 * only: results agree with any other split to rounding. 0 if invalid. */
int cke_xattn_whole_pairs(const cke_xattn_geom* g);

/* Create a handle over caller-allocated device regions k_dev, v_dev (each
 * cke_xattn_region_bytes) and ws_dev (cke_xattn_workspace_bytes, 256-byte
 * aligned). The handle starts NOT ready. The first creation of a handle with
 * a split geometry (cke_xattn_num_splits > 1) on a device runs a short
 * placement probe there (one kernel on a private stream, waited for; see
 * cke_xattn_set_merge_mode), so do it outside stream capture; later
 * creations reuse its result. */
int cke_xattn_cache_create(const cke_xattn_geom* g, void* k_dev, void* v_dev,
                           void* ws_dev, cke_xattn_cache** out);

/* Free the handle (host memory only). NULL is accepted. */
void cke_xattn_cache_destroy(cke_xattn_cache* c);

/* New encoder memory is about to be installed: clear the ready flag. The
 * cache contents are left as they are. */
int cke_xattn_invalidate(cke_xattn_cache* c);

/* 1 if populated and not invalidated since, 0 otherwise (or for NULL). */
int cke_xattn_is_ready(const cke_xattn_cache* c);

/* Where a split decode merges its per-split partial results (C-Kernel-Engine,
 * "Whisper: Trace One Encoder Tensor into Every Decoder Layer", "View 2":
 * one query against all key rows, here split over workgroups and merged with
 * the online-softmax rescaling).
 *   mode 1 (default): in the split kernel's own launch, by the last workgroup
 *          of each head to finish, on handles whose creation verified that
 *          the device keeps workgroups i and i + 8 of a launch on one XCD
 *          (a probe, once per device); otherwise, and for merges needing
 *          more than 32 KB of LDS, as in mode 0;
 *   mode 0: a second, small kernel on the same stream.
 * Both give identical bits. Process-wide; affects calls made (or captured)
 * after it. Returns the previous mode, or CKE_EINVAL for another value. */
int cke_xattn_set_merge_mode(int mode);

/* 1 if a decode of n_q queries on c would merge in the split kernel's launch
 * under the current mode, 0 otherwise (including NULL, unsplit geometries and
 * n_q outside [1, max_q]). */
int cke_xattn_merges_in_launch(const cke_xattn_cache* c, int n_q);

/* Prefill: fill every layer's K and V slab from encoder memory E.
 *   E   device, [B][T][d_model], e_dtype
 *   WK  HOST array of L device pointers, each [d_model][H*D], w_dtype
 *   WV  likewise
 * Supported (e_dtype, w_dtype, cache_dtype): (F32, F32, F32) -- fp32
 * products, fp32 accumulation on the matrix cores --, (BF16, BF16, BF16)
 * -- bf16 products, fp32 accumulation, result rounded to nearest-even bf16
 * -- and (BF16, BF16, FP8) -- the same products, result clamped to
 * [-448, 448] and rounded to nearest-even E4M3; this one needs
 * n_heads*head_dim to be a multiple of 256 (CKE_EINVAL otherwise).
 * Sets the ready flag once the work is enqueued. */
int cke_xattn_populate(cke_xattn_cache* c, const void* E, int e_dtype,
                       const void* const* WK, const void* const* WV,
                       int w_dtype, void* stream);

/* cke_xattn_populate with caller workspace for the fp32 path: E and every
 * weight are split once into bf16 planes hi = bf16(x), lo = bf16(x - hi)
 * (nearest-even; hi + lo is within 2^-17 |x| of x) in ws, E as is and each
 * weight transposed, and the projections run as three bf16 products
 * lo.hi + hi.lo + hi.hi per k step with fp32 accumulation (each product
 * within 2^-16 of its fp32 value), reading the planes instead of splitting
 * every tile as it is loaded. The result is the same projection as
 * cke_xattn_populate (same page and section: K_l = E x WK_l, V_l = E x WV_l,
 * stored layer-major, head-major).
 *   ws, ws_bytes  device, 256-byte aligned, at least
 *                 cke_xattn_populate_workspace_bytes(g, e_dtype, w_dtype)
 *                 bytes; contents need no initialisation and are dead after
 *                 the call (the caller may reuse them once it is ordered
 *                 after the call on its stream)
 * The workspace applies to fp32 inputs and cache with n_heads*head_dim a
 * multiple of 128 and d_model a multiple of 64; for any other combination
 * cke_xattn_populate_workspace_bytes returns 0 and this call is
 * cke_xattn_populate (ws may then be NULL). Errors as cke_xattn_populate,
 * plus CKE_EINVAL for a NULL, misaligned or too small workspace. */
size_t cke_xattn_populate_workspace_bytes(const cke_xattn_geom* g, int e_dtype,
                                          int w_dtype);
int cke_xattn_populate_ws(cke_xattn_cache* c, const void* E, int e_dtype,
                          const void* const* WK, const void* const* WV,
                          int w_dtype, void* ws, size_t ws_bytes, void* stream);

/* Weight planes prepared ahead of time. The projection weights are the same
 * for every encoder window (C-Kernel-Engine, "Whisper: Trace One Encoder
 * Tensor into Every Decoder Layer", "The concept": one E per window feeds
 * fixed per-layer WK_l, WV_l), so their split into bf16 planes can run once,
 * after the weights are loaded, instead of inside every populate.
 *
 * cke_weight_planes splits n_mat fp32 device matrices W[i], each [k][n]
 * row-major, into planes [n_mat][hi, lo][n][k] bf16 (each matrix transposed;
 * hi = bf16(x), lo = bf16(x - hi), both nearest-even), the same planes
 * cke_xattn_populate_ws writes into its workspace.
 *   W             HOST array of n_mat device pointers, each 16-byte aligned
 *   n_mat         1 .. 2 * CKE_MAX_LAYERS
 *   k, n          k a multiple of 64, n of 128
 *   planes, bytes device, 256-byte aligned, at least
 *                 cke_weight_planes_bytes(n_mat, k, n) bytes; owned by the
 *                 caller, valid until the caller overwrites or frees them
 * cke_weight_planes_bytes returns 0 for unsupported sizes; the call returns
 * CKE_EINVAL for them and for NULL, misaligned or too small arguments. */
size_t cke_weight_planes_bytes(int n_mat, int k, int n);
int cke_weight_planes(const float* const* W, int n_mat, int k, int n, void* planes,
                      size_t bytes, void* stream);

/* Bytes of the per-call planes of rows x k fp32 values (hi and lo, each
 * [rows][k] bf16, rounded up to 256): the workspace of
 * cke_xattn_populate_planes. 0 when k is not a multiple of 64 or rows < 1. */
size_t cke_row_planes_bytes(int rows, int k);

/* cke_xattn_populate_ws with the weights already split: the same
 * projection (same page and section as cke_xattn_populate), bit-identical to
 * cke_xattn_populate_ws on the same fp32 E and weights. Per call only E is
 * split, into ws.
 *   E         device fp32 [B][T][d_model], 16-byte aligned
 *   w_planes  cke_weight_planes of the 2L matrices WK_0 .. WK_{L-1},
 *             WV_0 .. WV_{L-1} in that order, k = d_model, n = H*D; w_bytes
 *             at least cke_weight_planes_bytes(2L, d_model, H*D)
 *   ws        device, 256-byte aligned, ws_bytes at least
 *             cke_row_planes_bytes(B*T, d_model); dead after the call
 * Only fp32 caches with d_model a multiple of 64 and H*D of 128. Sets the
 * ready flag once the work is enqueued. CKE_EINVAL for any other geometry
 * and for NULL, misaligned or too small arguments. */
int cke_xattn_populate_planes(cke_xattn_cache* c, const float* E, const void* w_planes,
                              size_t w_bytes, void* ws, size_t ws_bytes, void* stream);

/* Cross-attention decode at one layer:
 *   out[b][i][h][:] = sum_t softmax_t(scale * q[b][i][h].K_l[b][h][t]) V_l[b][h][t]
 * over all T rows (no mask).
 *   q, out  device fp32 [B][n_q][H][D] (out must not alias q)
 *   n_q     0..max_q queries per stream (0 is a no-op); queries of one stream
 *           share every K/V read
 * Returns CKE_ENOTREADY if the cache is not populated. */
int cke_xattn_decode(const float* q, int n_q, const cke_xattn_cache* c,
                     int layer, float scale, float* out, void* stream);

/* cke_xattn_decode plus the attention weights of selected heads, averaged
 * over them:
 *   weights[b][i][t] = (1 / n_heads_sel) * sum_k p_k[t],
 *   p_k[t] = softmax_t(scale * q[b][i][heads[k]].K_l[b][heads[k]][t])
 * normalised with the same (max, sum) the decode itself formed.
 *   WhisperKit case study, section 6: the decoder exposes the attention
 *   weights of its alignment heads, averaged over those heads, for word-level
 *   timing.
 *   heads        HOST array of n_heads_sel head indices in [0, H) (repeats
 *                allowed); 1 <= n_heads_sel <= 32
 *   weights      device fp32 [B][n_q][T], 16-byte aligned
 * Errors as cke_xattn_decode, plus CKE_EINVAL / CKE_ERANGE for the head
 * list. Uses the statistics part of the cache's workspace. */
int cke_xattn_decode_weights(const float* q, int n_q, const cke_xattn_cache* c,
                             int layer, float scale, const int32_t* heads,
                             int n_heads_sel, float* out, float* weights,
                             void* stream);

/* One layer's self-attention KV cache, caller-owned: k and v are device
 * [n_seqs][n_heads][max_pos][head_dim] of dtype (CKE_F32 or CKE_BF16). */
typedef struct cke_kv_layer {
    void* k;
    void* v;
    int32_t n_seqs;      /* S */
    int32_t n_heads;     /* H */
    int32_t head_dim;    /* D: 32, 64 or 128 */
    int32_t max_pos;     /* capacity in rows */
    int32_t dtype;       /* CKE_F32 or CKE_BF16 */
} cke_kv_layer;

/* Fused scatter-append + causal attend for one token per sequence:
 *   row pos of kv->k, kv->v  <-  k_new, v_new   (rounded to bf16 if dtype is)
 *   out[s][h][:] = sum_{t<=pos} softmax_t(scale * q[s][h].K[s][h][t]) V[s][h][t]
 * reading the stored (rounded) values. Rows > pos are never read or written.
 *   q, k_new, v_new, out  device fp32 [S][H][D]
 *   pos                   0 <= pos < max_pos, else CKE_ERANGE */
int cke_selfattn_decode_append(const float* q, const float* k_new,
                               const float* v_new, const cke_kv_layer* kv,
                               int pos, float scale, float* out, void* stream);

/* Several new tokens per sequence at once, with grouped key/value heads:
 * rows pos .. pos+n_new-1 of every (sequence, kv head) are written from
 * k_new, v_new (rounded to bf16 if dtype is), then query i of head h attends
 * causally over rows 0 .. pos+i of kv head h / (n_q_heads / kv->n_heads):
 *   out[s][i][h][:] = sum_{t<=pos+i} softmax_t(scale * q[s][i][h].K[s][g][t]) V[s][g][t]
 * reading the stored (rounded) values. Rows >= pos+n_new are never read or
 * written. With n_new = 1 and n_q_heads = kv->n_heads this is
 * cke_selfattn_decode_append with [S][1][H][D] tensors.
 *   WhisperKit case study, section 5: the decoder's ContextPrefill starts at a
 *   cache already holding several prefix positions (several rows written at
 *   once); section 3: heads may share key/value heads (MHA, GQA, MQA).
 *   q, out        device fp32 [S][n_new][n_q_heads][D] (out must not alias q)
 *   k_new, v_new  device fp32 [S][n_new][kv->n_heads][D]
 *   n_q_heads     a positive multiple of kv->n_heads, at most 65535
 *   n_new >= 1, pos >= 0 and pos + n_new <= max_pos, else CKE_ERANGE */
int cke_selfattn_prefill_append(const float* q, const float* k_new,
                                const float* v_new, const cke_kv_layer* kv,
                                int pos, int n_new, int n_q_heads, float scale,
                                float* out, void* stream);

/* One decoder layer's projection weights, each [d_model][d_model] stored
 * output-major: row j holds output feature j's d_model input weights
 * (y[j] = sum_c x[c] W[j][c], the nn.Linear layout). Device memory of w dtype
 * (CKE_F32 or CKE_BF16), 16-byte aligned. */
typedef struct cke_decoder_layer {
    const void* wq_self;   /* self-attention query, key, value, output */
    const void* wk_self;
    const void* wv_self;
    const void* wo_self;
    const void* wq_cross;  /* cross-attention query and output */
    const void* wo_cross;
    int32_t dtype;
} cke_decoder_layer;

/* Bytes of device workspace cke_decoder_layer_step needs for n_seqs
 * sequences: seven fp32 [n_seqs][d_model] buffers. 0 if invalid. */
size_t cke_decoder_step_workspace_bytes(const cke_xattn_geom* g, int n_seqs);

/* One decoder layer for one token of each of S = kv->n_seqs sequences, in the
 * decoder-body order of the C-Kernel-Engine page, "The concept" (self-
 * attention, then cross-attention whose queries come from the decoder and
 * whose keys and values come from the projection cache of this layer; the
 * MLP and norms have no weights in these workloads and are not part of it):
 *   x += SelfAttn(x.WQs^T, x.WKs^T, x.WVs^T; kv, pos) . WOs^T
 *   x += CrossAttn(x.WQ^T; slab `layer` of c) . WO^T
 * SelfAttn is cke_selfattn_decode_append (row pos of kv written, rows 0..pos
 * attended); CrossAttn is cke_xattn_decode with n_q = S / n_streams, sequence
 * s being query s % n_q of stream s / n_q. Products run on the matrix cores
 * with fp32 accumulation: fp32 weights exactly, bf16 weights against x split
 * into two bf16 terms (about 16 significant bits of x).
 *   x      device fp32 [S][d_model], updated in place
 *   kv     this layer's self cache: n_heads and head_dim equal the cache's
 *   ws     device, cke_decoder_step_workspace_bytes(geometry of c, S) bytes,
 *          256-byte aligned; needs no initialisation
 * Uses c's workspace too, so calls on one cache must be ordered on one
 * stream. Errors: CKE_ENOTREADY if c is not populated; CKE_ERANGE for layer,
 * pos, or S not n_streams x n_q with n_q <= max_q; CKE_EINVAL otherwise. */
int cke_decoder_layer_step(float* x, const cke_decoder_layer* w, const cke_kv_layer* kv,
                           int pos, const cke_xattn_cache* c, int layer, float scale,
                           void* ws, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decoder-layer step as cke_decoder_layer_step, with its seven step buffers
 * in a fixed array inside the library instead of a caller workspace. The
 * library holds one such array per GPU it runs on, of
 * cke_decoder_step_scratch_bytes() bytes (2 MiB), until the process ends;
 * the call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine). The array's device address is looked up once per GPU,
 * on the first call with that GPU current.
 *   Same arguments and results as cke_decoder_layer_step, minus ws; the
 *   projection cache's own workspace (given at cache creation) is still used.
 *   CKE_EINVAL if the seven buffers (each n_seqs x d_model fp32, 256-byte
 *   aligned) do not fit the array; CKE_EDEVICE if the array's address cannot
 *   be found.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (every buffer is written before it is read, so nothing needs
 * clearing); calls that overlap on one GPU (other streams, other threads)
 * race and must be ordered by the caller. */
size_t cke_decoder_step_scratch_bytes(void);
int cke_decoder_layer_step_noalloc(float* x, const cke_decoder_layer* w,
                                   const cke_kv_layer* kv, int pos,
                                   const cke_xattn_cache* c, int layer,
                                   float scale, void* stream);

/* Projector memory lift, the prologue that produces a Q-Former-style encoder
 * memory before it is populated:
 *   out[r][j] = gelu(sum_c x[r][c] w[c][j]) + pos[r % pos_rows][j]
 * with the exact (erf) GELU, fp32 inputs, accumulation and output, products
 * on the matrix cores: for k_in >= 1024 as three bf16 products of operands
 * split into two bf16 terms each (each product within 2^-16 of its fp32
 * value), otherwise as fp32 products.
 *   transcribe.cpp "Forward map - granite_nar", "Projector (NLE simplified
 *   Q-Former)": the normalised 4-way encoder concat is lifted 4096 -> 2048
 *   with a GELU, and the window position embedding is added to every block of
 *   15 frames before the blocks serve as key/value memory.
 *   x    device fp32 [rows][k_in], k_in a multiple of 32
 *   w    device fp32 [k_in][n] (y = x . w), n a multiple of 64
 *   pos  device fp32 [pos_rows][n], or NULL for no positions
 *   out  device fp32 [rows][n], token-major (usable as E of cke_xattn_populate
 *        with n_streams = rows / mem_len); must not alias x, w or pos
 * CKE_EINVAL for NULL or misaligned pointers and unsupported sizes. */
int cke_memory_lift_gelu(const float* x, int rows, int k_in, const float* w, int n,
                         const float* pos, int pos_rows, float* out, void* stream);

/* cke_memory_lift_gelu with caller workspace: x and w are split once into
 * bf16 hi/lo planes in ws (w transposed) and the product runs as three bf16
 * products over them, as cke_xattn_populate_ws does (same page and section
 * as cke_memory_lift_gelu; same result within the same bound). A lift with
 * too few 192 x 256 output tiles to occupy the compute units is also split
 * over k_in into 2 or 4 slices whose fp32 partial sums (in ws) are added in
 * slice order before the GELU; the result stays deterministic.
 *   ws, ws_bytes  device, 256-byte aligned, at least
 *                 cke_memory_lift_workspace_bytes(rows, k_in, n) bytes
 * Applies when k_in is a multiple of 64 and n of 128; otherwise the
 * workspace size is 0 and this call is cke_memory_lift_gelu (ws may be
 * NULL). Errors as cke_memory_lift_gelu, plus CKE_EINVAL for a NULL,
 * misaligned or too small workspace. */
size_t cke_memory_lift_workspace_bytes(int rows, int k_in, int n);
int cke_memory_lift_gelu_ws(const float* x, int rows, int k_in, const float* w, int n,
                            const float* pos, int pos_rows, float* out, void* ws,
                            size_t ws_bytes, void* stream);

/* cke_memory_lift_gelu_ws with the lift weight already split by
 * cke_weight_planes (n_mat = 1, k = k_in, n): bit-identical to
 * cke_memory_lift_gelu_ws on the same x and w (same page and section as
 * cke_memory_lift_gelu). Per call only x is split, into ws (followed by the
 * partial sums of a lift split over k_in).
 *   w_planes, w_bytes  at least cke_weight_planes_bytes(1, k_in, n) bytes
 *   ws, ws_bytes       device, 256-byte aligned, at least
 *                      cke_memory_lift_planes_workspace_bytes(rows, k_in, n);
 *                      dead after the call
 * k_in a multiple of 64, n of 128 (the size function returns 0 otherwise).
 * Errors as cke_memory_lift_gelu, plus CKE_EINVAL for unsupported sizes and
 * NULL, misaligned or too small planes or workspace. */
size_t cke_memory_lift_planes_workspace_bytes(int rows, int k_in, int n);
int cke_memory_lift_gelu_planes(const float* x, int rows, int k_in, const void* w_planes,
                                size_t w_bytes, int n, const float* pos, int pos_rows,
                                float* out, void* ws, size_t ws_bytes, void* stream);

/* Message for the last non-OK status returned on this thread. */
const char* cke_last_error(void);

/* Library version string. */
const char* cke_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CKE_XATTN_H */
