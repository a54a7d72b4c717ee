/*
 * Plain CPU oracle for encoder-decoder cross-attention over a projection cache.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the HIP library; the two see the same seeded inputs and nothing
 * else.
 *
 * Everything is naive loops in double precision, accumulated in ascending index
 * order. Build with -ffp-contract=off and without -ffast-math so every sum is
 * evaluated exactly as written (no fused multiply-add, no reassociation). The
 * OpenMP loops only split independent output units, so the result of every
 * element is the same for any thread count.
 *
 * Sources (page title, then section):
 *   [CKE]  "Whisper: Trace One Encoder Tensor into Every Decoder Layer"
 *          (C-Kernel-Engine) -- "The concept", "View 2", "View 3",
 *          "Deliberate failure".
 *   [TOP]  "Recurrence as feeds" (topos) -- "What it opened".
 *   [WK]   "Caso de estudio: WhisperKit" (ANE knowledge base) -- sections 2, 3, 4, 8.
 *   [GRN]  "Forward map - granite_nar" (transcribe.cpp) -- "Projector (NLE
 *          simplified Q-Former)".
 *
 * Parity pins live in tests/test_oracle_pins.py; every function below is
 * pinned there by something other than itself (library routines, closed forms,
 * invariants, brute force, bit-exact incremental == full-window recompute).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- threads */

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------ bf16 rounding
 * Round a double to the nearest bfloat16 value (8 significant bits, the
 * float32 exponent range), ties to even. Used where the workload stores a
 * cache in bfloat16: the stored value is the rounded one. Overflow to
 * infinity is not modelled (values here are O(1)).
 */
double orc_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    const double min_normal = ldexp(1.0, -126);
    if (fabs(x) < min_normal) {
        /* subnormal range: fixed spacing 2^-133 */
        return ldexp(nearbyint(ldexp(x, 133)), -133);
    }
    int e;
    double f = frexp(x, &e);            /* x = f * 2^e, 0.5 <= |f| < 1 */
    double r = nearbyint(ldexp(f, 8));  /* 8 significant bits, ties-to-even */
    return ldexp(r, e - 8);
}

void orc_round_bf16_array(const double* x, double* y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = orc_round_bf16(x[i]);
}

/* ----------------------------------------------------- fp8 (e4m3) rounding
 * The compressed projection cache stores 8-bit floats with 4 exponent bits
 * (bias 7) and 3 mantissa bits, no infinities: largest finite 448, smallest
 * normal 2^-6, subnormal spacing 2^-9 (the OCP "E4M3" format). A value is
 * first clamped to [-448, 448] (the cache saturates rather than storing a
 * non-finite code) and then rounded to the nearest representable value, ties
 * to even.
 */
double orc_round_fp8(double x)
{
    if (x != x) return x;
    if (x > 448.0) x = 448.0;
    if (x < -448.0) x = -448.0;
    if (x == 0.0) return x;
    const double min_normal = ldexp(1.0, -6);
    if (fabs(x) < min_normal) return ldexp(nearbyint(ldexp(x, 9)), -9);
    int e;
    double f = frexp(x, &e);            /* x = f * 2^e, 0.5 <= |f| < 1 */
    double r = nearbyint(ldexp(f, 4));  /* 4 significant bits, ties-to-even */
    return ldexp(r, e - 4);
}

void orc_round_fp8_array(const double* x, double* y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = orc_round_fp8(x[i]);
}

/* Storage rounding of a cache element: 0 none (fp32 stores the fp64 value
 * here), 1 bfloat16, 2 fp8 e4m3. */
static double round_store(double x, int mode)
{
    return mode == 1 ? orc_round_bf16(x) : (mode == 2 ? orc_round_fp8(x) : x);
}

/* ---------------------------------------------------------------- O1: project
 * [CKE] "The concept": every decoder layer l applies its own WK_l / WV_l to the
 * one encoder memory E (K_l = E x WK_l, V_l = E x WV_l); the encoder's internal
 * K/V are never reused. [CKE] "View 2" / "Deliberate failure": the cache is
 * stored head-major, [head][token][dim], and one slab per layer.
 *
 * orc_project_head writes one head's slab:
 *   out[t][d] = sum_{c ascending} E[t][c] * W[c][col0 + d],  t < T, d < D
 * E is token-major [T][dm]; W is [dm][ldw] row-major (y = x . W orientation).
 * round_mode: 0 stores the value as is, 1 rounds it to bfloat16, 2 to fp8
 * e4m3 (round_store).
 */
void orc_project_head(int T, int dm, int D, const double* E, const double* W,
                      int ldw, int col0, int round_mode, double* out)
{
    for (int t = 0; t < T; ++t) {
        const double* e = E + (size_t)t * dm;
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int c = 0; c < dm; ++c)
                acc += e[c] * W[(size_t)c * ldw + col0 + d];
            out[(size_t)t * D + d] = round_store(acc, round_mode);
        }
    }
}

/* Whole projection cache: Kc, Vc are [L][B][H][T][D]; E is [B][T][dm];
 * WK, WV are [L][dm][H*D]. */
void orc_populate(int L, int B, int T, int dm, int H, int D, const double* E,
                  const double* WK, const double* WV, int round_mode,
                  double* Kc, double* Vc)
{
    const int HD = H * D;
#pragma omp parallel for collapse(3) schedule(static)
    for (int l = 0; l < L; ++l)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h) {
                size_t slab = ((((size_t)l * B + b) * H + h) * T) * D;
                const double* Eb = E + (size_t)b * T * dm;
                orc_project_head(T, dm, D, Eb, WK + (size_t)l * dm * HD, HD,
                                 h * D, round_mode, Kc + slab);
                orc_project_head(T, dm, D, Eb, WV + (size_t)l * dm * HD, HD,
                                 h * D, round_mode, Vc + slab);
            }
}

/* Byte offset of layer l's slab in one cache region whose elements are
 * elem_bytes wide ([CKE] "View 2": layer 5 of Whisper Base sits 15,360,000
 * bytes past the K-cache base). */
size_t orc_layer_offset_bytes(int layer, int B, int H, int T, int D,
                              int elem_bytes)
{
    return (size_t)layer * B * H * T * D * (size_t)elem_bytes;
}

/* ------------------------------------------------------------ O2: attention
 * One query against n key/value rows (no mask: every row takes part):
 *   s_t   = (sum_{d asc} q[d] * K[t][d]) * scale
 *   m     = max_t s_t
 *   e_t   = exp(s_t - m)
 *   Z     = sum_{t asc} e_t
 *   out_d = (sum_{t asc} e_t * V[t][d]) / Z
 * The max shift does not change the result (softmax is shift invariant, [WK]
 * section 2) and keeps every exponent <= 0. K and V rows are D apart.
 * [CKE] "View 2": the decode call runs query_tokens = 1 against key_tokens
 * rows with an explicit scale.
 */
static void attend_one(int n, int D, double scale, const double* q,
                       const double* K, const double* V, double* out,
                       double* s)
{
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[d] * K[(size_t)t * D + d];
        s[t] = dot * scale;
        if (s[t] > m) m = s[t];
    }
    double Z = 0.0;
    for (int t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        Z += s[t];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int t = 0; t < n; ++t) acc += s[t] * V[(size_t)t * D + d];
        out[d] = acc / Z;
    }
}

/* Exported single-row attention (brute-force and invariance pins use it). */
void orc_attend(int n, int D, double scale, const double* q, const double* K,
                const double* V, double* out)
{
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    attend_one(n, D, scale, q, K, V, out, s);
    free(s);
}

/* Cross-attention decode over one layer's slab ([CKE] "The concept", "View 2";
 * non-causal per the circuit declaration):
 *   q, out: [B][nq][H][D];  Kc, Vc: this layer's slab [B][H][T][D]. */
void orc_cross_decode(int B, int nq, int H, int T, int D, double scale,
                      const double* q, const double* Kc, const double* Vc,
                      double* out)
{
#pragma omp parallel for collapse(3) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < nq; ++i)
            for (int h = 0; h < H; ++h) {
                double* s = (double*)malloc(sizeof(double) * (size_t)T);
                size_t qo = (((size_t)b * nq + i) * H + h) * D;
                size_t ko = (((size_t)b * H + h) * T) * D;
                attend_one(T, D, scale, q + qo, Kc + ko, Vc + ko, out + qo, s);
                free(s);
            }
}

/* Cross-attention weights of selected heads, averaged over them ([WK]
 * section 6: the decoder's alignment heads expose their attention weights,
 * which are averaged over those heads for word timing). For every stream b
 * and query i:
 *   p[h][t] = exp(scale q.K_t - max) / sum_u exp(scale q.K_u - max)   (head h)
 *   weights[b][i][t] = (1 / n_sel) * sum_k p[heads[k]][t]
 * in ascending k. Also returns the attention output of every head, as
 * orc_cross_decode does. */
void orc_cross_decode_weights(int B, int nq, int H, int T, int D, double scale,
                              const double* q, const double* Kc, const double* Vc,
                              const int* heads, int n_sel, double* out, double* weights)
{
    orc_cross_decode(B, nq, H, T, D, scale, q, Kc, Vc, out);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < nq; ++i) {
            double* w = weights + ((size_t)b * nq + i) * T;
            double* s = (double*)malloc(sizeof(double) * (size_t)T);
            for (int t = 0; t < T; ++t) w[t] = 0.0;
            for (int k = 0; k < n_sel; ++k) {
                const int h = heads[k];
                const double* qv = q + (((size_t)b * nq + i) * H + h) * D;
                const double* K = Kc + (((size_t)b * H + h) * T) * D;
                double m = -INFINITY;
                for (int t = 0; t < T; ++t) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += qv[d] * K[(size_t)t * D + d];
                    s[t] = dot * scale;
                    if (s[t] > m) m = s[t];
                }
                double Z = 0.0;
                for (int t = 0; t < T; ++t) {
                    s[t] = exp(s[t] - m);
                    Z += s[t];
                }
                for (int t = 0; t < T; ++t) w[t] += s[t] / Z;
            }
            for (int t = 0; t < T; ++t) w[t] /= n_sel;
            free(s);
        }
}

/* ---------------------------------------------- O3: self-attention decode
 * [TOP] "What it opened": the cache is an ordinary input and output; the new
 * row is written with scatter, then the token attends over the cache.
 * Causal with the current token included: rows 0..pos take part, rows > pos do
 * not (they are never read). Ks, Vs: [S][H][max_pos][D]; q, kn, vn, out:
 * [S][H][D]. If round_bf16 != 0 the stored rows are rounded to bfloat16 and
 * the attention reads the stored values.
 */
void orc_self_append_attend(int S, int H, int D, int max_pos, int pos,
                            double scale, int round_bf16, const double* q,
                            const double* kn, const double* vn, double* Ks,
                            double* Vs, double* out)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int s = 0; s < S; ++s)
        for (int h = 0; h < H; ++h) {
            size_t base = ((size_t)s * H + h) * (size_t)max_pos * D;
            size_t row = base + (size_t)pos * D;
            size_t io = ((size_t)s * H + h) * D;
            for (int d = 0; d < D; ++d) {
                double k = kn[io + d], v = vn[io + d];
                Ks[row + d] = round_bf16 ? orc_round_bf16(k) : k;
                Vs[row + d] = round_bf16 ? orc_round_bf16(v) : v;
            }
            double* sc = (double*)malloc(sizeof(double) * (size_t)(pos + 1));
            attend_one(pos + 1, D, scale, q + io, Ks + base, Vs + base,
                       out + io, sc);
            free(sc);
        }
}

/* Several new rows at once, with grouped key/value heads ([WK] section 3
 * lists the MHA/GQA/MQA head sharing; the ContextPrefill of [WK] section 5
 * starts the decoder from several prefix positions at once). Shapes:
 *   q, out [S][n][Hq][D];  kn, vn [S][n][Hkv][D];  Ks, Vs [S][Hkv][max_pos][D].
 * First rows pos .. pos+n-1 of every (sequence, kv head) are written (rounded
 * to bf16 when asked); then query i of head h attends, causally, rows
 * 0 .. pos+i of kv head h / (Hq / Hkv), the last n of them being the rows
 * just written. */
void orc_self_prefill_append(int S, int n, int Hq, int Hkv, int D, int max_pos, int pos,
                             double scale, int round_bf16, const double* q,
                             const double* kn, const double* vn, double* Ks,
                             double* Vs, double* out)
{
    for (int s = 0; s < S; ++s)
        for (int i = 0; i < n; ++i)
            for (int hk = 0; hk < Hkv; ++hk) {
                size_t row = (((size_t)s * Hkv + hk) * max_pos + pos + i) * D;
                size_t io = (((size_t)s * n + i) * Hkv + hk) * D;
                for (int d = 0; d < D; ++d) {
                    double k = kn[io + d], v = vn[io + d];
                    Ks[row + d] = round_bf16 ? orc_round_bf16(k) : k;
                    Vs[row + d] = round_bf16 ? orc_round_bf16(v) : v;
                }
            }
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(3) schedule(static)
    for (int s = 0; s < S; ++s)
        for (int i = 0; i < n; ++i)
            for (int h = 0; h < Hq; ++h) {
                size_t base = ((size_t)s * Hkv + h / G) * (size_t)max_pos * D;
                size_t qi = (((size_t)s * n + i) * Hq + h) * D;
                double* sc = (double*)malloc(sizeof(double) * (size_t)(pos + i + 1));
                attend_one(pos + i + 1, D, scale, q + qi, Ks + base, Vs + base, out + qi, sc);
                free(sc);
            }
}

/* [WK] section 4: the ANE decoder updates its fixed-length cache with a
 * one-hot mask m (1 at the current position): cache*(1-m) + cur*m, applied to
 * every row. Exported so the scatter above can be checked against it. */
void orc_kv_blend_update(int S, int H, int D, int max_pos, int pos,
                         const double* cur, double* cache)
{
    for (int s = 0; s < S; ++s)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < max_pos; ++t) {
                double m = (t == pos) ? 1.0 : 0.0;
                size_t row = (((size_t)s * H + h) * max_pos + t) * D;
                size_t io = ((size_t)s * H + h) * D;
                for (int d = 0; d < D; ++d)
                    cache[row + d] =
                        cache[row + d] * (1.0 - m) + cur[io + d] * m;
            }
}

/* --------------------------------------------------- projector memory lift
 * [GRN] "Forward map - granite_nar", "Projector (NLE simplified Q-Former)":
 * the projector's key/value memory is the GELU (the exact, erf-based one) of
 * a linear lift of the normalised 4-way encoder concat, plus the window
 * position embedding broadcast over the blocks of pos_rows frames:
 *   out[r][j] = gelu(sum_c x[r][c] W[c][j]) + pos[r % pos_rows][j]
 * x is [rows][k_in], W [k_in][n], pos [pos_rows][n] (NULL: no positions),
 * out [rows][n]. No bias (the page's linear names only a weight).
 */
static double gelu_exact(double v) { return 0.5 * v * (1.0 + erf(v / sqrt(2.0))); }

void orc_lift_gelu(int rows, int k_in, int n, const double* x, const double* W,
                   const double* pos, int pos_rows, double* out)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        double* o = out + (size_t)r * n;
        for (int j = 0; j < n; ++j) o[j] = 0.0;
        /* every o[j] still sums its k_in products in ascending c order */
        for (int c = 0; c < k_in; ++c) {
            const double xv = x[(size_t)r * k_in + c];
            const double* w = W + (size_t)c * n;
            for (int j = 0; j < n; ++j) o[j] += xv * w[j];
        }
        for (int j = 0; j < n; ++j)
            o[j] = gelu_exact(o[j]) + (pos ? pos[(size_t)(r % pos_rows) * n + j] : 0.0);
    }
}

double orc_gelu(double v) { return gelu_exact(v); }

/* ------------------------------------------------- harness decoder (O4/O5)
 * The workloads give projection weights but no norm, MLP or vocabulary, so the
 * decoder used to drive whole decode runs is the plainest one the pages allow:
 * per layer, in the decoder-body order of [CKE] "The concept" (self-attention
 * residual, then cross-attention, then the MLP, which has no weights here):
 *   qs = x.WQs, ks = x.WKs, vs = x.WVs
 *   x += SelfAttn(qs, ks, vs; cache, pos) . WOs
 *   qc = x.WQ
 *   x += CrossAttn(qc; projection cache of layer l) . WO
 * and the next token's input is x / rms(x). S = B*nq self sequences; sequence
 * s reads stream s / nq of the cross cache as its query s % nq.
 */
static void matvec(int dm, int n_out, const double* x, const double* W,
                   double* y)
{
    for (int j = 0; j < n_out; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dm; ++c) acc += x[c] * W[(size_t)c * n_out + j];
        y[j] = acc;
    }
}

static void add_matvec(int dm, const double* a, const double* W, double* x)
{
    for (int j = 0; j < dm; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dm; ++c) acc += a[c] * W[(size_t)c * dm + j];
        x[j] = x[j] + acc;
    }
}

static void rms_feedback(int dm, const double* x, double* y)
{
    double ss = 0.0;
    for (int c = 0; c < dm; ++c) ss += x[c] * x[c];
    double r = sqrt(ss / dm);
    for (int c = 0; c < dm; ++c) y[c] = x[c] / r;
}

/* Exported for the tests that build teacher-forced per-call inputs. */
void orc_matvec(int dm, int n_out, const double* x, const double* W, double* y)
{
    matvec(dm, n_out, x, W, y);
}

void orc_rms_feedback(int dm, const double* x, double* y)
{
    rms_feedback(dm, x, y);
}

/*
 * One decoder layer for one token of each of S = B*nq sequences, the body of
 * the harness decoder above: x ([S][dm]) is updated in place, the self-
 * attention row pos of every (sequence, head) is written into Ks, Vs
 * ([S][H][max_pos][D], rounded to bf16 when round_bf16), and sequence s
 * reads stream s / nq of the layer's projection-cache slab Kc, Vc
 * ([B][H][T][D]). Weights are [dm][dm] (y = x.W). rec_* ([S][dm], nullable)
 * receive the self query, new key, new value, self-attention output, cross
 * query and cross-attention output. Returns -1 for a bad geometry.
 */
int orc_decoder_layer_step(int S, int nq, int T, int dm, int H, int D,
                           int max_pos, int pos, double scale, int round_bf16,
                           double* x, const double* WQs, const double* WKs,
                           const double* WVs, const double* WOs,
                           const double* WQ, const double* WO,
                           const double* Kc, const double* Vc, double* Ks,
                           double* Vs, double* rec_qs, double* rec_kn,
                           double* rec_vn, double* rec_so, double* rec_qc,
                           double* rec_co)
{
    if (H * D != dm || T <= 0 || nq <= 0 || S % nq != 0 || pos < 0 || pos >= max_pos)
        return -1;
    double* qs = (double*)malloc(sizeof(double) * (size_t)dm);
    double* ks = (double*)malloc(sizeof(double) * (size_t)dm);
    double* vs = (double*)malloc(sizeof(double) * (size_t)dm);
    double* so = (double*)malloc(sizeof(double) * (size_t)dm);
    double* qc = (double*)malloc(sizeof(double) * (size_t)dm);
    double* co = (double*)malloc(sizeof(double) * (size_t)dm);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(T > max_pos ? T : max_pos));
    for (int s = 0; s < S; ++s) {
        const int b = s / nq;
        double* xr = x + (size_t)s * dm;
        matvec(dm, dm, xr, WQs, qs);
        matvec(dm, dm, xr, WKs, ks);
        matvec(dm, dm, xr, WVs, vs);
        for (int h = 0; h < H; ++h) {
            double* kh = Ks + (((size_t)s * H + h) * max_pos) * D;
            double* vh = Vs + (((size_t)s * H + h) * max_pos) * D;
            for (int d = 0; d < D; ++d) {
                kh[(size_t)pos * D + d] = round_bf16 ? orc_round_bf16(ks[h * D + d]) : ks[h * D + d];
                vh[(size_t)pos * D + d] = round_bf16 ? orc_round_bf16(vs[h * D + d]) : vs[h * D + d];
            }
            attend_one(pos + 1, D, scale, qs + h * D, kh, vh, so + h * D, sc);
        }
        add_matvec(dm, so, WOs, xr);
        matvec(dm, dm, xr, WQ, qc);
        for (int h = 0; h < H; ++h) {
            const size_t slab = (((size_t)b * H + h) * T) * D;
            attend_one(T, D, scale, qc + h * D, Kc + slab, Vc + slab, co + h * D, sc);
        }
        add_matvec(dm, co, WO, xr);
        if (rec_qs) memcpy(rec_qs + (size_t)s * dm, qs, sizeof(double) * dm);
        if (rec_kn) memcpy(rec_kn + (size_t)s * dm, ks, sizeof(double) * dm);
        if (rec_vn) memcpy(rec_vn + (size_t)s * dm, vs, sizeof(double) * dm);
        if (rec_so) memcpy(rec_so + (size_t)s * dm, so, sizeof(double) * dm);
        if (rec_qc) memcpy(rec_qc + (size_t)s * dm, qc, sizeof(double) * dm);
        if (rec_co) memcpy(rec_co + (size_t)s * dm, co, sizeof(double) * dm);
    }
    free(qs); free(ks); free(vs); free(so); free(qc); free(co); free(sc);
    return 0;
}

/*
 * Record layout (each nullable): rec_* are [n_steps][L][S][dm] holding, per
 * step and layer, the self query, new key, new value, self-attention output,
 * cross query and cross-attention output. x_seq is [n_steps+1][S][dm].
 * Kc, Vc ([L][B][H][T][D]) receive the cross caches and Ks, Vs
 * ([L][S][H][max_pos][D]) the self caches; in full-window mode they receive
 * the values recomputed in the last window.
 *
 * mode 0 (incremental): project E once into the cross cache ([CKE] "View 3":
 *   once per window, reused by every step), then each step appends one row to
 *   the self cache and attends.
 * mode 1 (full window, [TOP] "What it opened"): every step re-runs the whole
 *   window 0..t from the token inputs with no cache at all: E is re-projected
 *   and every position's self K/V row is recomputed. Only position t's values
 *   are recorded. The two modes must agree bit for bit.
 */
int orc_decoder_run(int mode, int L, int B, int nq, int T, int dm, int H,
                    int D, int max_pos, int n_steps, double scale,
                    int round_bf16, const double* E, const double* WK,
                    const double* WV, const double* WQ, const double* WO,
                    const double* WQs, const double* WKs, const double* WVs,
                    const double* WOs, const double* x0, double* rec_qs,
                    double* rec_kn, double* rec_vn, double* rec_so,
                    double* rec_qc, double* rec_co, double* x_seq, double* Kc,
                    double* Vc, double* Ks, double* Vs)
{
    if (H * D != dm || T <= 0 || n_steps > max_pos || n_steps < 0) return -1;
    const int S = B * nq;
    const size_t ws = (size_t)dm * dm;
    const size_t cross_n = (size_t)L * B * H * T * D;
    const size_t self_n = (size_t)L * S * H * max_pos * D;
    double* xs = (double*)calloc((size_t)(n_steps + 1) * S * dm, sizeof(double));
    double* qs = (double*)malloc(sizeof(double) * (size_t)dm);
    double* so = (double*)malloc(sizeof(double) * (size_t)dm);
    double* qc = (double*)malloc(sizeof(double) * (size_t)dm);
    double* co = (double*)malloc(sizeof(double) * (size_t)dm);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(T > max_pos ? T : max_pos));
    double* kc = (double*)malloc(sizeof(double) * cross_n);
    double* vc = (double*)malloc(sizeof(double) * cross_n);
    double* kself = (double*)calloc(self_n, sizeof(double));
    double* vself = (double*)calloc(self_n, sizeof(double));
    memcpy(xs, x0, sizeof(double) * (size_t)S * dm);

#define REC(p, t, l, s) ((p) + ((((size_t)(t) * L + (l)) * S + (s)) * dm))
#define XC(l, b, h) ((((size_t)(l) * B + (b)) * H + (h)) * (size_t)T * D)
#define XS(l, s, h) ((((size_t)(l) * S + (s)) * H + (h)) * (size_t)max_pos * D)

    if (mode == 0) {
        /* Populate once: per layer, per stream, per head. */
        for (int l = 0; l < L; ++l)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < H; ++h) {
                    orc_project_head(T, dm, D, E + (size_t)b * T * dm,
                                     WK + l * ws, dm, h * D, round_bf16,
                                     kc + XC(l, b, h));
                    orc_project_head(T, dm, D, E + (size_t)b * T * dm,
                                     WV + l * ws, dm, h * D, round_bf16,
                                     vc + XC(l, b, h));
                }
        /* every step runs the layers in order, each as one layer step over
         * all sequences; the sequences' hidden states live in xt */
        double* xt = (double*)malloc(sizeof(double) * (size_t)S * dm);
        for (int t = 0; t < n_steps; ++t) {
            memcpy(xt, xs + (size_t)t * S * dm, sizeof(double) * (size_t)S * dm);
            for (int l = 0; l < L; ++l)
                orc_decoder_layer_step(S, nq, T, dm, H, D, max_pos, t, scale, round_bf16, xt,
                                       WQs + l * ws, WKs + l * ws, WVs + l * ws, WOs + l * ws,
                                       WQ + l * ws, WO + l * ws, kc + XC(l, 0, 0),
                                       vc + XC(l, 0, 0), kself + XS(l, 0, 0),
                                       vself + XS(l, 0, 0),
                                       rec_qs ? REC(rec_qs, t, l, 0) : NULL,
                                       rec_kn ? REC(rec_kn, t, l, 0) : NULL,
                                       rec_vn ? REC(rec_vn, t, l, 0) : NULL,
                                       rec_so ? REC(rec_so, t, l, 0) : NULL,
                                       rec_qc ? REC(rec_qc, t, l, 0) : NULL,
                                       rec_co ? REC(rec_co, t, l, 0) : NULL);
            for (int s = 0; s < S; ++s)
                rms_feedback(dm, xt + (size_t)s * dm, xs + ((size_t)(t + 1) * S + s) * dm);
        }
        free(xt);
    } else {
        /* Full-window recompute, no cache carried between steps. */
        double* hid = (double*)malloc(sizeof(double) * (size_t)max_pos * dm);
        double* wk = (double*)malloc(sizeof(double) * (size_t)max_pos * D);
        double* wv = (double*)malloc(sizeof(double) * (size_t)max_pos * D);
        double* kall = (double*)malloc(sizeof(double) * (size_t)max_pos * dm);
        double* vall = (double*)malloc(sizeof(double) * (size_t)max_pos * dm);
        for (int t = 0; t < n_steps; ++t) {
            /* Re-project E for this window: a fresh loop, not the cache. */
            for (int l = 0; l < L; ++l)
                for (int b = 0; b < B; ++b)
                    for (int h = 0; h < H; ++h)
                        for (int r = 0; r < T; ++r)
                            for (int d = 0; d < D; ++d) {
                                double ak = 0.0, av = 0.0;
                                const double* e = E + ((size_t)b * T + r) * dm;
                                for (int c = 0; c < dm; ++c) {
                                    ak += e[c] * WK[l * ws + (size_t)c * dm + h * D + d];
                                    av += e[c] * WV[l * ws + (size_t)c * dm + h * D + d];
                                }
                                size_t o = XC(l, b, h) + (size_t)r * D + d;
                                kc[o] = round_bf16 ? orc_round_bf16(ak) : ak;
                                vc[o] = round_bf16 ? orc_round_bf16(av) : av;
                            }
            for (int s = 0; s < S; ++s) {
                const int b = s / nq;
                /* hidden state of every position 0..t entering layer 0 */
                for (int p = 0; p <= t; ++p)
                    memcpy(hid + (size_t)p * dm, xs + ((size_t)p * S + s) * dm,
                           sizeof(double) * dm);
                for (int l = 0; l < L; ++l) {
                    /* all positions' self K/V rows of this layer, unrounded */
                    for (int p = 0; p <= t; ++p) {
                        matvec(dm, dm, hid + (size_t)p * dm, WKs + l * ws, kall + (size_t)p * dm);
                        matvec(dm, dm, hid + (size_t)p * dm, WVs + l * ws, vall + (size_t)p * dm);
                    }
                    for (int p = 0; p <= t; ++p) {
                        double* x = hid + (size_t)p * dm;
                        matvec(dm, dm, x, WQs + l * ws, qs);
                        for (int h = 0; h < H; ++h) {
                            for (int r = 0; r <= p; ++r)
                                for (int d = 0; d < D; ++d) {
                                    double kv = kall[(size_t)r * dm + h * D + d];
                                    double vv = vall[(size_t)r * dm + h * D + d];
                                    wk[(size_t)r * D + d] = round_bf16 ? orc_round_bf16(kv) : kv;
                                    wv[(size_t)r * D + d] = round_bf16 ? orc_round_bf16(vv) : vv;
                                }
                            attend_one(p + 1, D, scale, qs + h * D, wk, wv, so + h * D, sc);
                        }
                        if (p == t) {
                            if (rec_qs) memcpy(REC(rec_qs, t, l, s), qs, sizeof(double) * dm);
                            if (rec_kn) memcpy(REC(rec_kn, t, l, s), kall + (size_t)p * dm, sizeof(double) * dm);
                            if (rec_vn) memcpy(REC(rec_vn, t, l, s), vall + (size_t)p * dm, sizeof(double) * dm);
                            if (rec_so) memcpy(REC(rec_so, t, l, s), so, sizeof(double) * dm);
                        }
                        add_matvec(dm, so, WOs + l * ws, x);
                        matvec(dm, dm, x, WQ + l * ws, qc);
                        for (int h = 0; h < H; ++h)
                            attend_one(T, D, scale, qc + h * D, kc + XC(l, b, h),
                                       vc + XC(l, b, h), co + h * D, sc);
                        add_matvec(dm, co, WO + l * ws, x);
                        if (p == t) {
                            if (rec_qc) memcpy(REC(rec_qc, t, l, s), qc, sizeof(double) * dm);
                            if (rec_co) memcpy(REC(rec_co, t, l, s), co, sizeof(double) * dm);
                        }
                    }
                    /* the self cache of this layer as the last window sees it */
                    if (t == n_steps - 1)
                        for (int p = 0; p <= t; ++p)
                            for (int h = 0; h < H; ++h)
                                for (int d = 0; d < D; ++d) {
                                    double kv = kall[(size_t)p * dm + h * D + d];
                                    double vv = vall[(size_t)p * dm + h * D + d];
                                    kself[XS(l, s, h) + (size_t)p * D + d] = round_bf16 ? orc_round_bf16(kv) : kv;
                                    vself[XS(l, s, h) + (size_t)p * D + d] = round_bf16 ? orc_round_bf16(vv) : vv;
                                }
                }
                rms_feedback(dm, hid + (size_t)t * dm,
                             xs + ((size_t)(t + 1) * S + s) * dm);
            }
        }
        free(hid); free(wk); free(wv); free(kall); free(vall);
    }

    if (x_seq) memcpy(x_seq, xs, sizeof(double) * (size_t)(n_steps + 1) * S * dm);
    if (Kc) memcpy(Kc, kc, sizeof(double) * cross_n);
    if (Vc) memcpy(Vc, vc, sizeof(double) * cross_n);
    if (Ks) memcpy(Ks, kself, sizeof(double) * self_n);
    if (Vs) memcpy(Vs, vself, sizeof(double) * self_n);
#undef REC
#undef XC
#undef XS
    free(xs); free(qs); free(so); free(qc);
    free(co); free(sc); free(kc); free(vc); free(kself); free(vself);
    return 0;
}
