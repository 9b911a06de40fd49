/*
 * Oracle: a plain, slow, f64 CPU forward of packed bidirectional encoder / DiT
 * blocks.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
 * CPU-baseline leg are the only callers.  It shares no code, header, table or
 * helper with the HIP library, and the library never calls it.
 *
 * Every step is the plain definition of what the pages compute, evaluated in
 * f64 in the order written, with inputs widened exactly from f32 / int8.  The
 * only blocking is none; the only parallelism is OpenMP over independent rows,
 * (item, head, query) triples or output columns.  Sources (the three pages):
 *   [EG]  cortiq-engine 0.8.39, src/gpu_metal/egemma2.rs (EmbeddingGemma 2 on Metal)
 *   [ZI]  cortiq-engine 0.7.6,  src/gpu_metal/zimage.rs  (Z-Image DiT on Metal)
 *   [VE]  cera 0.2.4, src/model/vision_encoder_gpu.rs    (LFM2-VL ViT)
 * Readings where the pages are silent are listed next to the code they shape.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_API __attribute__((visibility("default")))

/* OpenMP threads the oracle's parallel loops use. */
OR_API int or_threads(void)
{
    return omp_get_max_threads();
}

/* ------------------------------------------------------------------ binary16 */

/* Round to the nearest IEEE-754 binary16 value, ties to even, returned as f64.
 * [ZI] module doc "The chain" and `Acts`: the int8 path stores its GEMM inputs,
 * the qkv panel, the attention output and the SwiGLU hidden as half.
 * binary16: 11 significant bits, exponents 2^-14..2^15, subnormal step 2^-24,
 * max finite 65504; magnitudes from 65520 up round to infinity. */
OR_API double or_round_f16(double x)
{
    if (isnan(x) || isinf(x))
        return x;
    double a = fabs(x);
    if (a >= 65520.0)
        return copysign(INFINITY, x);
    if (a == 0.0)
        return x;
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int q = e - 11; /* spacing of 11-bit significands in that binade */
    if (q < -24)
        q = -24; /* subnormal spacing */
    double ulp = ldexp(1.0, q);
    double r = nearbyint(a / ulp) * ulp; /* default rounding mode: ties to even */
    return copysign(r, x);
}

static void round_f16_array(double *v, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        v[i] = or_round_f16(v[i]);
}

/* --------------------------------------------------------------------- norms */

/* RMSNorm of one row: y = x * w / sqrt(mean(x^2) + eps); the gain multiplies
 * directly (not 1 + w).  [EG] `Prog::rms` ("Y = rms(pre·X)·w"); w == NULL is
 * the weightless form of [EG] `eg_row_inv` / the pool. */
static void rms_row(const double *x, const float *w, int d, double eps, double *y)
{
    double ss = 0.0;
    for (int j = 0; j < d; j++)
        ss += x[j] * x[j];
    double inv = 1.0 / sqrt(ss / d + eps);
    for (int j = 0; j < d; j++)
        y[j] = x[j] * inv * (w ? (double)w[j] : 1.0);
}

/* LayerNorm of one row with population variance, eps inside the root:
 * y = (x - mean) / sqrt(var + eps) * w + b.  [VE] `VitGpuOps::layernorm`. */
static void ln_row(const double *x, const float *w, const float *b, int d, double eps, double *y)
{
    double mu = 0.0;
    for (int j = 0; j < d; j++)
        mu += x[j];
    mu /= d;
    double var = 0.0;
    for (int j = 0; j < d; j++)
        var += (x[j] - mu) * (x[j] - mu);
    var /= d;
    double inv = 1.0 / sqrt(var + eps);
    for (int j = 0; j < d; j++)
        y[j] = (x[j] - mu) * inv * (double)w[j] + (b ? (double)b[j] : 0.0);
}

OR_API void or_rms_norm(int64_t n, int d, const double *x, const float *w, double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        rms_row(x + i * d, w, d, eps, y + i * d);
}

OR_API void or_layer_norm(int64_t n, int d, const double *x, const float *w, const float *b,
                          double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        ln_row(x + i * d, w, b, d, eps, y + i * d);
}

/* ---------------------------------------------------------------- activations */

/* GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).  Named by
 * [EG] `Prog::gelu` and [VE] `VitGpuOps::gelu`; the pages print no constants, so
 * these are the textbook ones of that approximation. */
OR_API double or_gelu_tanh(double x)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* SiLU: x / (1 + e^-x).  [ZI] `PSw` / the SwiGLU step of the block. */
OR_API double or_silu(double x)
{
    return x / (1.0 + exp(-x));
}

/* --------------------------------------------------------------------- linear */

/* y[i][j] = sum_k x[i][k] * W[j][k] (+ b[j]); W is [m][k] row-major (the
 * nn.Linear layout, [VE] `VitGpuOps::linear`).  Each output is summed over k in
 * increasing order.  W is first widened into a [k][m] copy so the loop over j
 * runs along memory; the arithmetic per output is unchanged. */
OR_API void or_linear(int64_t n, int k, int m, const double *x, const float *w, const float *b,
                      double *y)
{
    double *wt = (double *)malloc(sizeof(double) * (size_t)k * m);
    for (int j = 0; j < m; j++)
        for (int kk = 0; kk < k; kk++)
            wt[(size_t)kk * m + j] = (double)w[(size_t)j * k + kk];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double *yi = y + i * m;
        for (int j = 0; j < m; j++)
            yi[j] = 0.0;
        for (int kk = 0; kk < k; kk++) {
            double xv = x[i * k + kk];
            const double *wr = wt + (size_t)kk * m;
            for (int j = 0; j < m; j++)
                yi[j] += xv * wr[j];
        }
        if (b)
            for (int j = 0; j < m; j++)
                yi[j] += (double)b[j];
    }
    free(wt);
}

/* int8 row-scaled weight: y[i][j] = rs[j] * sum_k q[j][k] * x[i][k].
 * [ZI] module doc "The chain": the int8 tile is used exactly (as half) and the
 * per-output-row scale is applied after the sum; `bench_gemm`'s host check is
 * the same formula. */
OR_API void or_linear_q8(int64_t n, int k, int m, const double *x, const int8_t *q,
                         const float *rs, double *y)
{
    double *wt = (double *)malloc(sizeof(double) * (size_t)k * m);
    for (int j = 0; j < m; j++)
        for (int kk = 0; kk < k; kk++)
            wt[(size_t)kk * m + j] = (double)q[(size_t)j * k + kk];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double *yi = y + i * m;
        for (int j = 0; j < m; j++)
            yi[j] = 0.0;
        for (int kk = 0; kk < k; kk++) {
            double xv = x[i * k + kk];
            const double *wr = wt + (size_t)kk * m;
            for (int j = 0; j < m; j++)
                yi[j] += xv * wr[j];
        }
        for (int j = 0; j < m; j++)
            yi[j] *= (double)rs[j];
    }
    free(wt);
}

/* ------------------------------------------------------------ items, positions */

/* One packed item: up to two row ranges, its rows taken in order (first range,
 * then the second).  [ZI] `PFa` (image range + caption range) and the module
 * doc's CFG program; a text sequence is a single range ([EG] the segment table
 * of `TextGpu::forward`).  grid > 0 marks a 2-D item: its first grid*grid rows
 * form a grid x grid image in row-major order. */
typedef struct {
    int32_t nr;
    int32_t r0[2];
    int32_t n[2];
    int32_t grid;
} or_item;

static int item_len(const or_item *it)
{
    int L = 0;
    for (int r = 0; r < it->nr; r++)
        L += it->n[r];
    return L;
}

/* physical row of the item's t-th row */
static int item_row(const or_item *it, int t)
{
    return t < it->n[0] ? it->r0[0] + t : it->r0[1] + (t - it->n[0]);
}

/* RoPE positions of every row, pos[row][0..sections-1].
 * 1-D: the row's index within its sequence, restarting at 0 per sequence
 *      ([EG] `TextGpu::forward`, `pos.extend(0..len)`).
 * 2-D: (column, row) of an image row in its grid; a caption row j of a grid-G
 *      item sits at (G + j, G + j).  The pages build these tables on the host
 *      without showing them; this diagonal continuation is the reading taken. */
OR_API void or_positions(int nitems, const or_item *items, int sections, int32_t *pos)
{
    for (int i = 0; i < nitems; i++) {
        const or_item *it = &items[i];
        int L = item_len(it);
        for (int t = 0; t < L; t++) {
            int row = item_row(it, t);
            if (sections == 1) {
                pos[row] = t;
            } else if (sections == 2) {
                int G = it->grid, c, r;
                if (t < G * G) {
                    c = t % G;
                    r = t / G;
                } else {
                    c = G + (t - G * G);
                    r = c;
                }
                pos[2 * row + 0] = c;
                pos[2 * row + 1] = r;
            }
        }
    }
}

/* ----------------------------------------------------------------------- RoPE */

/* Rotary embedding of one head vector x[hd] in place, rotate_half within each
 * section of S channels ([EG] `EgQkv.sec`): for i < S/2,
 *   theta = p * base^(-2i/S)
 *   y[i]       = x[i] cos(theta) - x[i+S/2] sin(theta)
 *   y[i+S/2]   = x[i+S/2] cos(theta) + x[i] sin(theta)
 * 1-D: one section, S = hd, p = position.  2-D: two sections of S = hd/2, the
 * first rotated by the column, the second by the row ([EG] `VisionGpu::forward`
 * doc: "the column half, then the row half"). */
static void rope_head(double *x, int hd, int sections, const int32_t *p, double base)
{
    int S = hd / sections;
    for (int s = 0; s < sections; s++) {
        double *v = x + s * S;
        for (int i = 0; i < S / 2; i++) {
            double th = (double)p[s] * pow(base, -2.0 * i / S);
            double c = cos(th), sn = sin(th);
            double a = v[i], b = v[i + S / 2];
            v[i] = a * c - b * sn;
            v[i + S / 2] = b * c + a * sn;
        }
    }
}

/* q/k per-head RMSNorm then RoPE, in place on q [rows][nh*hd] ([EG]
 * `Prog::qkv` "q/k norm + RoPE"; norm first, then the rotation). */
OR_API void or_qk_norm_rope(int64_t rows, int nh, int hd, double *x, const float *w, double eps,
                            int sections, const int32_t *pos, double base)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int h = 0; h < nh; h++) {
            double *v = x + (r * nh + h) * hd;
            rms_row(v, w, hd, eps, v);
            if (sections > 0)
                rope_head(v, hd, sections, pos + r * sections, base);
        }
    }
}

/* ------------------------------------------------------------------ attention */

/* Non-causal softmax attention per item and head:
 *   o_i = sum_{j in V(i)} e^{s_ij - m_i} v_j / sum_{j in V(i)} e^{s_ij - m_i},
 *   s_ij = scale * q_i . k_j,  m_i = max_{j in V(i)} s_ij,
 * with V(i) the item's rows t_j such that window == 0 or |t_i - t_j| <= window
 * (t = index in the item's row order).  [EG] module doc "Attention" and
 * `att_plan` (key span [q0 - W, q_last + W], clipped to the sequence);
 * [ZI] `PFa` (an item = its image and caption ranges).  GQA: query head h reads
 * kv head h / (nq / nkv) ([EG] `att_plan`).  q/k/v/o are [rows][ld*] with the
 * head's hd columns at h*hd. */
static void attention_impl(int nitems, const or_item *items, int nq, int nkv, int hd,
                           const double *q, int ldq, const double *k, int ldk, const double *v,
                           int ldv, double *o, int ldo, double scale, int window,
                           const char *qsel)
{
    for (int ii = 0; ii < nitems; ii++) {
        const or_item *it = &items[ii];
        int L = item_len(it);
        int group = nq / nkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
        for (int h = 0; h < nq; h++) {
            for (int ti = 0; ti < L; ti++) {
                int kvh = h / group;
                int ri = item_row(it, ti);
                if (qsel && !qsel[ri])
                    continue;
                const double *qi = q + (int64_t)ri * ldq + h * hd;
                double *s = (double *)malloc(sizeof(double) * L);
                char *vis = (char *)malloc((size_t)L);
                double m = -INFINITY;
                for (int tj = 0; tj < L; tj++) {
                    vis[tj] = window == 0 || abs(ti - tj) <= window;
                    if (!vis[tj])
                        continue;
                    const double *kj = k + (int64_t)item_row(it, tj) * ldk + kvh * hd;
                    double dot = 0.0;
                    for (int c = 0; c < hd; c++)
                        dot += qi[c] * kj[c];
                    s[tj] = scale * dot;
                    if (s[tj] > m)
                        m = s[tj];
                }
                double den = 0.0;
                for (int tj = 0; tj < L; tj++) {
                    if (!vis[tj])
                        continue;
                    s[tj] = exp(s[tj] - m);
                    den += s[tj];
                }
                double *oi = o + (int64_t)ri * ldo + h * hd;
                for (int c = 0; c < hd; c++) {
                    double acc = 0.0;
                    for (int tj = 0; tj < L; tj++)
                        if (vis[tj])
                            acc += s[tj] * v[(int64_t)item_row(it, tj) * ldv + kvh * hd + c];
                    oi[c] = acc / den;
                }
                free(vis);
                free(s);
            }
        }
    }
}

OR_API void or_attention(int nitems, const or_item *items, int nq, int nkv, int hd,
                         const double *q, int ldq, const double *k, int ldk, const double *v,
                         int ldv, double *o, int ldo, double scale, int window)
{
    attention_impl(nitems, items, nq, nkv, hd, q, ldq, k, ldk, v, ldv, o, ldo, scale, window,
                   NULL);
}

/* The same attention for the query rows r with qsel[r] != 0 only (the other
 * output rows are left untouched): the full-size checks sample query rows. */
OR_API void or_attention_rows(int nitems, const or_item *items, int nq, int nkv, int hd,
                              const double *q, int ldq, const double *k, int ldk,
                              const double *v, int ldv, double *o, int ldo, double scale,
                              int window, const char *qsel)
{
    attention_impl(nitems, items, nq, nkv, hd, q, ldq, k, ldk, v, ldv, o, ldo, scale, window,
                   qsel);
}

/* ---------------------------------------------------------------------- model */

enum { OR_PRE_LN = 0, OR_SANDWICH = 1 };
enum { OR_F32 = 0, OR_I8F16 = 1 };
enum { OR_GELU = 0, OR_GELU_GATED = 1, OR_SWIGLU = 2 };
enum { OR_FINAL_NONE = 0, OR_FINAL_LN = 1, OR_FINAL_RMS_MEANPOOL = 2 };

typedef struct {
    int32_t block, path, mlp;
    int32_t d, nq, nkv, hd, ff, window, rope_sections;
    double eps, attn_scale, rope_base;
    /* f32 path: float [out][in]; int8 path: int8 [out][in] + float row scales */
    const float *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
    const int8_t *qq, *qk, *qv, *qo, *q_gate, *q_up, *q_down;
    const float *sq, *sk, *sv, *so, *s_gate, *s_up, *s_down;
    const float *bq, *bk, *bv, *bo, *b_up, *b_down; /* nullable */
    /* pre-LN: norm1 = LN before attention, norm2 = LN before the MLP (w and b).
     * sandwich: norm1 = pre-attention RMS, post_attn, norm2 = pre-FF RMS,
     * post_ff; q_norm/k_norm per head. */
    const float *norm1_w, *norm1_b, *norm2_w, *norm2_b;
    const float *post_attn_w, *post_ff_w, *q_norm_w, *k_norm_w;
    /* text-encoder options of [EG] `LayerSpec` / `TextSpec` (sandwich block):
     * v_norm: weightless RMS of every v head ([EG] `Prog::qkv`, "v norm");
     * scalar: the layer's last residual update is H = (H + .) * scalar
     *   ([EG] `Prog::add_norm` "H = (H + rms(T)·w)·post", post = the layer
     *   scalar); 0 is read as 1;
     * n_ple > 0: the per-layer-input branch ([EG] `TextGpu::forward`, "per-layer
     *   input") with ple_in, ple_gate [n_ple][d], ple_proj [d][n_ple], the
     *   model-wide ple_in_norm_w [n_ple] and this layer's ple_post_w [d]. */
    int32_t v_norm, n_ple;
    double scalar, ple_scale;
    const float *ple_in, *ple_gate, *ple_proj, *ple_in_norm_w, *ple_post_w;
    /* the int8 DiT block's row-op contract ([ZI] `Enc::block`, `Enc::rowop`,
     * module doc "The chain"):
     * mod_*: adaLN modulation [d], NULL = off ([ZI] `block`: this block's
     *   [s_msa|g_msa|s_mlp|g_mlp]): a pre-norm output is multiplied by
     *   (1 + s), a residual update by g (s = 0, g = 1 is the unmodulated form
     *   of [ZI] `refine_caption`);
     * col_*: the q8_2f column field [in] of each weight, NULL = ones:
     *   W_eff[j][k] = rs[j] q[j][k] col[k], folded into the half input by its
     *   producer (the row op for q/k/v and w1/w3, the attention epilogue for
     *   the O projection, SwiGLU for w2);
     * guard_*: [ZI] `Guards`: the half site stores x 2^-s and its consumer
     *   multiplies 2^s back (int8 path). */
    const float *mod_s_attn, *mod_g_attn, *mod_s_ff, *mod_g_ff;
    const float *col_q, *col_k, *col_v, *col_o, *col_gate, *col_up, *col_down;
    int32_t guard_attn, guard_qkv, guard_ao, guard_ffn, guard_hid;
} or_layer;

typedef struct {
    int32_t d;
    int32_t nlayers;
    const or_layer *layers;
    int32_t final_kind;
    const float *final_w, *final_b;
    double final_eps;
} or_model;

/* y[i][k] = x[i][k] * (1 + s[k]) (s NULL: a copy) */
static void modulate(int64_t n, int d, const double *x, const float *s, double *y)
{
    for (int64_t i = 0; i < n; i++)
        for (int k = 0; k < d; k++)
            y[i * d + k] = x[i * d + k] * (s ? 1.0 + (double)s[k] : 1.0);
}

/* A half site of the int8 path: y = x * col[k] * 2^-guard, rounded to binary16
 * when r16 (col NULL: ones).  The amax slot (nullable) takes max |y|. */
static void half_site(int64_t n, int d, const double *x, const float *col, int guard, int r16,
                      double *y, double *amax)
{
    const double g = ldexp(1.0, -guard);
    for (int64_t i = 0; i < n; i++)
        for (int k = 0; k < d; k++) {
            double v = x[i * d + k] * (col ? (double)col[k] : 1.0) * g;
            if (r16)
                v = or_round_f16(v);
            y[i * d + k] = v;
            if (amax && fabs(v) > *amax)
                *amax = fabs(v);
        }
}

static void scale_all(double *v, int64_t n, double c)
{
    for (int64_t i = 0; i < n; i++)
        v[i] *= c;
}

/* One projection of the layer: f32 weight (+bias) or int8 weight x row scale. */
static void project(const or_layer *L, int64_t n, int k, int m, const double *x, const float *wf,
                    const int8_t *wq, const float *rs, const float *b, double *y)
{
    if (L->path == OR_F32)
        or_linear(n, k, m, x, wf, b, y);
    else
        or_linear_q8(n, k, m, x, wq, rs, y);
}

static void maybe_f16(int on, double *v, int64_t n)
{
    if (on)
        round_f16_array(v, n);
}

/* One layer over the packed rows, H updated in place.
 *
 * Sandwich block ([EG] `TextGpu::forward` layer loop; [ZI] module doc "The
 * chain" and `Enc::block`):
 *   A = rms(H; norm1)                         [f16 site on the int8 path]
 *   q|k|v = A W^T                             [f16 site]
 *   q_h, k_h = rope(rms(.; q_norm | k_norm))  [f16 site]
 *   att = attention(q, k, v)                  [f16 site]
 *   T = att Wo^T;  H += rms(T; post_attn)
 *   A = rms(H; norm2)                         [f16 site]
 *   m = act(A Wg^T) * (A Wu^T)                [f16 site] (gelu_tanh or silu)
 *   T = m Wd^T;  H += rms(T; post_ff)
 * Pre-LN block ([VE] `encode_image_gpu`, step 3):
 *   A = LN(H; norm1);  q|k|v = A W^T + b;  att = attention
 *   H += att Wo^T + bo;  A = LN(H; norm2);  H += gelu_tanh(A Wu^T + bu) Wd^T + bd
 * Options of the sandwich block: v_norm right after the q/k norm + RoPE; the
 * per-layer-input branch after the FFN, reading X0 (the forward's input rows);
 * the layer scalar multiplying H after the layer's last residual add; adaLN
 * modulation (each pre-norm output times (1 + s), each residual update times
 * g).  On the int8 path every half site stores x col 2^-guard (the column
 * field of the weight that reads it, its power-of-two guard) and the consumer
 * multiplies the guard back: the q/k/v and w1/w3 GEMM epilogues, the qk-norm's
 * eps (scaled by 2^-2 guard), the attention epilogue, the O and w2 epilogues.
 * `f16_sites` rounds to binary16 exactly where the int8 path stores half; 0
 * gives the pure-f64 diagnostic.  amax (nullable, [5]) takes max |stored
 * value| per site: q/k/v input, panel, attention output, w1/w3 input, hidden. */
static void layer_forward(const or_layer *L, int64_t rows, int nitems, const or_item *items,
                          const int32_t *pos, double *H, const double *X0, int f16_sites,
                          double *amax)
{
    int d = L->d, hd = L->hd, nq = L->nq, nkv = L->nkv, ff = L->ff;
    int qw = nq * hd, kw = nkv * hd;
    int i8 = L->path == OR_I8F16;
    int r16 = f16_sites && i8;
    /* guards exist on the int8 path only */
    int ga = i8 ? L->guard_attn : 0, gq = i8 ? L->guard_qkv : 0, gao = i8 ? L->guard_ao : 0;
    int gf = i8 ? L->guard_ffn : 0, gh = i8 ? L->guard_hid : 0;
    double *am = amax; /* [5]: xn, panel, attention out, FFN input, hidden */
    double *A = (double *)malloc(sizeof(double) * rows * d);
    double *Az = (double *)malloc(sizeof(double) * rows * d);
    double *Q = (double *)malloc(sizeof(double) * rows * qw);
    double *K = (double *)malloc(sizeof(double) * rows * kw);
    double *V = (double *)malloc(sizeof(double) * rows * kw);
    double *Att = (double *)malloc(sizeof(double) * rows * qw);
    double *T = (double *)malloc(sizeof(double) * rows * d);
    double *G = (double *)malloc(sizeof(double) * rows * ff);
    double *U = (double *)malloc(sizeof(double) * rows * ff);

    /* attention half */
    if (L->block == OR_SANDWICH) {
        or_rms_norm(rows, d, H, L->norm1_w, L->eps, A);
        modulate(rows, d, A, L->mod_s_attn, A);
    } else {
        or_layer_norm(rows, d, H, L->norm1_w, L->norm1_b, L->eps, A);
    }
    /* q, k, v each from its own half input A * col * 2^-ga; the GEMM epilogue
     * multiplies 2^(ga - gq) (undo the input guard, apply the panel's) */
    const float *cols[3] = {L->col_q, L->col_k, L->col_v};
    double *outs[3] = {Q, K, V};
    const int widths[3] = {qw, kw, kw};
    const float *wf[3] = {L->wq, L->wk, L->wv}, *rs[3] = {L->sq, L->sk, L->sv};
    const int8_t *wqq[3] = {L->qq, L->qk, L->qv};
    const float *bs[3] = {L->bq, L->bk, L->bv};
    for (int z = 0; z < 3; z++) {
        half_site(rows, d, A, cols[z], ga, r16, Az, am ? &am[0] : NULL);
        project(L, rows, d, widths[z], Az, wf[z], wqq[z], rs[z], bs[z], outs[z]);
        scale_all(outs[z], rows * widths[z], ldexp(1.0, ga - gq));
        half_site(rows, widths[z], outs[z], NULL, 0, r16, outs[z], am ? &am[1] : NULL);
    }
    if (L->block == OR_SANDWICH) {
        /* the panel holds x 2^-gq: eps scaled by 2^-2gq gives rms(x) exactly */
        double eps_q = L->eps * ldexp(1.0, -2 * gq);
        or_qk_norm_rope(rows, nq, hd, Q, L->q_norm_w, eps_q, L->rope_sections, pos, L->rope_base);
        or_qk_norm_rope(rows, nkv, hd, K, L->k_norm_w, eps_q, L->rope_sections, pos, L->rope_base);
        maybe_f16(r16, Q, rows * qw);
        maybe_f16(r16, K, rows * kw);
        if (L->v_norm) {
            /* every v head of every row is one hd-wide row of V */
            or_rms_norm(rows * nkv, hd, V, NULL, eps_q, V);
            maybe_f16(r16, V, rows * kw);
        }
    }
    or_attention(nitems, items, nq, nkv, hd, Q, qw, K, kw, V, kw, Att, qw, L->attn_scale, L->window);
    /* attention epilogue: v carried 2^-gq; the O input stores att col_o 2^-gao */
    scale_all(Att, rows * qw, ldexp(1.0, gq));
    half_site(rows, qw, Att, L->col_o, gao, r16, Att, am ? &am[2] : NULL);
    project(L, rows, qw, d, Att, L->wo, L->qo, L->so, L->bo, T);
    scale_all(T, rows * d, ldexp(1.0, gao));
    if (L->block == OR_SANDWICH) {
        or_rms_norm(rows, d, T, L->post_attn_w, L->eps, T);
        for (int64_t i = 0; i < rows * d; i++)
            H[i] += T[i] * (L->mod_g_attn ? (double)L->mod_g_attn[i % d] : 1.0);
        or_rms_norm(rows, d, H, L->norm2_w, L->eps, A);
        modulate(rows, d, A, L->mod_s_ff, A);
    } else {
        for (int64_t i = 0; i < rows * d; i++)
            H[i] += T[i];
        or_layer_norm(rows, d, H, L->norm2_w, L->norm2_b, L->eps, A);
    }

    /* MLP half: gate and up each from A * col * 2^-gf, times 2^gf after the GEMM */
    half_site(rows, d, A, L->col_up, gf, r16, Az, am ? &am[3] : NULL);
    project(L, rows, d, ff, Az, L->w_up, L->q_up, L->s_up, L->b_up, U);
    scale_all(U, rows * ff, ldexp(1.0, gf));
    if (L->mlp == OR_GELU) {
        for (int64_t i = 0; i < rows * ff; i++)
            U[i] = or_gelu_tanh(U[i]);
    } else {
        half_site(rows, d, A, L->col_gate, gf, r16, Az, am ? &am[3] : NULL);
        project(L, rows, d, ff, Az, L->w_gate, L->q_gate, L->s_gate, NULL, G);
        scale_all(G, rows * ff, ldexp(1.0, gf));
        for (int64_t i = 0; i < rows * ff; i++)
            U[i] = (L->mlp == OR_GELU_GATED ? or_gelu_tanh(G[i]) : or_silu(G[i])) * U[i];
    }
    /* the w2 input: hidden col_down 2^-gh */
    half_site(rows, ff, U, L->col_down, gh, r16, U, am ? &am[4] : NULL);
    project(L, rows, ff, d, U, L->w_down, L->q_down, L->s_down, L->b_down, T);
    scale_all(T, rows * d, ldexp(1.0, gh));
    const double scalar = L->scalar == 0.0 ? 1.0 : L->scalar;
    if (L->block == OR_SANDWICH) {
        or_rms_norm(rows, d, T, L->post_ff_w, L->eps, T);
        if (L->mod_g_ff)
            for (int64_t i = 0; i < rows * d; i++)
                T[i] *= (double)L->mod_g_ff[i % d];
    }
    for (int64_t i = 0; i < rows * d; i++)
        H[i] += T[i];
    if (L->n_ple > 0) {
        /* per-layer input ([EG] `TextGpu::forward`, after the FFN):
         *   P = rms(ple_scale * (X0 ple_in^T); ple_in_norm)   ("Y = rms(pre·X)·w")
         *   Z = gelu_tanh(H ple_gate^T) * P
         *   H = (H + rms(Z ple_proj^T; ple_post)) * scalar */
        int np = L->n_ple;
        double *P = (double *)malloc(sizeof(double) * rows * np);
        double *Z = (double *)malloc(sizeof(double) * rows * np);
        or_linear(rows, d, np, X0, L->ple_in, NULL, P);
        for (int64_t i = 0; i < rows * np; i++)
            P[i] *= L->ple_scale;
        or_rms_norm(rows, np, P, L->ple_in_norm_w, L->eps, P);
        or_linear(rows, d, np, H, L->ple_gate, NULL, Z);
        for (int64_t i = 0; i < rows * np; i++)
            Z[i] = or_gelu_tanh(Z[i]) * P[i];
        or_linear(rows, np, d, Z, L->ple_proj, NULL, T);
        or_rms_norm(rows, d, T, L->ple_post_w, L->eps, T);
        for (int64_t i = 0; i < rows * d; i++)
            H[i] += T[i];
        free(P);
        free(Z);
    }
    if (scalar != 1.0)
        for (int64_t i = 0; i < rows * d; i++)
            H[i] *= scalar;

    free(A); free(Az); free(Q); free(K); free(V); free(Att); free(T); free(G); free(U);
}

/* The whole forward: x [rows][d] -> out.
 * final NONE: out = H [rows][d];  LN: out = LN(H; final_w, final_b) [rows][d]
 * ([VE] step 4, the post-LN);  RMS_MEANPOOL: out[i] = mean over item i's rows of
 * rms(H_r; final_w), [nitems][d] ([EG] module doc "Text" and the "final norm +
 * mean pool" step of `TextGpu::forward`: the per-row inverse RMS first, then the
 * weighted mean).  Layers run in order, each starting from the H the previous
 * one left (the fused next-layer pre-norm of the pages computes the same A). */
OR_API void or_encoder_forward_pos(const or_model *M, int64_t rows, int nitems, const or_item *items,
                                   const int32_t *pos_in, const double *x, double *out, int f16_sites,
                                   double *amax)
{
    int d = M->d;
    int sec = M->nlayers > 0 ? M->layers[0].rope_sections : 0;
    int32_t *pos = (int32_t *)calloc((size_t)rows * (sec > 0 ? sec : 1), sizeof(int32_t));
    if (sec > 0 && pos_in)
        memcpy(pos, pos_in, sizeof(int32_t) * rows * sec);
    else if (sec > 0)
        or_positions(nitems, items, sec, pos);
    double *H = (double *)malloc(sizeof(double) * rows * d);
    memcpy(H, x, sizeof(double) * rows * d);
    for (int l = 0; l < M->nlayers; l++)
        layer_forward(&M->layers[l], rows, nitems, items, pos, H, x, f16_sites,
                      amax ? amax + 5 * l : NULL);
    if (M->final_kind == OR_FINAL_NONE) {
        memcpy(out, H, sizeof(double) * rows * d);
    } else if (M->final_kind == OR_FINAL_LN) {
        or_layer_norm(rows, d, H, M->final_w, M->final_b, M->final_eps, out);
    } else {
        double *R = (double *)malloc(sizeof(double) * rows * d);
        or_rms_norm(rows, d, H, M->final_w, M->final_eps, R);
        for (int i = 0; i < nitems; i++) {
            int L = item_len(&items[i]);
            for (int j = 0; j < d; j++) {
                double s = 0.0;
                for (int t = 0; t < L; t++)
                    s += R[(int64_t)item_row(&items[i], t) * d + j];
                out[(int64_t)i * d + j] = s / L;
            }
        }
        free(R);
    }
    free(H);
    free(pos);
}

/* The forward with the positions of or_positions (the usual case); pos_in of
 * or_encoder_forward_pos gives a stage of a larger program the positions its
 * rows have in that program. */
OR_API void or_encoder_forward(const or_model *M, int64_t rows, int nitems, const or_item *items,
                               const double *x, double *out, int f16_sites, double *amax)
{
    or_encoder_forward_pos(M, rows, nitems, items, NULL, x, out, f16_sites, amax);
}
