/*
 * enc.h — C ABI of libenc.so: the forward of a packed batch of rows through
 * bidirectional transformer-encoder and DiT blocks on one AMD Instinct MI355X
 * (gfx950).  Every kernel behind it is hand-written HIP for CDNA4.
 *
 * Sources of the operations (page title, item on that page):
 *   [EG] cortiq-engine 0.8.39, src/gpu_metal/egemma2.rs — EmbeddingGemma 2 on Metal
 *   [ZI] cortiq-engine 0.7.6,  src/gpu_metal/zimage.rs  — Z-Image DiT on Metal
 *   [VE] cera 0.2.4, src/model/vision_encoder_gpu.rs    — LFM2-VL ViT
 *
 * Conventions for every entry point:
 *  - Pointers marked (dev) are raw device addresses of caller-owned memory (for
 *    example PyTorch tensors on ROCm); (host) pointers are read during the call
 *    only.  The library allocates no device memory: scratch comes from the
 *    caller's workspace.  Matrices are row-major with the stated row strides
 *    (in elements).
 *  - Every call validates all arguments first.  On failure it returns a non-zero
 *    status, records a message readable with enc_last_error(), and has enqueued
 *    nothing ([ZI] module doc: an entry returns before changing any output when
 *    it cannot honour the full contract).  On success the work is enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *    without waiting.  ENC_EDEVICE (a failed launch) is the only status after
 *    which outputs may be partly written.
 *  - One enc_ctx per host thread, or callers serialise their calls on a ctx.
 *  - Item arrays are host memory copied into the kernel arguments at enqueue;
 *    the caller may free them as soon as the call returns.
 *  - A call enqueues kernels and device-to-device copies only (no memset, no
 *    allocation, no host synchronisation), so it may be recorded into a HIP
 *    graph by stream capture and replayed; a replay reads the item tables as
 *    they were at capture.  (enc_prof_enable's events are the exception: keep
 *    profiling off while capturing.)
 */
#ifndef ENC_H
#define ENC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENC_API __attribute__((visibility("default")))

typedef struct enc_ctx enc_ctx;
typedef void *enc_stream; /* hipStream_t */

typedef enum {
    ENC_OK = 0,
    ENC_EINVAL = 1,      /* null / overlapping / out-of-range items or pointers */
    ENC_ESHAPE = 2,      /* sizes that disagree with each other */
    ENC_EUNSUPPORTED = 3, /* geometry outside what the kernels take, or not a gfx950 device */
    ENC_EDEVICE = 4      /* a HIP launch or runtime error */
} enc_status;

/* Arithmetic path.  ENC_F32: f32 operands and accumulation throughout ([EG]
 * module doc, "f32 throughout").  ENC_I8F16: int8 weights with an f32 scale per
 * output row, f16 activations, f32 accumulation and f32 residual stream ([ZI]
 * module doc "The chain"). */
typedef enum { ENC_F32 = 0, ENC_I8F16 = 1 } enc_path;

/* Output flags of GEMM and row-op descriptors. */
enum {
    ENC_Y_F16 = 1u,              /* write f16 instead of f32 */
    ENC_Y_ACCUMULATE = 2u,       /* Y += result (residual add fused into the epilogue) */
    ENC_EPI_GELU_TANH = 4u,      /* Y = gelu_tanh(result) (before any accumulate) */
    ENC_EPI_GATE_GELU_TANH = 8u, /* gated: Y = gelu_tanh(gate) * up (see gemm_items) */
    ENC_EPI_GATE_SILU = 16u      /* gated: Y = silu(gate) * up */
};

/* ------------------------------------------------------------------ context */

/* Create a context on HIP device `device`.  ENC_EUNSUPPORTED unless the device
 * is gfx950; ENC_EDEVICE if HIP cannot query it.  *out is NULL on failure. */
ENC_API enc_status enc_create(int device, enc_ctx **out);
ENC_API void enc_destroy(enc_ctx *ctx);
/* Message of the last failed call on ctx (owned by ctx, valid until its next
 * call); "" after a success.  With ctx == NULL: the last enc_create failure. */
ENC_API const char *enc_last_error(const enc_ctx *ctx);

/* ------------------------------------------------------------- gemm_items */

/* Item-table batched GEMM, one launch for up to ENC_MAX_GEMM_ITEMS items ([EG]
 * module doc "GEMM" and `EgMm`: one item per grid z, so q/k/v are one launch
 * (z = 3) and gate/up another (z = 2); [ZI] `PMm`).  For item it and its
 * output row i < it.n, feature j < it.m:
 *   acc = sum_{k < it.k} X[it.x_off + i*it.ldx + k] * W_s[j*it.k + k]
 *   r   = alpha * acc              (ENC_F32)
 *   r   = alpha * rs_s[j] * acc    (ENC_I8F16: W_s int8, X f16, exact products,
 *                                   f32 accumulation — [ZI] module doc)
 *   r  += bias_s[j]                (when bias[s] != NULL)
 *   r   = gelu_tanh(r)             (ENC_EPI_GELU_TANH)
 *   r   = r * y_col[j] * y_scale   (y_col nullable; y_scale 0 is read as 1)
 *   Y[it.y_off + i*it.ldy + j] = r, or += r with ENC_Y_ACCUMULATE (f32 Y only)
 * where s = it.slot.  With ENC_EPI_GATE_GELU_TANH or ENC_EPI_GATE_SILU the item
 * is a gated MLP projection ([EG] `Prog::gelu` "O = gelu_tanh(G)·U" on the z = 2
 * gate/up launch; [ZI] SwiGLU `PSw`): gate_ij and up_ij are the r above for
 * slots s and s + 1 (no bias), and Y[i][j] = act(gate_ij) * up_ij * y_col[j] *
 * y_scale, so the gate/up pair never reaches memory.  (y_col and y_scale are
 * the q8_2f column field of the weight that reads Y and a power-of-two guard
 * of a half Y: [ZI] module doc "The chain", `Guards`.)  The result equals the unfused gate/up
 * GEMM followed by enc_gated_act bit for bit.  W_s is [m][k] row-major (the nn.Linear layout, [VE]
 * `VitGpuOps::linear`), dense with row stride k.
 * Geometry: k % 4 == 0 (F32) or k % 16 == 0 (I8F16); ldx, x_off multiples of 4
 * (F32) or 8 (I8F16); X, Y, W_s 16-byte aligned.  Items may not write
 * overlapping Y regions.  The summation order of an output does not depend on
 * it.n, so a row gives the same bits whatever batch it is packed in. */
#define ENC_MAX_GEMM_ITEMS 4
typedef struct {
    uint32_t n, m, k;   /* rows, output features, reduction length */
    uint32_t ldx, ldy;  /* row strides of X and Y (elements) */
    uint32_t slot;      /* weight slot 0..3 */
    uint64_t x_off, y_off; /* element offsets of the item's first row in X and Y */
} enc_gemm_item;

typedef struct {
    uint32_t path;            /* enc_path */
    const void *x;            /* (dev) F32: float; I8F16: _Float16 */
    void *y;                  /* (dev) float, or _Float16 with ENC_Y_F16 */
    const void *w[4];         /* (dev) per slot: F32 float [m][k]; I8F16 int8_t [m][k] */
    const float *row_scale[4];/* (dev) I8F16: float [m] per slot; F32: ignored */
    const float *bias[4];     /* (dev) nullable, float [m] */
    float alpha;              /* [EG] EgMm.alpha / [ZI] PMm.mul */
    uint32_t flags;           /* ENC_Y_F16 | ENC_Y_ACCUMULATE | ENC_EPI_GELU_TANH */
    const float *y_col;       /* (dev) nullable, float [m]: multiplies column j of the result */
    float y_scale;            /* multiplies every result; 0 is read as 1 */
} enc_gemm_desc;

ENC_API enc_status gemm_items(enc_ctx *ctx, const enc_gemm_desc *desc, const enc_gemm_item *items,
                      uint32_t nitems, enc_stream stream);

/* -------------------------------------------------------- attention_items */

/* A packed item: its rows are r[0] followed by r[1] (nr = 1 or 2).  Queries
 * and keys are the item's rows; t = a row's index in that concatenated order.
 * [EG] segment table (one range per text sequence); [ZI] `PFa` (image range +
 * caption range; the CFG program's items [img0|cap0] and [img1|cap1]). */
typedef struct { uint32_t r0, n; } enc_range;
typedef struct {
    enc_range r[2];
    uint32_t nr;
} enc_item;

/* Non-causal flash attention over items ([EG] `VisionGpu::forward` flash path
 * and module doc "Attention"; [ZI] module doc, flash `zi_flash_q64pf`; [VE]
 * `VitGpuOps::attention`).  For item I, query head h < nq, kv head
 * g = h / (nq / nkv), and every row i of I:
 *   out[i][h*hd + c] = sum_{j in V(i)} e^{s_ij - m_i} v_j[c] / sum_{j in V(i)} e^{s_ij - m_i}
 *   s_ij = scale * sum_c q_i[c] k_j[c],  m_i = max_{j in V(i)} s_ij
 *   q_i = qkv[i][q_col + h*hd ..], k_j = qkv[j][k_col + g*hd ..], v_j = qkv[j][v_col + g*hd ..]
 * V(i) = rows j of I with window == 0 or |t_i - t_j| <= window (the key span
 * [q0 - W, q_last + W] of [EG] `att_plan`).  Softmax in f32 on both paths.
 * Geometry: hd in {64, 128}; nq % nkv == 0; ld, ldo, the column offsets
 * multiples of 8; items disjoint and inside [0, rows).  Rows of the panel
 * outside every item are never read; out rows outside every item are not
 * written. */
typedef struct {
    uint32_t path;          /* ENC_F32: float panel/out; ENC_I8F16: _Float16 panel/out */
    const void *qkv;        /* (dev) panel [rows][ld] */
    uint32_t ld;
    uint32_t q_col, k_col, v_col; /* first column of the q / k / v blocks */
    void *out;              /* (dev) [rows][ldo]; head h at columns h*hd .. */
    uint32_t ldo;
    uint32_t nq, nkv, hd;
    float scale;
    uint32_t window;        /* 0 = full bidirectional */
    uint32_t rows;          /* panel rows (bound for the items) */
    void *ws;               /* (dev) scratch for key splits, 256-byte aligned, or NULL */
    size_t ws_bytes;        /* at least enc_attention_workspace_bytes() when ws != NULL */
    /* output epilogue: out[i][c] = o_i[c] * out_scale * out_col[c] ([ZI]: the
     * flash epilogue folds the O projection's column field and the guards) */
    const float *out_col;   /* (dev) nullable, float [nq*hd] */
    float out_scale;        /* 0 is read as 1 */
} enc_attn_desc;

/* Key splits (ENC_F32, windowless items): an item too short to occupy the GPU
 * with its query tiles alone is cut into key chunks whose partial softmax
 * results (running max, sum and unnormalised output, f32) go to ws and are
 * merged by a second kernel in a fixed order: the same softmax, regrouped.
 * Whether and how an item is split depends only on its length, nq, the path
 * and the window, so a packed batch gives the same bits as its items alone.
 * With ws == NULL nothing is split.  A ws smaller than needed is ENC_ESHAPE.
 * ENC_I8F16 at hd 128 never uses ws: a windowless item whose blocks of 64
 * queries times nq number at most 512 has each query's keys split in two
 * halves inside one block and merged there (the same length-only rule, so the
 * same invariance). */
ENC_API enc_status attention_items(enc_ctx *ctx, const enc_attn_desc *desc, const enc_item *items,
                           uint32_t nitems, enc_stream stream);

/* Bytes of ws attention_items uses for these items (0: nothing is split).
 * Host only; reads only the geometry fields of desc. */
ENC_API size_t enc_attention_workspace_bytes(const enc_attn_desc *desc, const enc_item *items,
                                             uint32_t nitems);

/* attention_items for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and split plan, with the key-split partials in a
 * static device array of ENC_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends, instead of a workspace.  The
 * call allocates nothing.  desc->ws must be NULL and ws_bytes 0 (ENC_EINVAL
 * otherwise); items whose splits need more than ENC_STATIC_SCRATCH_BYTES
 * (enc_attention_workspace_bytes) are refused with ENC_EUNSUPPORTED before
 * anything is enqueued.  Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (two streams, or two threads) race on it.  Nothing
 * in the array needs clearing: each split writes all of its partials before
 * the merge reads them.  ENC_EDEVICE if the array's address could not be
 * taken when ctx was created. */
#define ENC_STATIC_SCRATCH_BYTES (32u << 20)
ENC_API enc_status attention_items_static(enc_ctx *ctx, const enc_attn_desc *desc, const enc_item *items,
                                          uint32_t nitems, enc_stream stream);

/* ------------------------------------------------------------------ row ops */
/* One wavefront per row (or per row and head); f32 statistics.  Geometry:
 * d % 4 == 0 and d <= 4096; strides multiples of 4 (f32) or 8 (f16). */

/* RMSNorm y = rms(pre x) w = pre x w / sqrt(mean((pre x)^2) + eps), gain
 * multiplying directly ([EG] `Prog::rms`, "Y = rms(pre·X)·w").  LayerNorm
 * y = (x - mean) / sqrt(var + eps) * w + b, population variance ([VE]
 * `VitGpuOps::layernorm`; b may be NULL; pre must be 0 or 1).  Output f32, or
 * f16 with ENC_Y_F16.  rows = 0 is a no-op (the pointers may then be NULL). */
typedef struct {
    uint32_t rows, d;
    const float *x;   /* (dev) [rows][ldx] */
    uint32_t ldx;
    const float *w;   /* (dev) [d] */
    const float *b;   /* (dev) [d] or NULL (LayerNorm only) */
    float eps;
    void *y;          /* (dev) [rows][ldy]; may equal x for an f32 output */
    uint32_t ldy;
    uint32_t flags;   /* ENC_Y_F16 */
    float pre;        /* RMSNorm input prescale; 0 is read as 1 */
} enc_norm_desc;
ENC_API enc_status enc_rms_norm(enc_ctx *ctx, const enc_norm_desc *desc, enc_stream stream);
ENC_API enc_status enc_layer_norm(enc_ctx *ctx, const enc_norm_desc *desc, enc_stream stream);

/* Post-norm residual fused with the next pre-norm ([EG] `Prog::add_norm`
 * "H = (H + rms(T)·w)·post; then A = rms(H)·w2"; [ZI] `Enc::rowop`, with its
 * adaLN gate and scale, the q8_2f column fields of the next GEMM's weights and
 * the half site's guard):
 *   when t != NULL:      h = (h + gate * rms(t) * w_post) * post
 *   when w_next != NULL: for z < nout,
 *                        a_z = rms(h) * w_next * (1 + scale) * col[z] * oscale
 * gate, scale, col[z] nullable (ones / zeros); nout 0 is read as 1; the copy z
 * sits at a + z*rows*d.  h, t f32 [rows][d] (dense); a f32 or f16 (ENC_Y_F16). */
typedef struct {
    uint32_t rows, d;
    float *h;             /* (dev) residual, updated in place */
    const float *t;       /* (dev) block output */
    const float *w_post;  /* (dev) [d] */
    const float *w_next;  /* (dev) [d] or NULL */
    float eps;
    void *a;              /* (dev) next block input; unused when w_next == NULL */
    uint32_t flags;       /* ENC_Y_F16 */
    float post;           /* the layer scalar; 0 is read as 1 */
    const float *gate, *scale, *col[3]; /* (dev) nullable, float [d] each */
    uint32_t nout;        /* copies of a (1..3) */
    float oscale;         /* 0 is read as 1 */
} enc_add_norm_desc;
ENC_API enc_status enc_add_norm(enc_ctx *ctx, const enc_add_norm_desc *desc, enc_stream stream);

/* q/k RMSNorm per head, then RoPE, in place on the panel ([EG] `Prog::qkv` and
 * `EgQkv` — rotate_half within each `sec` channels; [ZI] `PQk`).  For every
 * row r and every q head (columns q_col + h*hd) and k head (k_col + g*hd):
 *   x = rms(x) * norm_w;  then for each section s of S = hd / sections channels
 *   and i < S/2, with (c, sn) = (cos, sin)[r][s*S/2 + i]:
 *     x[sS+i] <- x[sS+i] c - x[sS+i+S/2] sn;  x[sS+i+S/2] <- x[sS+i+S/2] c + x[sS+i] sn
 * sections = 0 skips the rotation.  cos/sin: (dev) f32 [rows][hd/2], built by
 * enc_rope_table.  With v_norm, every v head (columns v_col + g*hd) is also
 * replaced by x / sqrt(mean(x^2) + eps), without gain or rotation ([EG]
 * `Prog::qkv`: "q/k norm + RoPE, v norm"; the prep takes no v weight).  The
 * panel is f32 (ENC_F32) or f16 (ENC_I8F16, math in f32). */
typedef struct {
    uint32_t path;
    void *panel;          /* (dev) [rows][ld] */
    uint32_t rows, ld, q_col, k_col, nq, nkv, hd;
    const float *q_norm_w, *k_norm_w; /* (dev) [hd] */
    float eps;
    const float *cos, *sin;           /* (dev) [rows][hd/2] */
    uint32_t sections;                /* 0, 1 or 2 */
    uint32_t v_col, v_norm;           /* v block column; 1 = norm the v heads too */
} enc_qk_desc;
ENC_API enc_status enc_qk_norm_rope(enc_ctx *ctx, const enc_qk_desc *desc, enc_stream stream);

/* Gated activation out = act(g) * u * out_col * out_scale, elementwise over
 * [rows][ff] (out_col nullable, out_scale 0 read as 1; [ZI] `PSw` folds w2's
 * column field and the hidden's guard here):
 * ENC_ACT_GELU_TANH_GATED ([EG] `Prog::gelu` "O = gelu_tanh(G)·U") or
 * ENC_ACT_SWIGLU ([ZI] `PSw`, silu(g)·u).  Output f32 or f16 (ENC_Y_F16). */
typedef enum { ENC_ACT_GELU_TANH_GATED = 1, ENC_ACT_SWIGLU = 2 } enc_act_kind;
typedef struct {
    uint32_t kind, rows, ff;
    const float *g; uint32_t ldg;   /* (dev) */
    const float *u; uint32_t ldu;   /* (dev) */
    void *out; uint32_t ldo;        /* (dev) */
    uint32_t flags;                 /* ENC_Y_F16 */
    const float *out_col;           /* (dev) nullable, float [ff] */
    float out_scale;
} enc_act_desc;
ENC_API enc_status enc_gated_act(enc_ctx *ctx, const enc_act_desc *desc, enc_stream stream);

/* Mean of each item's rows: out[i][j] = (1/|I|) sum_{r in I} a[r][j], f32.
 * With a = rms(H) * w_final this is the final norm + mean pool of [EG]
 * `TextGpu::forward` (per-row inverse RMS, then the weighted mean).  Any number
 * of items; an empty item is ENC_EINVAL (its mean is undefined).  The rows of an
 * item are summed in a fixed order, so the result does not depend on the other
 * items. */
ENC_API enc_status enc_mean_pool(enc_ctx *ctx, uint32_t rows, uint32_t d, const float *a,
                         const enc_item *items, uint32_t nitems, float *out, enc_stream stream);

/* ------------------------------------------------------------ layer, model */

typedef enum { ENC_PRE_LN = 0, ENC_SANDWICH_RMS = 1 } enc_block;
typedef enum { ENC_MLP_GELU_TANH = 0, ENC_MLP_GELU_TANH_GATED = 1, ENC_MLP_SWIGLU = 2 } enc_mlp;
typedef enum { ENC_FINAL_NONE = 0, ENC_FINAL_LN = 1, ENC_FINAL_RMS_MEANPOOL = 2 } enc_final;

/* One layer's shape and device weights.
 * ENC_SANDWICH_RMS ([EG] `TextGpu::forward` layer loop; [ZI] module doc "The
 * chain", `Enc::block`):
 *   A = rms(H; norm1_w); q|k|v = A W^T; q, k = rope(rms(.; q_norm_w | k_norm_w));
 *   att = attention; H += rms(att Wo^T; post_attn_w); A = rms(H; norm2_w);
 *   m = act(A W_gate^T) * (A W_up^T); H += rms(m W_down^T; post_ff_w)
 * ENC_PRE_LN ([VE] `encode_image_gpu`, step 3):
 *   A = LN(H; norm1); q|k|v = A W^T + b; H += attention Wo^T + bo;
 *   A = LN(H; norm2); H += gelu_tanh(A W_up^T + b_up) W_down^T + b_down
 * ENC_I8F16 stores A, the q|k|v panel, the attention output and m as f16 and
 * keeps H, the projections' f32 outputs and gate/up in f32 ([ZI] `Acts`).
 * Weights [out][in]: F32 float, I8F16 int8 with f32 row scales s_*.
 * Biases and w_gate may be NULL where the block kind has none.
 * Supported: d, ff multiples of 64; d <= 4096; hd in {64, 128}; nq % nkv == 0;
 * rope_sections in {0, 1, 2}. */
typedef struct {
    uint32_t block, path, mlp;
    uint32_t d, nq, nkv, hd, ff, window, rope_sections;
    float eps, attn_scale;
    const void *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
    const float *sq, *sk, *sv, *so, *s_gate, *s_up, *s_down;
    const float *bq, *bk, *bv, *bo, *b_up, *b_down;
    const float *norm1_w, *norm1_b, *norm2_w, *norm2_b;
    const float *post_attn_w, *post_ff_w, *q_norm_w, *k_norm_w;
    /* Options of the text encoder's layer spec ([EG] `LayerSpec`; sandwich block,
     * zero-initialised = off):
     *  v_norm      weightless RMS of every v head after the projection;
     *  rope_table  which of the batch's RoPE tables the layer rotates with
     *              ([EG] `LayerSpec.rope`: one table per RoPE kind);
     *  scalar      the layer's last residual update is H = (H + .) * scalar
     *              ([EG] `add_norm(.., l.scalar)`); 0 is read as 1;
     *  n_ple       width of the per-layer-input branch ([EG] `TextGpu::forward`,
     *              after the FFN; f32 path, multiple of 64; 0 = none):
     *                P = rms(ple_scale * (X0 ple_in^T); ple_in_norm_w)
     *                Z = gelu_tanh(H ple_gate^T) * P
     *                H = (H + rms(Z ple_proj^T; ple_post_w)) * scalar
     *              with X0 the forward's input rows (enc_batch.ple_x). */
    uint32_t v_norm, rope_table;
    float scalar;
    uint32_t n_ple;
    float ple_scale;
    const float *ple_in, *ple_gate, *ple_proj; /* [n_ple][d], [n_ple][d], [d][n_ple] */
    const float *ple_in_norm_w, *ple_post_w;   /* [n_ple], [d] */
    /* The int8 DiT block's row-op contract ([ZI] `Enc::block`, `Enc::rowop`,
     * module doc "The chain"; sandwich block, NULL / 0 = off):
     *  mod_*    adaLN modulation, f32 [d] each: the pre-norm outputs are
     *           multiplied by (1 + mod_s_*), the residual updates by mod_g_*
     *           (the block's [s_msa | g_msa | s_mlp | g_mlp]);
     *  col_*    the q8_2f column field of each int8 weight, f32 [in]: the
     *           weight is rs[j] q[j][k] col[k], and col is folded into the half
     *           input by its producer (the row op writes q, k, v and w1/w3 their
     *           own copy of A; the attention epilogue multiplies col_o; the
     *           SwiGLU multiplies col_down; with col_gate/col_up the gate/up
     *           GEMM runs unfused, z = 2, as on the page);
     *  guard_*  [ZI] `Guards`, 0..14: each half site stores x 2^-guard and its
     *           consumer multiplies 2^guard back (q/k/v input, panel, attention
     *           output, w1/w3 input, SwiGLU hidden); the qk-norm's eps is scaled
     *           by 2^-2 guard_qkv.  Int8 path only. */
    const float *mod_s_attn, *mod_g_attn, *mod_s_ff, *mod_g_ff;
    const float *col_q, *col_k, *col_v, *col_o, *col_gate, *col_up, *col_down;
    uint32_t guard_attn, guard_qkv, guard_ao, guard_ffn, guard_hid;
} enc_layer;

/* The packed batch: `rows` rows, `nitems` disjoint items covering them, the
 * RoPE tables (dev, f32 [rows][hd/2] each; a layer rotates with table
 * rope_table; NULL where no layer uses it) and, for layers with a per-layer
 * input, the rows X0 that branch projects (dev, f32 [rows][d]; encoder_forward
 * takes its x when NULL, encoder_layer_forward needs it).  amax (dev, nullable,
 * f32 [nlayers][5], int8 path): each layer's max |stored half value| at its
 * q/k/v input, panel, attention output, w1/w3 input and SwiGLU hidden, after
 * the column fields and guards ([ZI] `amax`, the guard calibration). */
#define ENC_MAX_ROPE_TABLES 4
typedef struct {
    uint32_t rows;
    const enc_item *items; /* (host) */
    uint32_t nitems;
    const float *rope_cos[ENC_MAX_ROPE_TABLES], *rope_sin[ENC_MAX_ROPE_TABLES];
    const float *ple_x;
    float *amax;
} enc_batch;

/* All layers share d, path and block kind.  final: NONE -> out = H [rows][d];
 * LN -> out = LN(H; final_w, final_b) [rows][d] ([VE] step 4, post-LN);
 * RMS_MEANPOOL -> out[i] = mean over item i of rms(H_r; final_w), [nitems][d]
 * (every item must then be non-empty: ENC_EINVAL otherwise). */
typedef struct {
    uint32_t nlayers;
    const enc_layer *layers; /* (host) */
    uint32_t final_kind;
    const float *final_w, *final_b; /* (dev) */
    float final_eps;
} enc_model;

/* Workspace bytes encoder_forward / encoder_layer_forward need for this batch
 * (its rows, its items for the attention key splits, and a little more when
 * batch.amax is set).  0 on null input. */
ENC_API size_t enc_workspace_bytes(const enc_model *model, const enc_batch *batch);

/* One layer in place on h (dev, f32 [rows][d]).
 * a (dev, nullable): the layer's pre-normed input, the A that its q/k/v GEMM
 * reads: for the sandwich block rms(h; norm1_w) (times 1 + mod_s_attn, the
 * q/k/v column fields and 2^-guard_attn), one [rows][d] copy per column field
 * (three with col_q/col_k/col_v, else one); for pre-LN LN(h; norm1_w, norm1_b).
 * Half on the int8 path, f32 otherwise.  NULL: the layer computes it.
 * next (host, nullable; needs a): the following layer, same block kind, path
 * and width.  Its pre-normed input is then written into a from the updated h
 * before return, by the sandwich block's last row op itself ([EG] `Prog::add_norm`:
 * H = (H + rms(T) w) post, then A = rms(H) w2) and by one LN pass for pre-LN,
 * so a chain of calls (a = NULL for the first, then a and next) gives the bits
 * of encoder_forward.  a must then hold max(copies of this layer, copies of
 * next) x rows x d elements.  Without next, a is read and left unchanged. */
ENC_API enc_status encoder_layer_forward(enc_ctx *ctx, const enc_layer *layer, const enc_layer *next,
                                         const enc_batch *batch, float *h, void *a, void *ws,
                                         size_t ws_bytes, enc_stream stream);

/* The whole forward: x (dev, f32 [rows][d], not modified unless out == x) ->
 * out (dev, f32, [rows][d] or [nitems][d] for RMS_MEANPOOL).  Each layer's last
 * row op also writes the next layer's pre-norm input ([EG] `add_norm` with
 * the next in_norm), giving the same bits as encoder_layer_forward layer by
 * layer.  ws: (dev) at least enc_workspace_bytes, 256-byte aligned. */
ENC_API enc_status encoder_forward(enc_ctx *ctx, const enc_model *model, const enc_batch *batch,
                           const float *x, float *out, void *ws, size_t ws_bytes,
                           enc_stream stream);

/* A staged program ([ZI] `step`: the noise refiner blocks over the image rows
 * of every item, the caption rows copied in, then the main stack over all
 * rows; `refine_caption`: the unmodulated context refiner over the caption
 * rows).  Stage i runs its model's layers in place on rows [row0, row0 +
 * batch.rows) of the residual h, its batch's items and tables relative to row0;
 * with the rows of a packed batch in place ([img0 | img1 | cap0 | cap1]) no
 * row moves.  Every stage's final is ENC_FINAL_NONE; all share one width.
 * h (dev, f32 [rows][d]) starts as a copy of x (or is x). */
typedef struct {
    const enc_model *model; /* (host) */
    enc_batch batch;
    uint32_t row0;
} enc_stage;

ENC_API size_t enc_stages_workspace_bytes(const enc_stage *stages, uint32_t nstages);
ENC_API enc_status encoder_stages_forward(enc_ctx *ctx, const enc_stage *stages, uint32_t nstages,
                                          uint32_t rows, const float *x, float *h, void *ws,
                                          size_t ws_bytes, enc_stream stream);

/* --------------------------------------------------------- per-class timing */

/* Launch classes ([EG] `Rec` and [ZI] `Rec`: one GPU time per op class under a
 * profiling knob).  GEMM = gemm_items launches (also inside the layer/model
 * calls), ATTN = attention_items launches, ROWS = every row op. */
typedef enum { ENC_CLASS_GEMM = 0, ENC_CLASS_ATTN = 1, ENC_CLASS_ROWS = 2, ENC_NCLASS = 3 } enc_class;
typedef struct {
    uint64_t launches;
    double ms;     /* summed GPU time between each launch's bracketing events */
    double flops;  /* algorithmic: 2 n m k per GEMM item; 4 hd per visible (query, key) pair per head */
    double bytes;  /* algorithmic HBM bytes: inputs read once and outputs written once (row ops;
                      GEMM: X, the weights and Y; attention: not counted) */
} enc_prof_stat;

/* With profiling on, every kernel launch enqueued through ctx is bracketed by
 * two hipEvent records on its stream (the events are created once and reused;
 * no device memory is allocated).  enc_prof_read waits for the recorded events,
 * writes the per-class totals since the previous read into stats[ENC_NCLASS]
 * and starts a new interval.  Not for use under stream capture. */
ENC_API enc_status enc_prof_enable(enc_ctx *ctx, int on);
ENC_API enc_status enc_prof_read(enc_ctx *ctx, enc_prof_stat *stats);

/* MFMA issue-rate probe ([ZI] `bench_mma_peak`: a pure matrix-op loop with 16
 * independent accumulators and no memory traffic).  One launch of `blocks`
 * 256-thread blocks, each wave issuing iters x 16 MFMAs (ENC_F32:
 * v_mfma_f32_32x32x2_f32; ENC_I8F16: v_mfma_f32_32x32x16_f16, the GEMMs'
 * instructions) on random operands that change from one MFMA to the next, as
 * in a GEMM (constant operands let the chip hold a higher clock than real data
 * does); writes blocks*256 floats to out (dev) and the launch's flops to
 * *flops.  Time it with events on `stream`. */
ENC_API enc_status enc_mfma_peak(enc_ctx *ctx, uint32_t path, uint32_t blocks, uint32_t iters,
                                 float *out, double *flops, enc_stream stream);

/* ---------------------------------------------------- host-only helpers */
/* No HIP calls: usable and testable without a GPU. */

/* Validation of the descriptors the entry points take; the same checks the
 * entry points run first.  msg (host, nullable) receives a message. */
ENC_API enc_status enc_check_gemm(const enc_gemm_desc *desc, const enc_gemm_item *items,
                          uint32_t nitems, char *msg, size_t msg_len);
ENC_API enc_status enc_check_attention(const enc_attn_desc *desc, const enc_item *items,
                               uint32_t nitems, char *msg, size_t msg_len);
ENC_API enc_status enc_check_model(const enc_model *model, const enc_batch *batch, char *msg,
                           size_t msg_len);
/* The model and batch check alone, by the name the boundary's design gives it:
 * enc_check_model without the message (the same checks encoder_forward and
 * encoder_layer_forward run first, so a model it accepts is one they take). */
ENC_API enc_status enc_validate_model(const enc_model *model, const enc_batch *batch);

/* RoPE positions (host int32 [rows][sections]).  1-D (sections 1): the row's
 * index t within its item, restarting at 0 per item ([EG] `TextGpu::forward`,
 * positions per sequence).  2-D (sections 2): grids[i] = G > 0 marks item i as
 * a G x G image in row-major order at the start of its first range: t < G*G
 * sits at (column t % G, row t / G); rows of the first range past the image
 * are its padding ([ZI] `prepare`: image rows padded to a multiple of 32 with
 * the learned pad row) and sit at (0, 0); the rows of the second range are
 * captions, caption j at (G + j, G + j). */
ENC_API enc_status enc_positions(uint32_t rows, const enc_item *items, const uint32_t *grids,
                         uint32_t nitems, uint32_t sections, int32_t *pos);

/* RoPE tables (host f32 [rows][hd/2]) from positions: for section s of
 * S = hd / sections channels and i < S/2, angle = pos[r][s] * base^(-2i/S),
 * computed in double and rounded once ([EG] `TextSpec::ropes`, `[max_tokens,
 * head_dim/2]`; [EG] `VisionGpu::forward`: the column half, then the row half). */
ENC_API enc_status enc_rope_table(uint32_t rows, uint32_t hd, uint32_t sections, const int32_t *pos,
                          double base, float *cos_out, float *sin_out);

#ifdef __cplusplus
}
#endif
#endif /* ENC_H */
