// Kernel argument blocks and host launchers shared between the C-ABI layer
// (api.hip) and the kernel translation units.  Plain structs passed by value
// as kernel arguments; item tables live inside them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace enc {

constexpr int kMaxGemmItems = 4;
constexpr int kMaxAttnItems = 64;  // per launch; longer lists are split

struct GemmItemK {
    uint32_t n, m, k, ldx, ldy, slot;
    uint32_t tiles_m, tile0;  // tiles along m; first linear tile of this item
    uint64_t x_off, y_off;
};

struct GemmArgs {
    const void *x;
    void *y;
    const void *w[kMaxGemmItems];
    const float *rs[kMaxGemmItems];
    const float *bias[kMaxGemmItems];
    float alpha;
    uint32_t flags;
    uint32_t nitems;
    uint32_t total_tiles;
    const float *ycol;     // per output column multiplier of the stored value (nullable)
    float yscale;          // and a scale of every stored value (a power-of-two guard)
    GemmItemK items[kMaxGemmItems];
};

struct AttnItemK {
    uint32_t r0a, na, r0b, nb;  // ranges (nb = 0 for one range)
    uint32_t tile0;             // first tile of this item in the launch
    // key split (f32 path): nsplit chunks of `chunk` keys; the item's tiles are
    // (q-tile, split) pairs, split fastest.  Partial results of split s, item
    // row t, head h sit at record part0 + (s * L + t) * nq + h.
    uint32_t nsplit, chunk, part0;
};

struct AttnArgs {
    const void *qkv;
    void *out;
    uint32_t ld, ldo, q_col, k_col, v_col;
    uint32_t nq, group;     // group = nq / nkv
    float scale_log2;       // scale * log2(e): the softmax runs in base 2
    uint32_t window;
    uint32_t nitems, ntiles;
    float *part_o;   // [records][hd] unnormalised outputs of split items
    float *part_ml;  // [records][2] running max (base 2) and sum
    const float *ocol;   // output channel multiplier [nq*hd] (nullable)
    float oscale;        // output scale
    uint32_t rows;       // rows of the q/k/v panel
    AttnItemK items[kMaxAttnItems];
};

// Merge of the key-split partial results into the attention output.
struct CombineArgs {
    const float *part_o, *part_ml;
    void *out;
    uint32_t ldo, nq, hd, nitems;
    const float *ocol;
    float oscale;
    uint32_t row0[kMaxAttnItems + 1];  // prefix of item lengths over the split items
    AttnItemK items[kMaxAttnItems];
};

struct NormArgs {
    uint32_t rows, d, ldx, ldy;
    const float *x;
    const float *w;
    const float *b;
    float eps;
    void *y;
    float pre = 1.0f;  // RMSNorm of pre * x (1 = plain)
};

// Row op of the sandwich block: with t, h = (h + gate * rms(t) w_post) * post;
// then with w_next, for z < nout: a_z = rms(h) w_next (1 + scale) col_z oscale
// (a_z at a + z * a_stride elements).  gate, scale, col_z nullable.
struct AddNormArgs {
    uint32_t rows, d;
    float *h;
    const float *t;
    const float *w_post;
    const float *w_next;
    float eps;
    void *a;
    float post = 1.0f;
    const float *gate = nullptr, *scale = nullptr;
    const float *col[3] = {nullptr, nullptr, nullptr};
    uint32_t nout = 1;
    float oscale = 1.0f;
    uint64_t a_stride = 0;
};

struct QkArgs {
    void *panel;
    uint32_t rows, ld, q_col, k_col, nq, nkv, hd, sections;
    const float *qw, *kw;
    float eps;
    const float *cos, *sin;
    uint32_t v_col = 0, v_norm = 0;  // v_norm: weightless RMS of the nkv v heads too
};

struct ActArgs {
    uint32_t kind, rows, ff, ldg, ldu, ldo;
    const float *g, *u;
    void *out;
    const float *ocol = nullptr;  // per column multiplier of the stored value
    float oscale = 1.0f;
};

// Max |x| over n halves: per-block maxima into part[blocks], then one block
// reduces them into *out.
struct AmaxArgs {
    const _Float16 *x;
    uint64_t n;
    float *part;
    uint32_t blocks;
    float *out;
};

struct PoolArgs {
    uint32_t d, nitems;
    const float *a;
    float *out;
    AttnItemK items[kMaxAttnItems];
};

// Launchers return hipGetLastError() after the launch (hipSuccess on success).
hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemm_i8f16(const GemmArgs &a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs &a, uint32_t hd, hipStream_t s);
hipError_t launch_attn_f16(const AttnArgs &a, uint32_t hd, hipStream_t s);
hipError_t launch_attn_combine(const CombineArgs &a, bool f16_out, hipStream_t s);
hipError_t launch_rms_norm(const NormArgs &a, bool f16_out, hipStream_t s);
hipError_t launch_layer_norm(const NormArgs &a, bool f16_out, hipStream_t s);
hipError_t launch_add_norm(const AddNormArgs &a, bool f16_out, hipStream_t s);
hipError_t launch_qk_norm_rope(const QkArgs &a, bool f16, hipStream_t s);
hipError_t launch_gated_act(const ActArgs &a, bool f16_out, hipStream_t s);
hipError_t launch_mean_pool(const PoolArgs &a, hipStream_t s);
hipError_t launch_amax_f16(const AmaxArgs &a, hipStream_t s);
constexpr uint32_t kAmaxBlocks = 512;
hipError_t launch_mfma_peak(bool f16, uint32_t blocks, uint32_t iters, float *out, hipStream_t s);

// Tile sizes the launchers and the planner agree on.
constexpr int kGemmBM = 128, kGemmBN = 128;

}  // namespace enc
