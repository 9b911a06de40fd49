// C ABI of libenc.so (include/enc.h): validation, planning and launch order.
//
// Every entry point validates its whole argument set on the host before it
// enqueues anything (zimage.rs, cortiq-engine 0.7.6, module doc: an entry
// returns before changing any output when it cannot honour the full contract;
// egemma2.rs, cortiq-engine 0.8.39, `TextGpu::forward`: misshapen input is an
// error).  Item tables go into kernel arguments; scratch comes from the
// caller's workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/enc.h"
#include "kern.h"

struct ProfRec {
    int cls;
    size_t ev;  // index of the event pair in the pool
    double flops, bytes;
};

struct enc_ctx {
    int device = 0;
    std::string err;
    bool prof = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
    std::vector<ProfRec> recs;
    void *scratch = nullptr;   // this device's copy of `scratch` (attention_items_static)
    std::string scratch_err;   // why it is missing, if it is
};

// Scratch of attention_items_static: the key-split partials, in a file-scope
// device array rather than a caller workspace.  The runtime allocates one
// copy on every device the library runs on, held until the process ends; in
// host code `scratch` names a host-side stand-in, so its device address is
// taken once per device (enc_create) and only that address is used.
static __device__ __attribute__((aligned(256))) uint8_t scratch[ENC_STATIC_SCRATCH_BYTES];

namespace {

using namespace enc;

// The ctx whose entry point is running on this thread (profiling hooks).
thread_local enc_ctx *t_ctx = nullptr;

struct CtxScope {
    explicit CtxScope(enc_ctx *c) { t_ctx = c; }
    ~CtxScope() { t_ctx = nullptr; }
};

// Brackets one launch with events on its stream when profiling is on.
template <class F>
hipError_t prof_launch(int cls, hipStream_t s, double flops, double bytes, F &&launch) {
    enc_ctx *c = t_ctx;
    if (!c || !c->prof) return launch();
    const size_t i = c->recs.size();
    if (i == c->pool.size()) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return hipErrorOutOfMemory;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return hipErrorOutOfMemory;
        }
        c->pool.push_back({a, b});
    }
    hipError_t h = hipEventRecord(c->pool[i].first, s);
    if (h != hipSuccess) return h;
    h = launch();
    if (h != hipSuccess) return h;
    h = hipEventRecord(c->pool[i].second, s);
    if (h == hipSuccess) c->recs.push_back({cls, i, flops, bytes});
    return h;
}

std::string g_create_err;

struct Err {
    enc_status st = ENC_OK;
    std::string msg;
    enc_status set(enc_status s, const char *fmt, ...) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        st = s;
        msg = buf;
        return s;
    }
};

enc_status finish(enc_ctx *ctx, const Err &e) {
    if (ctx) ctx->err = e.st == ENC_OK ? std::string() : e.msg;
    return e.st;
}

void copy_msg(const Err &e, char *msg, size_t len) {
    if (msg && len) {
        size_t n = std::min(len - 1, e.msg.size());
        memcpy(msg, e.msg.data(), n);
        msg[n] = 0;
    }
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

enc_status launch_status(Err &e, hipError_t h, const char *what) {
    if (h != hipSuccess) return e.set(ENC_EDEVICE, "%s: %s", what, hipGetErrorString(h));
    return ENC_OK;
}

// ---------------------------------------------------------------- gemm

enc_status check_gemm(Err &e, const enc_gemm_desc *d, const enc_gemm_item *items, uint32_t n) {
    if (!d || !items) return e.set(ENC_EINVAL, "gemm_items: null descriptor or items");
    if (n < 1 || n > ENC_MAX_GEMM_ITEMS)
        return e.set(ENC_EINVAL, "gemm_items: nitems %u outside 1..%d", n, ENC_MAX_GEMM_ITEMS);
    if (d->path != ENC_F32 && d->path != ENC_I8F16)
        return e.set(ENC_EINVAL, "gemm_items: unknown path %u", d->path);
    if (!d->x || !d->y) return e.set(ENC_EINVAL, "gemm_items: null x or y");
    if (d->flags & ~31u) return e.set(ENC_EINVAL, "gemm_items: unknown flags 0x%x", d->flags);
    if ((d->flags & ENC_Y_F16) && (d->flags & ENC_Y_ACCUMULATE))
        return e.set(ENC_EUNSUPPORTED, "gemm_items: accumulate needs an f32 output");
    const bool gated = d->flags & (ENC_EPI_GATE_GELU_TANH | ENC_EPI_GATE_SILU);
    if (gated && ((d->flags & ENC_EPI_GATE_GELU_TANH) && (d->flags & ENC_EPI_GATE_SILU)))
        return e.set(ENC_EINVAL, "gemm_items: two gated activations");
    if (gated && (d->flags & (ENC_Y_ACCUMULATE | ENC_EPI_GELU_TANH)))
        return e.set(ENC_EUNSUPPORTED, "gemm_items: a gated epilogue takes no accumulate or GELU flag");
    const bool i8 = d->path == ENC_I8F16;
    const uint32_t kal = i8 ? 16 : 4, xal = i8 ? 8 : 4;
    if (!aligned(d->x, 16) || !aligned(d->y, 4))
        return e.set(ENC_EUNSUPPORTED, "gemm_items: x must be 16-byte aligned");
    for (uint32_t i = 0; i < n; i++) {
        const enc_gemm_item &it = items[i];
        if (it.slot >= 4) return e.set(ENC_EINVAL, "gemm_items: item %u slot %u", i, it.slot);
        if (!d->w[it.slot])
            return e.set(ENC_EINVAL, "gemm_items: item %u: null weight in slot %u", i, it.slot);
        if (!aligned(d->w[it.slot], 16))
            return e.set(ENC_EUNSUPPORTED, "gemm_items: weight slot %u not 16-byte aligned", it.slot);
        if (i8 && !d->row_scale[it.slot])
            return e.set(ENC_EINVAL, "gemm_items: item %u: int8 weights need row scales", i);
        if (gated) {
            if (it.slot + 1 >= 4 || !d->w[it.slot + 1] || (i8 && !d->row_scale[it.slot + 1]))
                return e.set(ENC_EINVAL, "gemm_items: gated item %u needs up weights in slot %u", i,
                             it.slot + 1);
            if (!aligned(d->w[it.slot + 1], 16))
                return e.set(ENC_EUNSUPPORTED, "gemm_items: weight slot %u not 16-byte aligned", it.slot + 1);
            if (d->bias[it.slot] || d->bias[it.slot + 1])
                return e.set(ENC_EUNSUPPORTED, "gemm_items: a gated item takes no bias");
        }
        if (it.m == 0 || it.k == 0)
            return e.set(ENC_ESHAPE, "gemm_items: item %u has m=%u k=%u", i, it.m, it.k);
        if (it.k % kal)
            return e.set(ENC_EUNSUPPORTED, "gemm_items: item %u: k=%u not a multiple of %u", i, it.k,
                         kal);
        if (it.ldx < it.k || it.ldy < it.m)
            return e.set(ENC_ESHAPE, "gemm_items: item %u: ldx %u < k %u or ldy %u < m %u", i,
                         it.ldx, it.k, it.ldy, it.m);
        if (it.ldx % xal || it.x_off % xal)
            return e.set(ENC_EUNSUPPORTED, "gemm_items: item %u: ldx/x_off not multiples of %u", i,
                         xal);
        if ((uint64_t)it.n * it.ldx > (1ull << 40) || (uint64_t)it.n * it.ldy > (1ull << 40))
            return e.set(ENC_ESHAPE, "gemm_items: item %u too large", i);
    }
    if (!std::isfinite(d->y_scale) || !std::isfinite(d->alpha))
        return e.set(ENC_EINVAL, "gemm_items: alpha or y_scale not finite");
    // Y regions of different items must not overlap (2-D rectangles when the
    // strides agree, else address intervals).
    for (uint32_t i = 0; i < n; i++)
        for (uint32_t j = i + 1; j < n; j++) {
            const enc_gemm_item &a = items[i], &b = items[j];
            if (!a.n || !b.n) continue;
            bool overlap;
            if (a.ldy == b.ldy && a.y_off % a.ldy + a.m <= a.ldy && b.y_off % b.ldy + b.m <= b.ldy) {
                const uint64_t ar = a.y_off / a.ldy, ac = a.y_off % a.ldy;
                const uint64_t br = b.y_off / b.ldy, bc = b.y_off % b.ldy;
                overlap = ar < br + b.n && br < ar + a.n && ac < bc + b.m && bc < ac + a.m;
            } else {
                const uint64_t a0 = a.y_off, a1 = a.y_off + (uint64_t)(a.n - 1) * a.ldy + a.m;
                const uint64_t b0 = b.y_off, b1 = b.y_off + (uint64_t)(b.n - 1) * b.ldy + b.m;
                overlap = a0 < b1 && b0 < a1;
            }
            if (overlap) return e.set(ENC_EINVAL, "gemm_items: items %u and %u write overlapping Y", i, j);
        }
    return ENC_OK;
}

void plan_gemm(const enc_gemm_desc *d, const enc_gemm_item *items, uint32_t n, GemmArgs &g) {
    memset(&g, 0, sizeof g);
    g.x = d->x;
    g.y = d->y;
    for (int s = 0; s < 4; s++) {
        g.w[s] = d->w[s];
        g.rs[s] = d->row_scale[s];
        g.bias[s] = d->bias[s];
    }
    g.alpha = d->alpha;
    g.flags = d->flags;
    g.ycol = d->y_col;
    g.yscale = d->y_scale == 0.0f ? 1.0f : d->y_scale;
    g.nitems = n;
    uint32_t tiles = 0;
    for (uint32_t i = 0; i < n; i++) {
        GemmItemK &k = g.items[i];
        k.n = items[i].n;
        k.m = items[i].m;
        k.k = items[i].k;
        k.ldx = items[i].ldx;
        k.ldy = items[i].ldy;
        k.slot = items[i].slot;
        k.x_off = items[i].x_off;
        k.y_off = items[i].y_off;
        k.tiles_m = (k.m + kGemmBN - 1) / kGemmBN;
        k.tile0 = tiles;
        tiles += k.tiles_m * ((k.n + kGemmBM - 1) / kGemmBM);
    }
    // unused trailing items never match (tile0 beyond every tile)
    for (uint32_t i = n; i < (uint32_t)kMaxGemmItems; i++) g.items[i].tile0 = 0xffffffffu;
    g.total_tiles = tiles;
}

hipError_t run_gemm(const enc_gemm_desc *d, const enc_gemm_item *items, uint32_t n, hipStream_t s) {
    GemmArgs g;
    plan_gemm(d, items, n, g);
    // algorithmic work: 2 n m k flops per product; bytes = X read once, each
    // weight matrix read once, Y written once (read too when accumulating)
    double flops = 0, bytes = 0;
    const bool gated = d->flags & (ENC_EPI_GATE_GELU_TANH | ENC_EPI_GATE_SILU);
    const double mul = gated ? 2.0 : 1.0;
    const double xs = d->path == ENC_I8F16 ? 2 : 4, ws = d->path == ENC_I8F16 ? 1 : 4;
    const double ys = (d->flags & ENC_Y_F16) ? 2 : 4, yrw = (d->flags & ENC_Y_ACCUMULATE) ? 2 : 1;
    for (uint32_t i = 0; i < n; i++) {
        const enc_gemm_item &it = items[i];
        flops += 2.0 * mul * it.n * it.m * it.k;
        bytes += xs * it.n * it.k + ws * mul * it.m * it.k + ys * yrw * it.n * it.m;
    }
    return prof_launch(ENC_CLASS_GEMM, s, flops, bytes, [&] {
        return d->path == ENC_I8F16 ? launch_gemm_i8f16(g, s) : launch_gemm_f32(g, s);
    });
}

// ----------------------------------------------------------- attention

uint32_t item_len(const enc_item &it) { return it.r[0].n + (it.nr > 1 ? it.r[1].n : 0); }

// (query, key) pairs the mask lets through in an item of L rows: L^2 when
// full, else L(2W+1) - W(W+1) (each edge row loses the part of its band that
// falls outside the item).
double visible_pairs(uint32_t L, uint32_t W) {
    if (W == 0 || W + 1 >= L) return (double)L * L;
    return (double)L * (2.0 * W + 1.0) - (double)W * (W + 1.0);
}

enc_status check_items(Err &e, const char *who, const enc_item *items, uint32_t n, uint32_t rows) {
    if (!items && n) return e.set(ENC_EINVAL, "%s: null items", who);
    std::vector<std::pair<uint64_t, uint64_t>> rr;
    for (uint32_t i = 0; i < n; i++) {
        const enc_item &it = items[i];
        if (it.nr < 1 || it.nr > 2) return e.set(ENC_EINVAL, "%s: item %u has %u ranges", who, i, it.nr);
        for (uint32_t r = 0; r < it.nr; r++) {
            const uint64_t a = it.r[r].r0, b = a + it.r[r].n;
            if (b > rows)
                return e.set(ENC_EINVAL, "%s: item %u range [%llu,%llu) past %u rows", who, i,
                             (unsigned long long)a, (unsigned long long)b, rows);
            if (b > a) rr.push_back({a, b});
        }
    }
    std::sort(rr.begin(), rr.end());
    for (size_t i = 1; i < rr.size(); i++)
        if (rr[i].first < rr[i - 1].second) return e.set(ENC_EINVAL, "%s: items overlap", who);
    return ENC_OK;
}

// Key split of one item.  An item whose q-tiles alone would leave most CUs
// idle is cut into nsplit key chunks (multiples of the 32-key block); each
// (q-tile, chunk) block writes a partial softmax, merged afterwards in a fixed
// order.  The plan depends only on the item's own length and the launch-wide
// geometry (path, heads, window), never on the other items, so a packed batch
// and its items run alone give the same bits.  f32 path, windowless items only.
constexpr uint32_t kAttnQT = 128;      // queries per f32 attention block
constexpr uint32_t kSplitTarget = 768; // blocks an item alone should reach
constexpr uint32_t kSplitMinKeys = 128;
constexpr uint32_t kSplitMax = 8;

struct KvSplit {
    uint32_t n, chunk;
};

KvSplit kv_split(const enc_attn_desc *d, uint32_t L) {
    if (d->path != ENC_F32 || d->window || L < 2 * kSplitMinKeys) return {1, L};
    const uint32_t blocks = (L + kAttnQT - 1) / kAttnQT * d->nq;
    const uint32_t s = std::min({kSplitMax, kSplitTarget / blocks, L / kSplitMinKeys});
    if (s < 2) return {1, L};
    const uint32_t chunk = ((L + s - 1) / s + 31) / 32 * 32;
    return {(L + chunk - 1) / chunk, chunk};
}

// Items in launch order (longest first: their tiles carry the most key blocks).
std::vector<uint32_t> attn_order(const enc_item *items, uint32_t n) {
    std::vector<uint32_t> order;
    for (uint32_t i = 0; i < n; i++)
        if (item_len(items[i])) order.push_back(i);
    std::stable_sort(order.begin(), order.end(),
                     [&](uint32_t a, uint32_t b) { return item_len(items[a]) > item_len(items[b]); });
    return order;
}

// Partial-result records (one per split, item row and head) of the largest
// launch; launches run in stream order and reuse the same workspace.
uint64_t attn_records(const enc_attn_desc *d, const enc_item *items, uint32_t n) {
    const std::vector<uint32_t> order = attn_order(items, n);
    uint64_t most = 0;
    for (size_t c0 = 0; c0 < order.size(); c0 += kMaxAttnItems) {
        uint64_t r = 0;
        for (size_t c = c0; c < std::min(order.size(), c0 + (size_t)kMaxAttnItems); c++) {
            const uint32_t L = item_len(items[order[c]]);
            const KvSplit k = kv_split(d, L);
            if (k.n > 1) r += (uint64_t)k.n * L * d->nq;
        }
        most = std::max(most, r);
    }
    return most;
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t attn_ws_bytes(const enc_attn_desc *d, const enc_item *items, uint32_t n) {
    const uint64_t r = attn_records(d, items, n);
    return r ? up256(r * d->hd * 4) + up256(r * 8) : 0;
}

enc_status check_attn(Err &e, const enc_attn_desc *d, const enc_item *items, uint32_t n) {
    if (!d) return e.set(ENC_EINVAL, "attention_items: null descriptor");
    if (d->path != ENC_F32 && d->path != ENC_I8F16)
        return e.set(ENC_EINVAL, "attention_items: unknown path %u", d->path);
    if (!d->qkv || !d->out) return e.set(ENC_EINVAL, "attention_items: null panel or output");
    if (d->hd != 64 && d->hd != 128)
        return e.set(ENC_EUNSUPPORTED, "attention_items: head dim %u (64 or 128)", d->hd);
    if (!d->nq || !d->nkv || d->nq % d->nkv)
        return e.set(ENC_EINVAL, "attention_items: nq %u not a multiple of nkv %u", d->nq, d->nkv);
    if (d->ld % 8 || d->ldo % 8 || d->q_col % 8 || d->k_col % 8 || d->v_col % 8)
        return e.set(ENC_EUNSUPPORTED, "attention_items: strides and column offsets must be multiples of 8");
    if (d->q_col + d->nq * d->hd > d->ld || d->k_col + d->nkv * d->hd > d->ld ||
        d->v_col + d->nkv * d->hd > d->ld)
        return e.set(ENC_ESHAPE, "attention_items: q/k/v blocks do not fit the panel width %u", d->ld);
    if (d->ldo < d->nq * d->hd)
        return e.set(ENC_ESHAPE, "attention_items: ldo %u < nq*hd %u", d->ldo, d->nq * d->hd);
    if (!aligned(d->qkv, 16) || !aligned(d->out, 16))
        return e.set(ENC_EUNSUPPORTED, "attention_items: panel/output must be 16-byte aligned");
    if (!(d->scale == d->scale) || std::isinf(d->scale) || !std::isfinite(d->out_scale))
        return e.set(ENC_EINVAL, "attention_items: scale or out_scale is not finite");
    if (d->out_col && !aligned(d->out_col, 16))
        return e.set(ENC_EUNSUPPORTED, "attention_items: out_col must be 16-byte aligned");
    if (check_items(e, "attention_items", items, n, d->rows) != ENC_OK) return e.st;
    if (d->ws) {
        if (!aligned(d->ws, 256))
            return e.set(ENC_EUNSUPPORTED, "attention_items: workspace must be 256-byte aligned");
        const size_t need = attn_ws_bytes(d, items, n);
        if (d->ws_bytes < need)
            return e.set(ENC_ESHAPE, "attention_items: workspace of %zu bytes, %zu needed",
                         (size_t)d->ws_bytes, need);
    }
    return ENC_OK;
}

hipError_t run_attention(const enc_attn_desc *d, const enc_item *items, uint32_t n, hipStream_t s) {
    const std::vector<uint32_t> order = attn_order(items, n);
    const uint64_t records = d->ws ? attn_records(d, items, n) : 0;
    float *part_o = (float *)d->ws;
    float *part_ml = records ? (float *)((char *)d->ws + up256(records * d->hd * 4)) : nullptr;
    for (size_t c0 = 0; c0 < order.size(); c0 += kMaxAttnItems) {
        AttnArgs a;
        memset(&a, 0, sizeof a);
        a.qkv = d->qkv;
        a.out = d->out;
        a.ld = d->ld;
        a.ldo = d->ldo;
        a.q_col = d->q_col;
        a.k_col = d->k_col;
        a.v_col = d->v_col;
        a.nq = d->nq;
        a.group = d->nq / d->nkv;
        a.scale_log2 = (float)((double)d->scale * 1.4426950408889634);
        a.window = d->window;
        a.part_o = part_o;
        a.part_ml = part_ml;
        a.ocol = d->out_col;
        a.oscale = d->out_scale == 0.0f ? 1.0f : d->out_scale;
        a.rows = d->rows;
        CombineArgs cb;
        memset(&cb, 0, sizeof cb);
        cb.part_o = part_o;
        cb.part_ml = part_ml;
        cb.out = d->out;
        cb.ldo = d->ldo;
        cb.nq = d->nq;
        cb.hd = d->hd;
        cb.ocol = a.ocol;
        cb.oscale = a.oscale;
        uint32_t k = 0, part = 0;
        double pairs = 0;
        for (size_t c = c0; c < std::min(order.size(), c0 + (size_t)kMaxAttnItems); c++, k++) {
            const enc_item &it = items[order[c]];
            AttnItemK &ik = a.items[k];
            ik.r0a = it.r[0].r0;
            ik.na = it.r[0].n;
            ik.r0b = it.nr > 1 ? it.r[1].r0 : 0;
            ik.nb = it.nr > 1 ? it.r[1].n : 0;
            const uint32_t L = item_len(it);
            const KvSplit ks = records ? kv_split(d, L) : KvSplit{1, L};
            ik.nsplit = ks.n;
            ik.chunk = ks.chunk;
            if (ks.n > 1) {
                ik.part0 = part;
                part += ks.n * L * d->nq;
                cb.items[cb.nitems] = ik;
                cb.row0[cb.nitems + 1] = cb.row0[cb.nitems] + L;
                cb.nitems++;
            }
            pairs += visible_pairs(L, d->window);
        }
        a.nitems = k;
        hipError_t h = prof_launch(ENC_CLASS_ATTN, s, 4.0 * d->hd * d->nq * pairs, 0.0, [&] {
            return d->path == ENC_I8F16 ? launch_attn_f16(a, d->hd, s) : launch_attn_f32(a, d->hd, s);
        });
        if (h != hipSuccess) return h;
        if (cb.nitems) {
            // bytes: every partial (hd + 2 floats) read once, the merged rows written once
            const double rec = (double)part, esz = d->path == ENC_I8F16 ? 2 : 4;
            const double bytes = rec * (d->hd + 2) * 4 + (double)cb.row0[cb.nitems] * d->nq * d->hd * esz;
            h = prof_launch(ENC_CLASS_ATTN, s, 0.0, bytes, [&] {
                return launch_attn_combine(cb, d->path == ENC_I8F16, s);
            });
            if (h != hipSuccess) return h;
        }
    }
    return hipSuccess;
}

// ------------------------------------------------------------ row ops

enc_status check_norm(Err &e, const char *who, const enc_norm_desc *d) {
    if (!d) return e.set(ENC_EINVAL, "%s: null descriptor", who);
    // no rows: nothing is read or written, so the pointers may be null
    if (d->rows && (!d->x || !d->w || !d->y)) return e.set(ENC_EINVAL, "%s: null x, w or y", who);
    if (d->flags & ~1u) return e.set(ENC_EINVAL, "%s: unknown flags", who);
    if (d->d == 0 || d->d % 4 || d->d > 4096)
        return e.set(ENC_EUNSUPPORTED, "%s: width %u (multiple of 4, <= 4096)", who, d->d);
    if (d->ldx < d->d || d->ldy < d->d) return e.set(ENC_ESHAPE, "%s: stride below width", who);
    if (d->ldx % 4 || d->ldy % 4 || !aligned(d->x, 16) || !aligned(d->y, 16) || !aligned(d->w, 16) ||
        (d->b && !aligned(d->b, 16)))
        return e.set(ENC_EUNSUPPORTED, "%s: pointers 16-byte aligned, strides multiples of 4", who);
    if (!std::isfinite(d->pre)) return e.set(ENC_EINVAL, "%s: pre is not finite", who);
    return ENC_OK;
}

enc_status check_add_norm(Err &e, const enc_add_norm_desc *d) {
    if (!d) return e.set(ENC_EINVAL, "enc_add_norm: null descriptor");
    if (!d->h) return e.set(ENC_EINVAL, "enc_add_norm: null h");
    if (d->t && !d->w_post) return e.set(ENC_EINVAL, "enc_add_norm: null w_post");
    if (!d->t && !d->w_next) return e.set(ENC_EINVAL, "enc_add_norm: neither t nor w_next");
    if (d->w_next && !d->a) return e.set(ENC_EINVAL, "enc_add_norm: w_next without an output");
    if (d->nout > 3) return e.set(ENC_EINVAL, "enc_add_norm: nout %u (1..3)", d->nout);
    if (!std::isfinite(d->oscale)) return e.set(ENC_EINVAL, "enc_add_norm: oscale is not finite");
    for (const float *v : {d->gate, d->scale, d->col[0], d->col[1], d->col[2]})
        if (v && !aligned(v, 16)) return e.set(ENC_EUNSUPPORTED, "enc_add_norm: vectors must be 16-byte aligned");
    if (d->flags & ~1u) return e.set(ENC_EINVAL, "enc_add_norm: unknown flags");
    if (d->d == 0 || d->d % 4 || d->d > 4096)
        return e.set(ENC_EUNSUPPORTED, "enc_add_norm: width %u (multiple of 4, <= 4096)", d->d);
    if (!aligned(d->h, 16) || (d->t && (!aligned(d->t, 16) || !aligned(d->w_post, 16))) ||
        (d->w_next && (!aligned(d->w_next, 16) || !aligned(d->a, 16))))
        return e.set(ENC_EUNSUPPORTED, "enc_add_norm: pointers must be 16-byte aligned");
    if (!std::isfinite(d->post)) return e.set(ENC_EINVAL, "enc_add_norm: post is not finite");
    return ENC_OK;
}

enc_status check_qk(Err &e, const enc_qk_desc *d) {
    if (!d) return e.set(ENC_EINVAL, "enc_qk_norm_rope: null descriptor");
    if (d->path != ENC_F32 && d->path != ENC_I8F16) return e.set(ENC_EINVAL, "enc_qk_norm_rope: path");
    if (!d->panel || !d->q_norm_w || !d->k_norm_w)
        return e.set(ENC_EINVAL, "enc_qk_norm_rope: null panel or norm weights");
    if (d->hd != 64 && d->hd != 128)
        return e.set(ENC_EUNSUPPORTED, "enc_qk_norm_rope: head dim %u (64 or 128)", d->hd);
    if (d->sections > 2) return e.set(ENC_EINVAL, "enc_qk_norm_rope: sections %u", d->sections);
    if (d->sections && (!d->cos || !d->sin)) return e.set(ENC_EINVAL, "enc_qk_norm_rope: null cos/sin");
    if (d->q_col + d->nq * d->hd > d->ld || d->k_col + d->nkv * d->hd > d->ld ||
        (d->v_norm && d->v_col + d->nkv * d->hd > d->ld))
        return e.set(ENC_ESHAPE, "enc_qk_norm_rope: heads do not fit the panel width");
    if (d->v_norm > 1) return e.set(ENC_EINVAL, "enc_qk_norm_rope: v_norm %u", d->v_norm);
    if (d->ld % 8 || d->q_col % 8 || d->k_col % 8 || d->v_col % 8 || !aligned(d->panel, 16))
        return e.set(ENC_EUNSUPPORTED,
                     "enc_qk_norm_rope: panel 16-byte aligned, stride and columns multiples of 8");
    if ((uint64_t)d->rows * (d->nq + d->nkv) >= (1ull << 32) / 4)
        return e.set(ENC_ESHAPE, "enc_qk_norm_rope: too many rows");
    return ENC_OK;
}

enc_status check_act(Err &e, const enc_act_desc *d) {
    if (!d) return e.set(ENC_EINVAL, "enc_gated_act: null descriptor");
    if (d->kind != ENC_ACT_GELU_TANH_GATED && d->kind != ENC_ACT_SWIGLU)
        return e.set(ENC_EINVAL, "enc_gated_act: unknown kind %u", d->kind);
    if (!d->g || !d->u || !d->out) return e.set(ENC_EINVAL, "enc_gated_act: null pointer");
    if (d->flags & ~1u) return e.set(ENC_EINVAL, "enc_gated_act: unknown flags");
    if (d->ff % 4 || d->ldg % 4 || d->ldu % 4 || d->ldo % 4 || !aligned(d->g, 16) ||
        !aligned(d->u, 16) || !aligned(d->out, 16))
        return e.set(ENC_EUNSUPPORTED, "enc_gated_act: widths/strides multiples of 4, 16-byte pointers");
    if (d->ldg < d->ff || d->ldu < d->ff || d->ldo < d->ff)
        return e.set(ENC_ESHAPE, "enc_gated_act: stride below width");
    if ((d->out_col && !aligned(d->out_col, 16)) || !std::isfinite(d->out_scale))
        return e.set(ENC_EINVAL, "enc_gated_act: out_col 16-byte aligned, out_scale finite");
    return ENC_OK;
}

// ------------------------------------------------------------ model

// Row-op launches with their algorithmic HBM bytes (inputs read once, outputs
// written once, per-channel weights once).
hipError_t rows_rms(const NormArgs &n, bool f16, hipStream_t s) {
    const double b = (double)n.rows * n.d * (4 + (f16 ? 2 : 4)) + 4.0 * n.d;
    return prof_launch(ENC_CLASS_ROWS, s, 0, b, [&] { return launch_rms_norm(n, f16, s); });
}
hipError_t rows_ln(const NormArgs &n, bool f16, hipStream_t s) {
    const double b = (double)n.rows * n.d * (4 + (f16 ? 2 : 4)) + 8.0 * n.d;
    return prof_launch(ENC_CLASS_ROWS, s, 0, b, [&] { return launch_layer_norm(n, f16, s); });
}
hipError_t rows_add_norm(const AddNormArgs &a, bool f16, hipStream_t s) {
    const double b = (double)a.rows * a.d * ((a.t ? 12 : 4) + (a.w_next ? (f16 ? 2 : 4) * a.nout : 0)) +
                     8.0 * a.d;
    return prof_launch(ENC_CLASS_ROWS, s, 0, b, [&] { return launch_add_norm(a, f16, s); });
}
hipError_t rows_qk(const QkArgs &q, bool f16, hipStream_t s) {
    const double b = (double)q.rows * (q.nq + q.nkv) * q.hd * (f16 ? 4 : 8) +
                     (q.sections ? (double)q.rows * q.hd * 4 : 0.0) + 8.0 * q.hd;
    return prof_launch(ENC_CLASS_ROWS, s, 0, b, [&] { return launch_qk_norm_rope(q, f16, s); });
}
hipError_t rows_act(const ActArgs &a, bool f16, hipStream_t s) {
    const double b = (double)a.rows * a.ff * (8 + (f16 ? 2 : 4));
    return prof_launch(ENC_CLASS_ROWS, s, 0, b, [&] { return launch_gated_act(a, f16, s); });
}
hipError_t rows_pool(const PoolArgs &p, uint32_t rows, hipStream_t s) {
    const double b = (double)rows * p.d * 4 + (double)p.nitems * p.d * 4;
    return prof_launch(ENC_CLASS_ROWS, s, 0, b, [&] { return launch_mean_pool(p, s); });
}

// Mean pool of any number of items: launches of at most kMaxAttnItems items.
hipError_t pool_items(const enc_item *items, uint32_t nitems, uint32_t rows, uint32_t d, const float *a,
                      float *out, hipStream_t s) {
    for (uint32_t i0 = 0; i0 < nitems; i0 += kMaxAttnItems) {
        PoolArgs p;
        memset(&p, 0, sizeof p);
        p.d = d;
        p.nitems = std::min<uint32_t>(kMaxAttnItems, nitems - i0);
        p.a = a;
        p.out = out + (size_t)i0 * d;
        for (uint32_t i = 0; i < p.nitems; i++) {
            const enc_item &it = items[i0 + i];
            p.items[i].r0a = it.r[0].r0;
            p.items[i].na = it.r[0].n;
            p.items[i].r0b = it.nr > 1 ? it.r[1].r0 : 0;
            p.items[i].nb = it.nr > 1 ? it.r[1].n : 0;
        }
        const hipError_t hr = rows_pool(p, rows, s);
        if (hr != hipSuccess) return hr;
    }
    return hipSuccess;
}

struct WsPlan {
    size_t a = 0, panel = 0, att = 0, t = 0, part = 0, m = 0, h = 0, pin = 0, z = 0, gu = 0, amax = 0,
           total = 0;
    size_t part_bytes = 0;
};

float p2(int e) { return ldexpf(1.0f, e); }

// Copies of the attention input A the q/k/v GEMM reads (one per column field)
// and of the FFN input the gate/up GEMM reads.
uint32_t nout_attn(const enc_layer &L) { return (L.col_q || L.col_k || L.col_v) ? 3 : 1; }
uint32_t nout_ff(const enc_layer &L) { return (L.col_gate || L.col_up) ? 2 : 1; }
bool unfused_gate(const enc_layer &L) { return L.mlp != ENC_MLP_GELU_TANH && nout_ff(L) > 1; }

// The attention descriptor of one layer over the batch's panel.
enc_attn_desc layer_attn_desc(const enc_layer &L, uint32_t rows) {
    const uint32_t qw = L.nq * L.hd, kw = L.nkv * L.hd;
    enc_attn_desc a{};
    a.path = L.path;
    a.ld = qw + 2 * kw;
    a.q_col = 0;
    a.k_col = qw;
    a.v_col = qw + kw;
    a.ldo = qw;
    a.nq = L.nq;
    a.nkv = L.nkv;
    a.hd = L.hd;
    a.scale = L.attn_scale;
    a.window = L.window;
    a.rows = rows;
    return a;
}

WsPlan plan_ws(const enc_model *M, const enc_batch *B) {
    WsPlan p;
    const uint32_t rows = B->rows;
    size_t a = 0, panel = 0, att = 0, t = 0, part = 0, m = 0, h = 0, ple = 0, gu = 0;
    for (uint32_t l = 0; l < M->nlayers; l++) {
        const enc_layer &L = M->layers[l];
        const size_t esz = L.path == ENC_I8F16 ? 2 : 4;
        a = std::max(a, (size_t)rows * L.d * esz * std::max(nout_attn(L), nout_ff(L)));
        if (unfused_gate(L)) gu = std::max(gu, (size_t)rows * 2 * L.ff * 4);
        panel = std::max(panel, (size_t)rows * (L.nq + 2 * L.nkv) * L.hd * esz);
        att = std::max(att, (size_t)rows * L.nq * L.hd * esz);
        t = std::max(t, (size_t)rows * L.d * 4);
        const enc_attn_desc ad = layer_attn_desc(L, rows);
        part = std::max(part, attn_ws_bytes(&ad, B->items, B->nitems));
        m = std::max(m, (size_t)rows * L.ff * (L.mlp == ENC_MLP_GELU_TANH ? 4 : esz));
        h = std::max(h, (size_t)rows * L.d * 4);
        ple = std::max(ple, (size_t)rows * L.n_ple * 4);
    }
    size_t off = 0;
    p.a = off; off += up256(a);
    p.panel = off; off += up256(panel);
    p.att = off; off += up256(att);
    p.t = off; off += up256(t);
    p.part = off; off += up256(part);
    p.part_bytes = up256(part);
    p.m = off; off += up256(m);
    p.h = off; off += up256(h);  // residual stream (out holds it when final is NONE)
    p.pin = off; off += up256(ple);  // per-layer input: normed projection of X0
    p.z = off; off += up256(ple);    // and its gate
    p.gu = off; off += up256(gu);    // gate|up of an unfused gated MLP
    p.amax = off; off += B->amax ? up256(kAmaxBlocks * 4) : 0;  // per-block maxima of the amax pass
    p.total = off;
    return p;
}

enc_status check_layer(Err &e, uint32_t l, const enc_layer &L, const enc_layer &L0) {
    if (L.block > 1 || L.path > 1 || L.mlp > 2)
        return e.set(ENC_EINVAL, "layer %u: unknown block/path/mlp", l);
    if (L.block != L0.block || L.path != L0.path || L.d != L0.d)
        return e.set(ENC_EUNSUPPORTED, "layer %u: block kind, path and width must match layer 0", l);
    if (L.d == 0 || L.d % 64 || L.d > 4096)
        return e.set(ENC_EUNSUPPORTED, "layer %u: d %u (multiple of 64, <= 4096)", l, L.d);
    if (L.ff == 0 || L.ff % 64) return e.set(ENC_EUNSUPPORTED, "layer %u: ff %u (multiple of 64)", l, L.ff);
    if (L.hd != 64 && L.hd != 128) return e.set(ENC_EUNSUPPORTED, "layer %u: head dim %u", l, L.hd);
    if (!L.nq || !L.nkv || L.nq % L.nkv) return e.set(ENC_EINVAL, "layer %u: nq %% nkv != 0", l);
    if (L.rope_sections > 2) return e.set(ENC_EINVAL, "layer %u: rope_sections %u", l, L.rope_sections);
    if (!(L.eps >= 0.0f) || !std::isfinite(L.attn_scale))
        return e.set(ENC_EINVAL, "layer %u: eps/scale not finite", l);
    if (!L.wq || !L.wk || !L.wv || !L.wo || !L.w_up || !L.w_down)
        return e.set(ENC_EINVAL, "layer %u: null projection weight", l);
    if (L.mlp != ENC_MLP_GELU_TANH && !L.w_gate) return e.set(ENC_EINVAL, "layer %u: gated MLP needs w_gate", l);
    if (L.path == ENC_I8F16 &&
        (!L.sq || !L.sk || !L.sv || !L.so || !L.s_up || !L.s_down || (L.w_gate && !L.s_gate)))
        return e.set(ENC_EINVAL, "layer %u: int8 weights need row scales", l);
    if (!L.norm1_w || !L.norm2_w) return e.set(ENC_EINVAL, "layer %u: null norm weights", l);
    if (L.block == ENC_SANDWICH_RMS) {
        if (!L.post_attn_w || !L.post_ff_w || !L.q_norm_w || !L.k_norm_w)
            return e.set(ENC_EINVAL, "layer %u: sandwich block needs post/q/k norm weights", l);
        if (L.mlp == ENC_MLP_GELU_TANH)
            return e.set(ENC_EUNSUPPORTED, "layer %u: sandwich block takes a gated MLP", l);
        if (L.v_norm > 1) return e.set(ENC_EINVAL, "layer %u: v_norm %u", l, L.v_norm);
        if (L.rope_table >= ENC_MAX_ROPE_TABLES)
            return e.set(ENC_EINVAL, "layer %u: rope_table %u", l, L.rope_table);
        if (!std::isfinite(L.scalar)) return e.set(ENC_EINVAL, "layer %u: scalar not finite", l);
        const uint32_t gmax = std::max({L.guard_attn, L.guard_qkv, L.guard_ao, L.guard_ffn, L.guard_hid});
        const bool cols = L.col_q || L.col_k || L.col_v || L.col_o || L.col_gate || L.col_up || L.col_down;
        if (L.path != ENC_I8F16 && (gmax || cols))
            return e.set(ENC_EUNSUPPORTED, "layer %u: column fields and guards are int8-path options", l);
        if (gmax > 14) return e.set(ENC_EINVAL, "layer %u: guard above 14", l);
        if (L.v_norm && L.guard_qkv)
            return e.set(ENC_EUNSUPPORTED, "layer %u: v-norm takes no panel guard", l);
        for (const float *v : {L.mod_s_attn, L.mod_g_attn, L.mod_s_ff, L.mod_g_ff, L.col_q, L.col_k, L.col_v,
                               L.col_o, L.col_gate, L.col_up, L.col_down})
            if (v && !aligned(v, 16))
                return e.set(ENC_EUNSUPPORTED, "layer %u: modulation and column fields 16-byte aligned", l);
        if (L.n_ple) {
            if (L.path != ENC_F32)
                return e.set(ENC_EUNSUPPORTED, "layer %u: the per-layer input runs the f32 path", l);
            if (L.n_ple % 64) return e.set(ENC_EUNSUPPORTED, "layer %u: n_ple %u (multiple of 64)", l, L.n_ple);
            if (!L.ple_in || !L.ple_gate || !L.ple_proj || !L.ple_in_norm_w || !L.ple_post_w)
                return e.set(ENC_EINVAL, "layer %u: per-layer input needs its weights", l);
            if (!std::isfinite(L.ple_scale)) return e.set(ENC_EINVAL, "layer %u: ple_scale not finite", l);
        }
    } else {
        if (L.v_norm || L.n_ple || (L.scalar != 0.0f && L.scalar != 1.0f) || L.rope_table || L.mod_s_attn ||
            L.mod_g_attn || L.mod_s_ff || L.mod_g_ff)
            return e.set(ENC_EUNSUPPORTED,
                         "layer %u: v-norm, per-layer input, scalar and modulation are sandwich options", l);
        if (L.path == ENC_I8F16) return e.set(ENC_EUNSUPPORTED, "layer %u: pre-LN block runs the f32 path", l);
        if (L.mlp != ENC_MLP_GELU_TANH)
            return e.set(ENC_EUNSUPPORTED, "layer %u: pre-LN block takes the GELU MLP", l);
        if (L.rope_sections) return e.set(ENC_EUNSUPPORTED, "layer %u: pre-LN block has no RoPE", l);
    }
    return ENC_OK;
}

enc_status check_model(Err &e, const enc_model *M, const enc_batch *B) {
    if (!M || !B) return e.set(ENC_EINVAL, "null model or batch");
    if (M->nlayers && !M->layers) return e.set(ENC_EINVAL, "null layers");
    if (M->final_kind > 2) return e.set(ENC_EINVAL, "unknown final kind %u", M->final_kind);
    if (M->final_kind != ENC_FINAL_NONE && !M->final_w) return e.set(ENC_EINVAL, "final norm needs final_w");
    if (M->nlayers == 0 && M->final_kind != ENC_FINAL_NONE)
        return e.set(ENC_EINVAL, "a final norm needs at least one layer (for the width)");
    for (uint32_t l = 0; l < M->nlayers; l++)
        if (check_layer(e, l, M->layers[l], M->layers[0]) != ENC_OK) return e.st;
    if (!B->rows) return e.set(ENC_ESHAPE, "empty batch");
    if (!B->nitems || !B->items) return e.set(ENC_EINVAL, "batch has no items");
    if (check_items(e, "batch", B->items, B->nitems, B->rows) != ENC_OK) return e.st;
    uint64_t covered = 0;
    for (uint32_t i = 0; i < B->nitems; i++) covered += item_len(B->items[i]);
    if (covered != B->rows) return e.set(ENC_ESHAPE, "items cover %llu of %u rows", (unsigned long long)covered, B->rows);
    if (M->final_kind == ENC_FINAL_RMS_MEANPOOL)
        for (uint32_t i = 0; i < B->nitems; i++)
            if (!item_len(B->items[i]))
                return e.set(ENC_EINVAL, "item %u is empty: its mean pool is undefined", i);
    for (uint32_t l = 0; l < M->nlayers; l++) {
        const enc_layer &L = M->layers[l];
        if (L.rope_sections && (!B->rope_cos[L.rope_table] || !B->rope_sin[L.rope_table]))
            return e.set(ENC_EINVAL, "layer %u: RoPE table %u missing", l, L.rope_table);
        if (B->amax && L.path != ENC_I8F16)
            return e.set(ENC_EUNSUPPORTED, "amax records the int8 path's half sites");
    }
    return ENC_OK;
}

struct Bufs {
    void *a, *panel, *att;
    float *t;
    void *part;
    size_t part_bytes;
    void *m;
    float *h, *pin, *z, *gu, *amax;
};

Bufs carve(void *ws, const WsPlan &p) {
    char *b = (char *)ws;
    return Bufs{b + p.a, b + p.panel, b + p.att, (float *)(b + p.t), p.part_bytes ? b + p.part : nullptr,
                p.part_bytes, b + p.m, (float *)(b + p.h), (float *)(b + p.pin), (float *)(b + p.z),
                (float *)(b + p.gu), (float *)(b + p.amax)};
}

#define TRY(expr)                                                                               \
    do {                                                                                        \
        hipError_t _h = (expr);                                                                 \
        if (_h != hipSuccess) return _h;                                                        \
    } while (0)

// What a sandwich row op writes after the residual update: the next GEMM's
// half (or f32) inputs, A_z = rms(h) w (1 + scale) col_z 2^-guard.
struct NextIn {
    const float *w = nullptr, *scale = nullptr;
    const float *col[3] = {nullptr, nullptr, nullptr};
    uint32_t nout = 1;
    float oscale = 1.0f;
};

// the q/k/v input of layer N
NextIn attn_in(const enc_layer &N) {
    NextIn r;
    r.w = N.norm1_w;
    r.scale = N.mod_s_attn;
    r.nout = nout_attn(N);
    if (r.nout > 1) {
        r.col[0] = N.col_q;
        r.col[1] = N.col_k;
        r.col[2] = N.col_v;
    }
    r.oscale = p2(-(int)N.guard_attn);
    return r;
}

// the gate/up (or up) input of layer L
NextIn ff_in(const enc_layer &L) {
    NextIn r;
    r.w = L.norm2_w;
    r.scale = L.mod_s_ff;
    r.nout = nout_ff(L);
    if (r.nout > 1) {
        r.col[0] = L.col_gate;
        r.col[1] = L.col_up;
    }
    r.oscale = p2(-(int)L.guard_ffn);
    return r;
}

// The sandwich row op: with t, h = (h + gate rms(t) w_post) post; then the
// next inputs `nx` (none when nx.w == NULL).
hipError_t row_op(const enc_layer &L, uint32_t rows, float *h, const float *t, const float *w_post,
                  const float *gate, float post, const NextIn &nx, void *a, bool f16, hipStream_t s) {
    AddNormArgs an{rows, L.d, h, t, w_post, nx.w, L.eps, a, post};
    an.gate = gate;
    an.scale = nx.scale;
    for (int z = 0; z < 3; z++) an.col[z] = nx.col[z];
    an.nout = nx.nout;
    an.oscale = nx.oscale;
    an.a_stride = (uint64_t)rows * L.d;
    return rows_add_norm(an, f16, s);
}

hipError_t pre_norm(const enc_layer &L, uint32_t rows, float *h, void *a, hipStream_t s) {
    const bool f16 = L.path == ENC_I8F16;
    if (L.block == ENC_SANDWICH_RMS)  // rms(h) of the same helpers as rms_norm: the same bits
        return row_op(L, rows, h, nullptr, nullptr, nullptr, 1.0f, attn_in(L), a, f16, s);
    NormArgs n{rows, L.d, L.d, L.d, h, L.norm1_w, L.norm1_b, L.eps, a};
    return rows_ln(n, f16, s);
}

// max |x| of n halves into *out (the guard calibration of the int8 path)
hipError_t amax_site(const void *x, uint64_t n, float *part, float *out, hipStream_t s) {
    if (!out || !n) return hipSuccess;
    AmaxArgs a{reinterpret_cast<const _Float16 *>(x), n, part,
               (uint32_t)std::min<uint64_t>(kAmaxBlocks, std::max<uint64_t>(1, (n / 8 + 255) / 256)), out};
    return prof_launch(ENC_CLASS_ROWS, s, 0, 2.0 * n, [&] { return launch_amax_f16(a, s); });
}

// The final RMS of a sandwich f32 stack is the last row op's next-norm output
// (same eps), as the pages fuse it.
bool fused_final(const enc_model *M) {
    const enc_layer &L0 = M->layers[0], &Ll = M->layers[M->nlayers - 1];
    return M->final_kind == ENC_FINAL_RMS_MEANPOOL && L0.block == ENC_SANDWICH_RMS && L0.path == ENC_F32 &&
           M->final_eps == Ll.eps;
}

// Per-layer input of a text layer, up to its projection T = Z ple_proj^T:
// P = rms(ple_scale * X0 ple_in^T; ple_in_norm), Z = gelu_tanh(H ple_gate^T) * P.
hipError_t run_ple(const enc_layer &L, uint32_t rows, const float *x0, const float *h, const Bufs &b,
                   hipStream_t s) {
    const uint32_t d = L.d, np = L.n_ple;
    auto proj = [&](const float *x, uint32_t k, const float *w, uint32_t m, float *y) {
        enc_gemm_desc g{};
        g.path = ENC_F32;
        g.x = x;
        g.y = y;
        g.w[0] = w;
        g.alpha = 1.0f;
        enc_gemm_item it{rows, m, k, k, m, 0, 0, 0};
        return run_gemm(&g, &it, 1, s);
    };
    TRY(proj(x0, d, L.ple_in, np, b.pin));
    NormArgs n{rows, np, np, np, b.pin, L.ple_in_norm_w, nullptr, L.eps, b.pin, L.ple_scale};
    TRY(rows_rms(n, false, s));
    TRY(proj(h, d, L.ple_gate, np, b.z));
    ActArgs act{ENC_ACT_GELU_TANH_GATED, rows, np, np, np, np, b.z, b.pin, b.z};
    TRY(rows_act(act, false, s));
    return proj(b.z, np, L.ple_proj, d, b.t);
}

// One layer on h.  ain: for the sandwich block the layer's q/k/v input(s)
// (its pre-norm, already computed); for pre-LN the LN1 output, or NULL for the
// layer to compute it into b.a.  On exit the last row op of a sandwich layer
// has written the next inputs `nx` into aout (none when nx.w == NULL); ain may
// equal aout or b.a (each is read before it is written).  amax: this layer's
// five slots, or NULL.
hipError_t run_layer(const enc_layer &L, const enc_batch *B, const float *x0, float *h, const Bufs &b,
                     const void *ain, void *aout, const NextIn &nx, float *amax, hipStream_t s) {
    const uint32_t rows = B->rows, d = L.d, hd = L.hd;
    const uint32_t qw = L.nq * hd, kw = L.nkv * hd, ld = qw + 2 * kw;
    const bool i8 = L.path == ENC_I8F16;
    const bool sandwich = L.block == ENC_SANDWICH_RMS;
    const int ga = L.guard_attn, gq = L.guard_qkv, gao = L.guard_ao, gf = L.guard_ffn, gh = L.guard_hid;
    const uint64_t rd = (uint64_t)rows * d;
    if (!ain) {
        TRY(pre_norm(L, rows, h, b.a, s));
        ain = b.a;
    }
    if (amax) TRY(amax_site(ain, rd * nout_attn(L), b.amax, amax + 0, s));

    // q|k|v projections: one launch, three items (each reading its own copy of
    // A when the weights carry column fields); 2^(ga - gq): undo the input
    // guard, apply the panel's
    {
        enc_gemm_desc g{};
        g.path = L.path;
        g.x = ain;
        g.y = b.panel;
        g.w[0] = L.wq; g.w[1] = L.wk; g.w[2] = L.wv;
        g.row_scale[0] = L.sq; g.row_scale[1] = L.sk; g.row_scale[2] = L.sv;
        g.bias[0] = L.bq; g.bias[1] = L.bk; g.bias[2] = L.bv;
        g.alpha = p2(ga - gq);
        g.flags = i8 ? ENC_Y_F16 : 0;
        const uint64_t xs = nout_attn(L) > 1 ? rd : 0;
        enc_gemm_item it[3] = {{rows, qw, d, d, ld, 0, 0, 0},
                               {rows, kw, d, d, ld, 1, xs, qw},
                               {rows, kw, d, d, ld, 2, 2 * xs, qw + kw}};
        TRY(run_gemm(&g, it, 3, s));
    }
    if (amax) TRY(amax_site(b.panel, (uint64_t)rows * ld, b.amax, amax + 1, s));
    if (sandwich) {
        // the panel holds x 2^-gq: eps 2^-2gq gives the norm of x exactly
        QkArgs q{b.panel, rows, ld, 0, qw, L.nq, L.nkv, hd, L.rope_sections, L.q_norm_w, L.k_norm_w,
                 L.eps * p2(-2 * gq), B->rope_cos[L.rope_table], B->rope_sin[L.rope_table], qw + kw,
                 L.v_norm};
        TRY(rows_qk(q, i8, s));
    }
    {
        // v carried 2^-gq; the O projection reads att col_o 2^-gao
        enc_attn_desc a = layer_attn_desc(L, rows);
        a.qkv = b.panel;
        a.out = b.att;
        a.ws = b.part;
        a.ws_bytes = b.part_bytes;
        a.out_col = L.col_o;
        a.out_scale = p2(gq - gao);
        TRY(run_attention(&a, B->items, B->nitems, s));
    }
    if (amax) TRY(amax_site(b.att, (uint64_t)rows * qw, b.amax, amax + 2, s));
    // output projection: sandwich -> T; pre-LN -> h += att Wo^T + bo
    {
        enc_gemm_desc g{};
        g.path = L.path;
        g.x = b.att;
        g.y = sandwich ? (void *)b.t : (void *)h;
        g.w[0] = L.wo;
        g.row_scale[0] = L.so;
        g.bias[0] = L.bo;
        g.alpha = p2(gao);
        g.flags = sandwich ? 0 : ENC_Y_ACCUMULATE;
        enc_gemm_item it{rows, d, qw, qw, d, 0, 0, 0};
        TRY(run_gemm(&g, &it, 1, s));
    }
    if (sandwich) {
        TRY(row_op(L, rows, h, b.t, L.post_attn_w, L.mod_g_attn, 1.0f, ff_in(L), b.a, i8, s));
    } else {
        NormArgs n{rows, d, d, d, h, L.norm2_w, L.norm2_b, L.eps, b.a};
        TRY(rows_ln(n, false, s));
    }
    if (amax) TRY(amax_site(b.a, rd * nout_ff(L), b.amax, amax + 3, s));
    // MLP; gate/up times 2^gf (the input guard); the hidden stores
    // act(gate) up col_down 2^-gh for the down projection
    if (L.mlp == ENC_MLP_GELU_TANH) {
        enc_gemm_desc g{};
        g.path = L.path;
        g.x = b.a;
        g.y = b.m;
        g.w[0] = L.w_up;
        g.row_scale[0] = L.s_up;
        g.bias[0] = L.b_up;
        g.alpha = 1.0f;
        g.flags = ENC_EPI_GELU_TANH;
        enc_gemm_item it{rows, L.ff, d, d, L.ff, 0, 0, 0};
        TRY(run_gemm(&g, &it, 1, s));
    } else if (!unfused_gate(L)) {
        // gate and up in one launch, act(gate) * up formed in the epilogue
        enc_gemm_desc g{};
        g.path = L.path;
        g.x = b.a;
        g.y = b.m;
        g.w[0] = L.w_gate; g.w[1] = L.w_up;
        g.row_scale[0] = L.s_gate; g.row_scale[1] = L.s_up;
        g.alpha = p2(gf);
        g.flags = (L.mlp == ENC_MLP_GELU_TANH_GATED ? ENC_EPI_GATE_GELU_TANH : ENC_EPI_GATE_SILU) |
                  (i8 ? ENC_Y_F16 : 0u);
        g.y_col = L.col_down;
        g.y_scale = p2(-gh);
        enc_gemm_item it{rows, L.ff, d, d, L.ff, 0, 0, 0};
        TRY(run_gemm(&g, &it, 1, s));
    } else {
        // gate and up read their own copies of A (column fields): z = 2 into
        // gate|up, then the gated activation
        enc_gemm_desc g{};
        g.path = L.path;
        g.x = b.a;
        g.y = b.gu;
        g.w[0] = L.w_gate; g.w[1] = L.w_up;
        g.row_scale[0] = L.s_gate; g.row_scale[1] = L.s_up;
        g.alpha = p2(gf);
        enc_gemm_item it[2] = {{rows, L.ff, d, d, 2 * L.ff, 0, 0, 0}, {rows, L.ff, d, d, 2 * L.ff, 1, rd, L.ff}};
        TRY(run_gemm(&g, it, 2, s));
        ActArgs act{L.mlp == ENC_MLP_GELU_TANH_GATED ? (uint32_t)ENC_ACT_GELU_TANH_GATED : (uint32_t)ENC_ACT_SWIGLU,
                    rows, L.ff, 2 * L.ff, 2 * L.ff, L.ff, b.gu, b.gu + L.ff, b.m, L.col_down, p2(-gh)};
        TRY(rows_act(act, i8, s));
    }
    if (amax) TRY(amax_site(b.m, (uint64_t)rows * L.ff, b.amax, amax + 4, s));
    {
        enc_gemm_desc g{};
        g.path = L.path;
        g.x = b.m;
        g.y = sandwich ? (void *)b.t : (void *)h;
        g.w[0] = L.w_down;
        g.row_scale[0] = L.s_down;
        g.bias[0] = L.b_down;
        g.alpha = p2(gh);
        g.flags = sandwich ? 0 : ENC_Y_ACCUMULATE;
        enc_gemm_item it{rows, d, L.ff, L.ff, d, 0, 0, 0};
        TRY(run_gemm(&g, &it, 1, s));
    }
    if (sandwich) {
        const float scalar = L.scalar == 0.0f ? 1.0f : L.scalar;
        if (!L.n_ple) {
            TRY(row_op(L, rows, h, b.t, L.post_ff_w, L.mod_g_ff, scalar, nx, aout, i8, s));
        } else {
            TRY(row_op(L, rows, h, b.t, L.post_ff_w, L.mod_g_ff, 1.0f, NextIn{}, nullptr, false, s));
            TRY(run_ple(L, rows, x0, h, b, s));
            TRY(row_op(L, rows, h, b.t, L.ple_post_w, nullptr, scalar, nx, aout, false, s));
        }
    }
    return hipSuccess;
}

// The layers of a model in place on h (every layer's last row op writes the
// next layer's inputs, or the fused final RMS).
hipError_t run_stack(const enc_model *model, const enc_batch *batch, const float *x0, float *h, const Bufs &b,
                     hipStream_t s) {
    const enc_layer &L0 = model->layers[0];
    if (L0.block == ENC_SANDWICH_RMS) TRY(pre_norm(L0, batch->rows, h, b.a, s));
    for (uint32_t l = 0; l < model->nlayers; l++) {
        NextIn nx;
        if (L0.block == ENC_SANDWICH_RMS) {
            if (l + 1 < model->nlayers)
                nx = attn_in(model->layers[l + 1]);
            else if (fused_final(model))
                nx.w = model->final_w;  // the final RMS (f32) written by the last row op
        }
        const void *ain = L0.block == ENC_SANDWICH_RMS ? b.a : nullptr;
        TRY(run_layer(model->layers[l], batch, x0, h, b, ain, b.a, nx, batch->amax ? batch->amax + 5 * l : nullptr,
                      s));
    }
    return hipSuccess;
}

// A staged program: every stage valid, in range, final NONE, one width.
enc_status check_stages(Err &e, const enc_stage *st, uint32_t n, uint32_t rows, WsPlan *most) {
    if (!st || !n) return e.set(ENC_EINVAL, "encoder_stages_forward: no stages");
    uint32_t d = 0;
    size_t total = 0;
    for (uint32_t i = 0; i < n; i++) {
        const enc_model *M = st[i].model;
        if (check_model(e, M, &st[i].batch) != ENC_OK) {
            const std::string m = e.msg;
            return e.set(e.st, "stage %u: %s", i, m.c_str());
        }
        if (!M->nlayers) return e.set(ENC_EINVAL, "stage %u: no layers", i);
        if (M->final_kind != ENC_FINAL_NONE)
            return e.set(ENC_EUNSUPPORTED, "stage %u: a stage's final must be NONE", i);
        if ((uint64_t)st[i].row0 + st[i].batch.rows > rows)
            return e.set(ENC_EINVAL, "stage %u: rows [%u, %u) past the program's %u", i, st[i].row0,
                         st[i].row0 + st[i].batch.rows, rows);
        if (i && M->layers[0].d != d) return e.set(ENC_ESHAPE, "stage %u: width differs", i);
        d = M->layers[0].d;
        const WsPlan p = plan_ws(M, &st[i].batch);
        if (p.total > total) {
            total = p.total;
            *most = p;
        }
    }
    return ENC_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

enc_status enc_create(int device, enc_ctx **out) {
    if (!out) return ENC_EINVAL;
    *out = nullptr;
    hipDeviceProp_t p;
    hipError_t h = hipGetDeviceProperties(&p, device);
    if (h != hipSuccess) {
        g_create_err = std::string("enc_create: ") + hipGetErrorString(h);
        return ENC_EDEVICE;
    }
    if (!strstr(p.gcnArchName, "gfx950")) {
        g_create_err = std::string("enc_create: device is ") + p.gcnArchName + ", the kernels are gfx950";
        return ENC_EUNSUPPORTED;
    }
    enc_ctx *c = new enc_ctx;
    c->device = device;
    // this device's copy of the static scratch, taken with the device current
    int cur = 0;
    h = hipGetDevice(&cur);
    if (h == hipSuccess) h = hipSetDevice(device);
    if (h == hipSuccess) {
        void *ptr = nullptr;
        h = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (h == hipSuccess) c->scratch = ptr;
        const hipError_t back = hipSetDevice(cur);
        if (h == hipSuccess) h = back;
    }
    if (h != hipSuccess) {
        c->scratch = nullptr;
        c->scratch_err = std::string("static scratch unavailable: ") + hipGetErrorString(h);
    }
    *out = c;
    g_create_err.clear();
    return ENC_OK;
}

void enc_destroy(enc_ctx *ctx) {
    if (!ctx) return;
    for (auto &p : ctx->pool) {
        (void)hipEventDestroy(p.first);
        (void)hipEventDestroy(p.second);
    }
    delete ctx;
}

enc_status enc_prof_enable(enc_ctx *ctx, int on) {
    if (!ctx) return ENC_EINVAL;
    ctx->prof = on != 0;
    ctx->err.clear();
    return ENC_OK;
}

enc_status enc_prof_read(enc_ctx *ctx, enc_prof_stat *stats) {
    if (!ctx || !stats) return ENC_EINVAL;
    Err e;
    for (int c = 0; c < ENC_NCLASS; c++) stats[c] = enc_prof_stat{0, 0.0, 0.0, 0.0};
    for (const ProfRec &r : ctx->recs) {
        const auto &ev = ctx->pool[r.ev];
        float ms = 0.0f;
        hipError_t h = hipEventSynchronize(ev.second);
        if (h == hipSuccess) h = hipEventElapsedTime(&ms, ev.first, ev.second);
        if (h != hipSuccess) {
            e.set(ENC_EDEVICE, "enc_prof_read: %s", hipGetErrorString(h));
            break;
        }
        enc_prof_stat &st = stats[r.cls];
        st.launches++;
        st.ms += ms;
        st.flops += r.flops;
        st.bytes += r.bytes;
    }
    ctx->recs.clear();
    return finish(ctx, e);
}

const char *enc_last_error(const enc_ctx *ctx) { return ctx ? ctx->err.c_str() : g_create_err.c_str(); }

enc_status enc_check_gemm(const enc_gemm_desc *desc, const enc_gemm_item *items, uint32_t nitems,
                          char *msg, size_t msg_len) {
    Err e;
    check_gemm(e, desc, items, nitems);
    copy_msg(e, msg, msg_len);
    return e.st;
}

enc_status enc_check_attention(const enc_attn_desc *desc, const enc_item *items, uint32_t nitems,
                               char *msg, size_t msg_len) {
    Err e;
    check_attn(e, desc, items, nitems);
    copy_msg(e, msg, msg_len);
    return e.st;
}

enc_status enc_check_model(const enc_model *model, const enc_batch *batch, char *msg, size_t msg_len) {
    Err e;
    check_model(e, model, batch);
    copy_msg(e, msg, msg_len);
    return e.st;
}

enc_status enc_validate_model(const enc_model *model, const enc_batch *batch) {
    return enc_check_model(model, batch, nullptr, 0);
}

enc_status gemm_items(enc_ctx *ctx, const enc_gemm_desc *desc, const enc_gemm_item *items,
                      uint32_t nitems, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (check_gemm(e, desc, items, nitems) == ENC_OK)
        launch_status(e, run_gemm(desc, items, nitems, (hipStream_t)stream), "gemm_items");
    return finish(ctx, e);
}

enc_status attention_items(enc_ctx *ctx, const enc_attn_desc *desc, const enc_item *items,
                           uint32_t nitems, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (check_attn(e, desc, items, nitems) == ENC_OK)
        launch_status(e, run_attention(desc, items, nitems, (hipStream_t)stream), "attention_items");
    return finish(ctx, e);
}

enc_status attention_items_static(enc_ctx *ctx, const enc_attn_desc *desc, const enc_item *items,
                                  uint32_t nitems, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (!desc) {
        e.set(ENC_EINVAL, "attention_items_static: null descriptor");
        return finish(ctx, e);
    }
    if (desc->ws || desc->ws_bytes) {
        e.set(ENC_EINVAL, "attention_items_static: ws must be NULL (the call uses the library's static scratch)");
        return finish(ctx, e);
    }
    if (!ctx->scratch) {
        e.set(ENC_EDEVICE, "attention_items_static: %s", ctx->scratch_err.c_str());
        return finish(ctx, e);
    }
    enc_attn_desc d = *desc;
    d.ws = ctx->scratch;
    d.ws_bytes = ENC_STATIC_SCRATCH_BYTES;
    // the needed size first, so that the error names it rather than the
    // workspace check's generic message
    if (items || !nitems) {
        const size_t need = attn_ws_bytes(&d, items, nitems);
        if (need > ENC_STATIC_SCRATCH_BYTES) {
            e.set(ENC_EUNSUPPORTED,
                  "attention_items_static: the key splits of these items need %zu bytes of scratch, "
                  "the static scratch holds %zu (use attention_items with a workspace)",
                  need, (size_t)ENC_STATIC_SCRATCH_BYTES);
            return finish(ctx, e);
        }
    }
    if (check_attn(e, &d, items, nitems) == ENC_OK)
        launch_status(e, run_attention(&d, items, nitems, (hipStream_t)stream), "attention_items_static");
    return finish(ctx, e);
}

enc_status enc_rms_norm(enc_ctx *ctx, const enc_norm_desc *d, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (check_norm(e, "enc_rms_norm", d) == ENC_OK) {
        NormArgs n{d->rows, d->d, d->ldx, d->ldy, d->x, d->w, nullptr, d->eps, d->y,
                   d->pre == 0.0f ? 1.0f : d->pre};
        launch_status(e, rows_rms(n, d->flags & ENC_Y_F16, (hipStream_t)stream), "enc_rms_norm");
    }
    return finish(ctx, e);
}

enc_status enc_layer_norm(enc_ctx *ctx, const enc_norm_desc *d, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (check_norm(e, "enc_layer_norm", d) == ENC_OK) {
        NormArgs n{d->rows, d->d, d->ldx, d->ldy, d->x, d->w, d->b, d->eps, d->y};
        launch_status(e, rows_ln(n, d->flags & ENC_Y_F16, (hipStream_t)stream), "enc_layer_norm");
    }
    return finish(ctx, e);
}

enc_status enc_add_norm(enc_ctx *ctx, const enc_add_norm_desc *d, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (check_add_norm(e, d) == ENC_OK) {
        AddNormArgs a{d->rows, d->d, d->h, d->t, d->w_post, d->w_next, d->eps, d->a,
                      d->post == 0.0f ? 1.0f : d->post};
        a.gate = d->gate;
        a.scale = d->scale;
        for (int z = 0; z < 3; z++) a.col[z] = d->col[z];
        a.nout = d->nout ? d->nout : 1;
        a.oscale = d->oscale == 0.0f ? 1.0f : d->oscale;
        a.a_stride = (uint64_t)d->rows * d->d;
        launch_status(e, rows_add_norm(a, d->flags & ENC_Y_F16, (hipStream_t)stream), "enc_add_norm");
    }
    return finish(ctx, e);
}

enc_status enc_qk_norm_rope(enc_ctx *ctx, const enc_qk_desc *d, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (check_qk(e, d) == ENC_OK) {
        QkArgs q{d->panel, d->rows, d->ld, d->q_col, d->k_col, d->nq, d->nkv, d->hd, d->sections,
                 d->q_norm_w, d->k_norm_w, d->eps, d->cos, d->sin, d->v_col, d->v_norm ? 1u : 0u};
        launch_status(e, rows_qk(q, d->path == ENC_I8F16, (hipStream_t)stream), "enc_qk_norm_rope");
    }
    return finish(ctx, e);
}

enc_status enc_gated_act(enc_ctx *ctx, const enc_act_desc *d, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (check_act(e, d) == ENC_OK) {
        ActArgs a{d->kind, d->rows, d->ff, d->ldg, d->ldu, d->ldo, d->g, d->u, d->out, d->out_col,
                  d->out_scale == 0.0f ? 1.0f : d->out_scale};
        launch_status(e, rows_act(a, d->flags & ENC_Y_F16, (hipStream_t)stream), "enc_gated_act");
    }
    return finish(ctx, e);
}

enc_status enc_mean_pool(enc_ctx *ctx, uint32_t rows, uint32_t d, const float *a, const enc_item *items,
                         uint32_t nitems, float *out, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (!a || !out) {
        e.set(ENC_EINVAL, "enc_mean_pool: null pointer");
    } else if (check_items(e, "enc_mean_pool", items, nitems, rows) == ENC_OK) {
        for (uint32_t i = 0; i < nitems; i++)
            if (!item_len(items[i])) {
                e.set(ENC_EINVAL, "enc_mean_pool: item %u is empty (its mean is undefined)", i);
                return finish(ctx, e);
            }
        launch_status(e, pool_items(items, nitems, rows, d, a, out, (hipStream_t)stream), "enc_mean_pool");
    }
    return finish(ctx, e);
}

enc_status enc_mfma_peak(enc_ctx *ctx, uint32_t path, uint32_t blocks, uint32_t iters, float *out,
                         double *flops, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    if (!out || !flops || !blocks || path > 1) {
        e.set(ENC_EINVAL, "enc_mfma_peak: null output or bad arguments");
        return finish(ctx, e);
    }
    const double per = path == ENC_I8F16 ? 32.0 * 32 * 16 * 2 : 32.0 * 32 * 2 * 2;
    *flops = (double)blocks * 4 * iters * 16 * per;
    launch_status(e, launch_mfma_peak(path == ENC_I8F16, blocks, iters, out, (hipStream_t)stream),
                  "enc_mfma_peak");
    return finish(ctx, e);
}

size_t enc_workspace_bytes(const enc_model *model, const enc_batch *batch) {
    if (!model || (model->nlayers && !model->layers) || !batch || (batch->nitems && !batch->items))
        return 0;
    return plan_ws(model, batch).total;
}

size_t enc_attention_workspace_bytes(const enc_attn_desc *desc, const enc_item *items, uint32_t nitems) {
    if (!desc || (nitems && !items)) return 0;
    return attn_ws_bytes(desc, items, nitems);
}

enc_status encoder_layer_forward(enc_ctx *ctx, const enc_layer *layer, const enc_layer *next,
                                 const enc_batch *batch, float *h, void *a, void *ws, size_t ws_bytes,
                                 enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (!layer || !h || !ws) {
        e.set(ENC_EINVAL, "encoder_layer_forward: null layer, h or workspace");
        return finish(ctx, e);
    }
    if (next && !a) {
        e.set(ENC_EINVAL, "encoder_layer_forward: the next layer's input needs a (the buffer it is written to)");
        return finish(ctx, e);
    }
    // the layer (and the next one, which must match its block kind, path and width)
    const enc_layer pair[2] = {*layer, next ? *next : *layer};
    enc_model M{next ? 2u : 1u, pair, ENC_FINAL_NONE, nullptr, nullptr, 0.0f};
    if (check_model(e, &M, batch) != ENC_OK) return finish(ctx, e);
    if (layer->n_ple && (!batch->ple_x || batch->ple_x == h)) {
        e.set(ENC_EINVAL, "encoder_layer_forward: the per-layer input needs batch ple_x (not h)");
        return finish(ctx, e);
    }
    const WsPlan p = plan_ws(&M, batch);
    if (ws_bytes < p.total || !aligned(ws, 256) || !aligned(h, 16) || (a && !aligned(a, 16))) {
        e.set(ENC_EINVAL, "encoder_layer_forward: workspace needs %zu bytes, 256-byte aligned (h, a 16-byte)",
              p.total);
        return finish(ctx, e);
    }
    const Bufs b = carve(ws, p);
    hipStream_t s = (hipStream_t)stream;
    hipError_t hr = hipSuccess;
    const bool sandwich = layer->block == ENC_SANDWICH_RMS;
    const void *ain = a;
    if (!ain && sandwich) {
        hr = pre_norm(*layer, batch->rows, h, b.a, s);
        ain = b.a;
    }
    const NextIn nx = next && sandwich ? attn_in(*next) : NextIn{};
    if (hr == hipSuccess) hr = run_layer(*layer, batch, batch->ple_x, h, b, ain, a, nx, batch->amax, s);
    // pre-LN: the next layer's LN1 of the updated rows
    if (hr == hipSuccess && next && !sandwich) hr = pre_norm(*next, batch->rows, h, a, s);
    launch_status(e, hr, "encoder_layer_forward");
    return finish(ctx, e);
}

enc_status encoder_forward(enc_ctx *ctx, const enc_model *model, const enc_batch *batch, const float *x,
                           float *out, void *ws, size_t ws_bytes, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (!x || !out || !ws) {
        e.set(ENC_EINVAL, "encoder_forward: null x, out or workspace");
        return finish(ctx, e);
    }
    if (check_model(e, model, batch) != ENC_OK) return finish(ctx, e);
    if (model->nlayers == 0) {
        e.set(ENC_EINVAL, "encoder_forward: no layers");
        return finish(ctx, e);
    }
    const WsPlan p = plan_ws(model, batch);
    if (ws_bytes < p.total || !aligned(ws, 256) || !aligned(x, 16) || !aligned(out, 16)) {
        e.set(ENC_EINVAL, "encoder_forward: workspace needs %zu bytes, 256-byte aligned", p.total);
        return finish(ctx, e);
    }
    const enc_layer &L0 = model->layers[0];
    const uint32_t rows = batch->rows, d = L0.d;
    const Bufs b = carve(ws, p);
    hipStream_t s = (hipStream_t)stream;
    float *h = model->final_kind == ENC_FINAL_NONE ? out : b.h;
    const float *x0 = batch->ple_x ? batch->ple_x : x;  // rows the per-layer inputs project
    bool ple = false;
    for (uint32_t l = 0; l < model->nlayers; l++) ple |= model->layers[l].n_ple != 0;
    if (ple && x0 == h) {
        e.set(ENC_EINVAL, "encoder_forward: the per-layer input reads x in every layer; out must not alias it");
        return finish(ctx, e);
    }
    hipError_t hr = hipSuccess;
    if (h != x) hr = hipMemcpyAsync(h, x, (size_t)rows * d * 4, hipMemcpyDeviceToDevice, s);
    if (hr == hipSuccess) hr = run_stack(model, batch, x0, h, b, s);
    if (hr == hipSuccess && model->final_kind == ENC_FINAL_LN) {
        NormArgs n{rows, d, d, d, h, model->final_w, model->final_b, model->final_eps, out};
        hr = rows_ln(n, false, s);
    } else if (hr == hipSuccess && model->final_kind == ENC_FINAL_RMS_MEANPOOL) {
        float *a = (float *)b.t;  // f32 rows of rms(H; final_w)
        if (fused_final(model)) {
            a = (float *)b.a;
        } else {
            NormArgs n{rows, d, d, d, h, model->final_w, nullptr, model->final_eps, a};
            hr = rows_rms(n, false, s);
        }
        if (hr == hipSuccess) hr = pool_items(batch->items, batch->nitems, rows, d, a, out, s);
    }
    launch_status(e, hr, "encoder_forward");
    return finish(ctx, e);
}

size_t enc_stages_workspace_bytes(const enc_stage *stages, uint32_t nstages) {
    size_t most = 0;
    if (!stages) return 0;
    for (uint32_t i = 0; i < nstages; i++) {
        const enc_model *M = stages[i].model;
        if (!M || (M->nlayers && !M->layers) || (stages[i].batch.nitems && !stages[i].batch.items)) return 0;
        most = std::max(most, plan_ws(M, &stages[i].batch).total);
    }
    return most;
}

enc_status encoder_stages_forward(enc_ctx *ctx, const enc_stage *stages, uint32_t nstages, uint32_t rows,
                                  const float *x, float *h, void *ws, size_t ws_bytes, enc_stream stream) {
    Err e;
    if (!ctx) return ENC_EINVAL;
    CtxScope cs(ctx);
    if (!x || !h || !ws) {
        e.set(ENC_EINVAL, "encoder_stages_forward: null x, h or workspace");
        return finish(ctx, e);
    }
    WsPlan p;
    if (check_stages(e, stages, nstages, rows, &p) != ENC_OK) return finish(ctx, e);
    if (ws_bytes < p.total || !aligned(ws, 256) || !aligned(x, 16) || !aligned(h, 16)) {
        e.set(ENC_EINVAL, "encoder_stages_forward: workspace needs %zu bytes, 256-byte aligned", p.total);
        return finish(ctx, e);
    }
    const uint32_t d = stages[0].model->layers[0].d;
    for (uint32_t i = 0; i < nstages; i++) {
        bool ple = false;
        for (uint32_t l = 0; l < stages[i].model->nlayers; l++) ple |= stages[i].model->layers[l].n_ple != 0;
        if (ple && (!stages[i].batch.ple_x || stages[i].batch.ple_x == h + (size_t)stages[i].row0 * d)) {
            e.set(ENC_EINVAL, "stage %u: a per-layer input needs its batch ple_x", i);
            return finish(ctx, e);
        }
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t hr = hipSuccess;
    if (h != x) hr = hipMemcpyAsync(h, x, (size_t)rows * d * 4, hipMemcpyDeviceToDevice, s);
    for (uint32_t i = 0; i < nstages && hr == hipSuccess; i++) {
        // each stage's buffers carved for its own batch (all fit the largest plan)
        const WsPlan sp = plan_ws(stages[i].model, &stages[i].batch);
        const Bufs b = carve(ws, sp);
        float *hs = h + (size_t)stages[i].row0 * d;
        hr = run_stack(stages[i].model, &stages[i].batch, stages[i].batch.ple_x, hs, b, s);
    }
    launch_status(e, hr, "encoder_stages_forward");
    return finish(ctx, e);
}

// ------------------------------------------------------------ host helpers

enc_status enc_positions(uint32_t rows, const enc_item *items, const uint32_t *grids, uint32_t nitems,
                         uint32_t sections, int32_t *pos) {
    if (!pos || (nitems && !items) || sections < 1 || sections > 2) return ENC_EINVAL;
    if (sections == 2 && !grids) return ENC_EINVAL;
    Err e;
    if (check_items(e, "enc_positions", items, nitems, rows) != ENC_OK) return e.st;
    for (uint32_t i = 0; i < nitems; i++) {
        const enc_item &it = items[i];
        const uint32_t L = item_len(it);
        const uint32_t G = sections == 2 ? grids[i] : 0;
        for (uint32_t t = 0; t < L; t++) {
            const uint32_t row = t < it.r[0].n ? it.r[0].r0 + t : it.r[1].r0 + (t - it.r[0].n);
            if (sections == 1) {
                pos[row] = (int32_t)t;
            } else if (t < G * G) {
                pos[2 * row] = (int32_t)(t % G);      // column
                pos[2 * row + 1] = (int32_t)(t / G);  // row
            } else if (t < it.r[0].n) {
                pos[2 * row] = pos[2 * row + 1] = 0;  // pad row of the image range
            } else {
                pos[2 * row] = pos[2 * row + 1] = (int32_t)(G + (t - it.r[0].n));  // caption
            }
        }
    }
    return ENC_OK;
}

enc_status enc_rope_table(uint32_t rows, uint32_t hd, uint32_t sections, const int32_t *pos, double base,
                          float *cos_out, float *sin_out) {
    if (!pos || !cos_out || !sin_out || sections < 1 || sections > 2 || hd == 0 || hd % (2 * sections))
        return ENC_EINVAL;
    const uint32_t S = hd / sections, half = S / 2;
    for (uint32_t r = 0; r < rows; r++)
        for (uint32_t s = 0; s < sections; s++)
            for (uint32_t i = 0; i < half; i++) {
                const double ang = (double)pos[(size_t)r * sections + s] * std::pow(base, -2.0 * i / S);
                cos_out[(size_t)r * (hd / 2) + s * half + i] = (float)std::cos(ang);
                sin_out[(size_t)r * (hd / 2) + s * half + i] = (float)std::sin(ang);
            }
    return ENC_OK;
}

}  // extern "C"
