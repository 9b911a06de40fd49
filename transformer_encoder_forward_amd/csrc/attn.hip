// Launchers of the flash attention.
//
// f16 path (attn_impl.h): hd 128 without a window in attn_f16s_kernel
// (software-pipelined, K/V by direct global -> LDS loads), with a window in
// attn_f16d_kernel, hd 64 in the attn_kernel template.
// f32 path: the kernel below, the same S^T = K Q^T / O^T = V^T P^T scheme in its
// plain form: with 64-cycle FP32 MFMAs the softmax VALU work is hidden anyway,
// and the plain form keeps the register count low enough for three waves per
// SIMD.  V is staged transposed, so the P V operand comes in 16-byte reads;
// short windowless items are split over the keys (attn_combine_kernel merges).
// What both compute: egemma2.rs (cortiq-engine 0.8.39), module doc "Attention"
// and `att_plan`; zimage.rs (cortiq-engine 0.7.6), module doc and `PFa`.
#include <math.h>

#include <algorithm>

#include "attn_impl.h"

namespace enc {

namespace f32path {

constexpr int KB = 32;   // keys per block

struct ItemCtx {
    AttnItemK it;
    int L, q_lo, q_hi, k_lo, k_hi;
};

// Item, query range and key range of a block.  A key-split item's tiles are
// (q-tile, split) pairs, split fastest; split s sees keys [s*chunk, (s+1)*chunk).
template <int QT>
__device__ __forceinline__ void locate(const AttnArgs &a, uint32_t tile, ItemCtx &c, int &split) {
    uint32_t sel = 0;
    for (uint32_t i = 1; i < a.nitems; i++)
        if (tile >= a.items[i].tile0) sel = i;
    c.it = a.items[sel];
    c.L = (int)(c.it.na + c.it.nb);
    const uint32_t local = tile - c.it.tile0;
    split = (int)(local % c.it.nsplit);
    c.q_lo = (int)(local / c.it.nsplit) * QT;
    c.q_hi = min(c.q_lo + QT, c.L);
    c.k_lo = 0;
    c.k_hi = c.L;
    if (c.it.nsplit > 1) {
        c.k_lo = split * (int)c.it.chunk;
        c.k_hi = min(c.L, c.k_lo + (int)c.it.chunk);
    } else if (a.window) {
        c.k_lo = max(0, c.q_lo - (int)a.window);
        c.k_hi = min(c.L, c.q_hi + (int)a.window);
    }
}

__device__ __forceinline__ int row_of(const AttnItemK &it, int t) {
    return t < (int)it.na ? (int)it.r0a + t : (int)it.r0b + (t - (int)it.na);
}

// Does any (query, key) pair of queries [q0, q1) x keys [kb, kb + KB) pass the mask?
__device__ __forceinline__ bool block_active(int q0, int q1, int kb, int k_hi, uint32_t W) {
    if (q0 >= q1 || kb >= k_hi) return false;
    if (!W) return true;
    return kb <= q1 - 1 + (int)W && kb + KB - 1 >= q0 - (int)W;
}

// Column of the 16-byte group g (keys 4g..4g+3) in row `row` of the staged V^T:
// groups are XOR-swizzled by bits 4-6 of the row so that both the transposing
// 4-byte stores (16 rows x 4 keys per wave) and the 16-byte reads (consecutive
// rows, one group) spread over all banks.
__device__ __forceinline__ int vt_col(int row, int g) { return 4 * (g ^ ((row >> 4) & 7)); }

// Online-softmax update of one lane's 16 scores (query = lane%32).  sv holds
// scaled dot products; masked keys are -inf.  Returns p in place.  The running
// max moves, to this block's max, only when that passes it by more than 8 (log2
// units): p stays at most 256, the factor alpha is exactly 1 otherwise, and the
// quotient o / l does not depend on where m sits.  2^x is the bare v_exp_f32
// (results below 2^-126 flush to 0, far below anything a row sum of at least 1
// registers).
__device__ __forceinline__ float softmax_step(float (&sv)[16], float &m_run, float &l_run) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, sv[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = mx > m_run + 8.0f ? mx : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rs = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        sv[r] = __builtin_amdgcn_exp2f(sv[r] - m_use);
        rs += sv[r];
    }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    return alpha;
}

// ------------------------------------------------------------------ f32 path

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_f32_kernel(AttnArgs a) {
    constexpr int NT = 64 * NW, QT = 32 * NW;
    constexpr int LDK = HD + 4;
    constexpr int LDT = KB + 4;                // V^T rows: 32 keys + pad
    constexpr int NQ4 = HD / 8;                // float4 of q per lane (hd/2 floats)
    constexpr int NLD = KB * HD / 4 / NT;      // float4 of K (and of V) per thread per block
    __shared__ __attribute__((aligned(16))) float Ks[2][KB][LDK];
    __shared__ __attribute__((aligned(16))) float Vs[2][HD][LDT];  // V transposed

    const uint32_t head = blockIdx.x % a.nq, tile = blockIdx.x / a.nq;
    ItemCtx c;
    int split;
    locate<QT>(a, tile, c, split);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int kvh = head / a.group;
    const float *P = reinterpret_cast<const float *>(a.qkv);
    const uint32_t W = a.window;

    const int tq = c.q_lo + wave * 32 + li;
    const bool qvalid = tq < c.q_hi;
    const int wq0 = c.q_lo + wave * 32, wq1 = min(wq0 + 32, c.q_hi);
    // keys this lane's query sees: [vlo, vhi), empty for a padding lane
    const int vlo = W ? max(c.k_lo, tq - (int)W) : c.k_lo;
    const int vhi = !qvalid ? vlo : max(vlo, W ? min(c.k_hi, tq + (int)W + 1) : c.k_hi);

    // this lane's query, channels (hd/2)*hf .. +hd/2 (its half of the dot product)
    f32x4 qf[NQ4];
    {
        const float *qp = P + (size_t)row_of(c.it, qvalid ? tq : c.q_lo) * a.ld + a.q_col + head * HD +
                          (HD / 2) * hf;
#pragma unroll
        for (int j = 0; j < NQ4; j++) qf[j] = qvalid ? ld4(qp + 4 * j) : f32x4{0, 0, 0, 0};
    }

    f32x4 rk[NLD], rv[NLD];
    auto gload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int f = tid + NT * i, key = f / (HD / 4), ch = (f % (HD / 4)) * 4;
            const int t = kb + key;
            if (t < c.k_hi) {
                const float *base = P + (size_t)row_of(c.it, t) * a.ld + kvh * HD + ch;
                rk[i] = ld4(base + a.k_col);
                rv[i] = ld4(base + a.v_col);
            } else {
                rk[i] = f32x4{0, 0, 0, 0};
                rv[i] = f32x4{0, 0, 0, 0};
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int f = tid + NT * i, key = f / (HD / 4), ch = (f % (HD / 4)) * 4;
            st4(&Ks[buf][key][ch], rk[i]);
#pragma unroll
            for (int e = 0; e < 4; e++) Vs[buf][ch + e][vt_col(ch + e, key >> 2) + (key & 3)] = rv[i][e];
        }
    };

    f32x16 o[HD / 32];
#pragma unroll
    for (int b = 0; b < HD / 32; b++)
#pragma unroll
        for (int r = 0; r < 16; r++) o[b][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const int nblk = (c.k_hi - c.k_lo + KB - 1) / KB;
    if (nblk > 0) {
        gload(c.k_lo);
        sstore(0);
    }
    __syncthreads();
    for (int b = 0; b < nblk; b++) {
        const int kb = c.k_lo + b * KB, buf = b & 1;
        if (b + 1 < nblk) gload(kb + KB);
        if (block_active(wq0, wq1, kb, c.k_hi, W)) {
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; r++) s[r] = 0.0f;
            const float *kr = &Ks[buf][li][(HD / 2) * hf];
            f32x4 kf[NQ4];
#pragma unroll
            for (int j = 0; j < NQ4; j++) kf[j] = ld4(kr + 4 * j);
#pragma unroll
            for (int j = 0; j < NQ4; j++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[j][e], qf[j][e], s, 0, 0, 0);
            // every pair of the wave x block visible: all 32 queries valid, all
            // keys inside the range and inside every query's window
            const bool full = wq1 - wq0 == 32 && kb + KB <= c.k_hi &&
                              (!W || (wq1 - 1 - kb <= (int)W && kb + KB - 1 - wq0 <= (int)W));
            float sv[16];
            if (full) {
#pragma unroll
                for (int r = 0; r < 16; r++) sv[r] = s[r] * a.scale_log2;
            } else {
                // key kb + off(r) is visible iff it lies in [vlo, vhi)
                const uint32_t base = (uint32_t)(kb + 4 * hf - vlo), span = (uint32_t)(vhi - vlo);
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const bool vis = base + (uint32_t)(8 * (r >> 2) + (r & 3)) < span;
                    sv[r] = vis ? s[r] * a.scale_log2 : -INFINITY;
                }
            }
            const float m_old = m_run;
            const float alpha = softmax_step(sv, m_run, l_run);
            // o is rescaled only when some query's max moved (else alpha is 1)
            if (__any(m_run != m_old)) {
#pragma unroll
                for (int d = 0; d < HD / 32; d++)
#pragma unroll
                    for (int r = 0; r < 16; r++) o[d][r] *= alpha;
            }
            // O^T[d][q] += V^T[d][key] P^T[key][q]; step r pairs lane halves'
            // keys 8(r/4) + 4 hf + r%4, so the keys of steps 4g..4g+3 are four
            // consecutive floats of a V^T row: one 16-byte read per 4 MFMAs
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++)
#pragma unroll
                for (int d = 0; d < HD / 32; d++) {
                    const f32x4 v4 = ld4(&Vs[buf][32 * d + li][vt_col(32 * d + li, 2 * g4 + hf)]);
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(v4[e], sv[4 * g4 + e], o[d], 0, 0, 0);
                }
        }
        if (b + 1 < nblk) sstore(buf ^ 1);
        __syncthreads();
    }
    if (!qvalid) return;
    if (c.it.nsplit > 1) {
        // partial result of this key split: unnormalised O, running max and sum
        const size_t rec = c.it.part0 + ((size_t)split * c.L + tq) * a.nq + head;
        float *po = a.part_o + rec * HD;
#pragma unroll
        for (int d = 0; d < HD / 32; d++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                f32x4 v = {o[d][4 * q], o[d][4 * q + 1], o[d][4 * q + 2], o[d][4 * q + 3]};
                st4(po + 32 * d + 8 * q + 4 * hf, v);
            }
        if (hf == 0) {
            a.part_ml[2 * rec] = m_run;
            a.part_ml[2 * rec + 1] = l_run;
        }
        return;
    }
    const float inv = 1.0f / l_run;
    float *out = reinterpret_cast<float *>(a.out) + (size_t)row_of(c.it, tq) * a.ldo + head * HD;
#pragma unroll
    for (int d = 0; d < HD / 32; d++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int ch = 32 * d + 8 * q + 4 * hf;
            f32x4 v = {o[d][4 * q] * inv, o[d][4 * q + 1] * inv, o[d][4 * q + 2] * inv,
                       o[d][4 * q + 3] * inv};
            st4(out + ch, out_scale(a, head * HD + ch, v));
        }
}

// Merge of the key splits: for item row t and head h with partials
// (o_s, m_s, l_s), s = 0..S-1 in increasing order,
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
// the same softmax as one pass over all keys.  A thread owns 4 channels of one
// (row, head); the order over s is fixed, so the result is deterministic.
template <bool F16>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineArgs a) {
    const uint32_t c4 = a.hd / 4;
    const uint64_t total = (uint64_t)a.row0[a.nitems] * a.nq * c4;
    for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t ch = (uint32_t)(g % c4);
        const uint64_t rh = g / c4;
        const uint32_t head = (uint32_t)(rh % a.nq), rt = (uint32_t)(rh / a.nq);
        uint32_t sel = 0;
        for (uint32_t i = 1; i < a.nitems; i++)
            if (rt >= a.row0[i]) sel = i;
        const AttnItemK &it = a.items[sel];
        const uint32_t t = rt - a.row0[sel], L = it.na + it.nb, S = it.nsplit;
        float M = -INFINITY;
        for (uint32_t s = 0; s < S; s++)
            M = fmaxf(M, a.part_ml[2 * (it.part0 + ((size_t)s * L + t) * a.nq + head)]);
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float lsum = 0.0f;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (uint32_t s = 0; s < S; s++) {
            const size_t rec = it.part0 + ((size_t)s * L + t) * a.nq + head;
            const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * rec] - Mu);
            lsum += w * a.part_ml[2 * rec + 1];
            const f32x4 v = ld4(a.part_o + rec * a.hd + 4 * ch);
#pragma unroll
            for (int e = 0; e < 4; e++) acc[e] += w * v[e];
        }
        const float inv = 1.0f / lsum;
#pragma unroll
        for (int e = 0; e < 4; e++) acc[e] *= inv;
        if (a.ocol) {
            const f32x4 m = ld4(a.ocol + head * a.hd + 4 * ch);
#pragma unroll
            for (int e = 0; e < 4; e++) acc[e] *= m[e];
        }
#pragma unroll
        for (int e = 0; e < 4; e++) acc[e] *= a.oscale;
        const size_t off = (size_t)row_of(it, (int)t) * a.ldo + head * a.hd + 4 * ch;
        if (F16)
            st4h(reinterpret_cast<_Float16 *>(a.out) + off, acc);
        else
            st4(reinterpret_cast<float *>(a.out) + off, acc);
    }
}

}  // namespace f32path

template <int HD, int NW>
hipError_t launch_f32(AttnArgs a, hipStream_t s) {
    const uint32_t tiles = attn::plan_tiles(a, 32 * NW);
    if (!tiles) return hipSuccess;
    hipLaunchKernelGGL((f32path::attn_f32_kernel<HD, NW>), dim3(tiles * a.nq), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// 128 queries per block (four waves; blocks of one wave were measured slower
// even where 128-query blocks leave CUs idle).
hipError_t launch_attn_f32(const AttnArgs &a, uint32_t hd, hipStream_t s) {
    if (hd == 64) return launch_f32<64, 4>(a, s);
    return launch_f32<128, 4>(a, s);
}

hipError_t launch_attn_combine(const CombineArgs &a, bool f16_out, hipStream_t s) {
    const uint64_t total = (uint64_t)a.row0[a.nitems] * a.nq * (a.hd / 4);
    if (!total) return hipSuccess;
    const uint32_t blocks = (uint32_t)std::min<uint64_t>((total + 255) / 256, 8192);
    if (f16_out)
        hipLaunchKernelGGL(f32path::attn_combine_kernel<true>, dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(f32path::attn_combine_kernel<false>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// hd 128 takes the direct-to-LDS kernels.  With a window, a block's first key
// depends on its query tile, so the tile size must not change between launches
// of the same item: always 128 queries.  Without one, an item whose 64-query
// blocks times heads number at most 512 (alone, it would fill one round of two
// such blocks per CU of a 256-CU device: up to 1088 rows at 30 heads) takes
// the kernel that splits each query's keys two ways inside the block.  The
// choice follows the item alone (its length and head count; a launch with both
// kinds of item is issued as two), so an item's bits never depend on the batch.
// Longer items take the pipelined kernel, in blocks of 256 queries (8 waves,
// one block per CU, each K/V block staged once for twice the queries) when the
// launch still has two such blocks per CU, else 128, which sum each query's
// keys in the same order.
// Measured per launch at 30 heads: one 1056-row item 39.3 -> 30.4 us split;
// a 1536-row item (720 blocks, not split) 62.6 unsplit against 64.4 split; two
// 960-row items are split (450 blocks each) and run 46.2 -> 51.6 us: unsplit
// their 480 blocks of 128 queries already give each SIMD two waves.
constexpr uint32_t kSplitBlocks = 512;

static bool f16_split_item(const AttnItemK &it, uint32_t nq) {
    return (uint64_t)((it.na + it.nb + 63) / 64) * nq <= kSplitBlocks;
}

hipError_t launch_attn_f16(const AttnArgs &a, uint32_t hd, hipStream_t s) {
    if (hd == 64) return attn::launch<64, true, 4, 4, true>(a, s);
    if (a.window) return attn::launch_f16d<4, 2>(a, s);
    AttnArgs sp = a, lo = a;
    sp.nitems = lo.nitems = 0;
    for (uint32_t i = 0; i < a.nitems; i++) {
        if (f16_split_item(a.items[i], a.nq))
            sp.items[sp.nitems++] = a.items[i];
        else
            lo.items[lo.nitems++] = a.items[i];
    }
    if (sp.nitems) {
        const hipError_t h = attn::launch_f16k(sp, s);
        if (h != hipSuccess || !lo.nitems) return h;
    }
    if (!lo.nitems) return hipSuccess;
    uint32_t t256 = 0;
    for (uint32_t i = 0; i < lo.nitems; i++) t256 += (lo.items[i].na + lo.items[i].nb + 255) / 256;
    if (t256 * lo.nq >= 512) return attn::launch_f16s<8, 1>(lo, s);
    return attn::launch_f16s<4, 2>(lo, s);
}

}  // namespace enc
