// Non-causal flash attention over packed items on gfx950 MFMA: the kernel
// template (attn.hip picks the instantiation).
//
// What it computes: egemma2.rs (cortiq-engine 0.8.39), module doc "Attention"
// and `att_plan` (bidirectional window: keys [q0 - W, q_last + W] clipped to
// the sequence; GQA head map h / (nq / nkv)), and the staged flash of
// `VisionGpu::forward`; zimage.rs (cortiq-engine 0.7.6), module doc (flash with
// K/V blocks staged in threadgroup memory; an item = its image range plus its
// caption range, `PFa`).  Online softmax: no score matrix is written.
//
// Design for CDNA4: a block of NW waves takes 32*NW queries of one item and
// one head; each wave owns 32 queries.  Per 32-key block the wave computes the
// TRANSPOSED scores S^T = K Q^T with 32x32 MFMAs, so lane l holds query l%32
// and 16 of the block's keys: the row max and row sum are 16 lane-local steps
// plus one exchange with lane l^32, and P^T is already in the B-operand layout
// of O^T = V^T P^T.  K/V blocks are staged in LDS (double-buffered through
// registers in the template below, rings of direct global -> LDS loads in
// attn_f16d_kernel, attn_f16s_kernel and attn_f16k_kernel) and shared by the
// block's waves (attn_f16k_kernel: by the two waves of each key half).  VALU
// work per score is kept small: blocks that lie wholly inside every query's
// window skip the mask, and the running output is rescaled only when the
// running max moves (otherwise the factor is exactly 1).  Waves whose queries
// see none of a block skip it.  The softmax runs in base 2 with log2(e) folded
// into the scale.
//  - f32 path: v_mfma_f32_32x32x2_f32 for both products.
//  - f16 path: v_mfma_f32_32x32x16_f16; V is staged transposed in LDS as key
//    pairs (one 32-bit write per channel and pair), so the A operand of O^T is
//    two 8-byte reads; P is rounded to f16 for P V, the softmax stays f32.
#pragma once
#include <math.h>

#include <type_traits>

#include "dev.h"
#include "kern.h"

namespace enc {

// The attention epilogue's output scale: out[c] = o[c] * oscale * ocol[c] for
// the four channels c0.. (ocol nullable).  With oscale 1 and no ocol the value
// is unchanged, bit for bit.
__device__ __forceinline__ f32x4 out_scale(const AttnArgs &a, int c0, f32x4 v) {
    if (a.ocol) {
        const f32x4 m = ld4(a.ocol + c0);
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] *= m[e];
    }
#pragma unroll
    for (int e = 0; e < 4; e++) v[e] *= a.oscale;
    return v;
}

namespace attn {

constexpr int KB = 32;  // keys per block

struct ItemCtx {
    AttnItemK it;
    int L, q_lo, q_hi, k_lo, k_hi;
};

template <int QT>
__device__ __forceinline__ void locate(const AttnArgs &a, uint32_t tile, ItemCtx &c) {
    uint32_t sel = 0;
    for (uint32_t i = 1; i < a.nitems; i++)
        if (tile >= a.items[i].tile0) sel = i;
    c.it = a.items[sel];
    c.L = (int)(c.it.na + c.it.nb);
    c.q_lo = (int)(tile - c.it.tile0) * QT;
    c.q_hi = min(c.q_lo + QT, c.L);
    c.k_lo = 0;
    c.k_hi = c.L;
    if (a.window) {
        c.k_lo = max(0, c.q_lo - (int)a.window);
        c.k_hi = min(c.L, c.q_hi + (int)a.window);
    }
}

__device__ __forceinline__ int row_of(const AttnItemK &it, int t) {
    return t < (int)it.na ? (int)it.r0a + t : (int)it.r0b + (t - (int)it.na);
}

// OPT: the mask fast path and the lazy rescale (they pay off where the VALU
// competes with fast FP16 MFMAs; with FP32 MFMAs they only cost registers).
template <int HD, bool F16, int NW, int MINW, bool OPT>
__global__ __launch_bounds__(64 * NW, MINW) void attn_kernel(AttnArgs a) {
    using T = typename std::conditional<F16, _Float16, float>::type;
    constexpr int QT = 32 * NW, NT = 64 * NW;
    constexpr int CE = F16 ? 8 : 4;              // elements per 16-byte chunk
    constexpr int LDK = HD + CE;                 // K rows (elements)
    // f16: V^T rows of KB/2 key pairs (u32), stride 18 words so that the four
    // channel groups one staging instruction writes land on distinct banks; f32: V rows
    constexpr int LDV = F16 ? KB / 2 + 2 : HD + 8;
    constexpr int KU = KB * HD / CE;                            // K chunks per block
    constexpr int VU = F16 ? (KB / 2) * (HD / 8) : KB * HD / CE;  // V units per block
    constexpr int NKC = (KU + NT - 1) / NT, NVC = (VU + NT - 1) / NT;  // per thread
    __shared__ __attribute__((aligned(16))) T Ks[2][KB][LDK];
    using VS = typename std::conditional<F16, uint32_t, float>::type;
    __shared__ __attribute__((aligned(16))) VS Vs[2][F16 ? HD : KB][LDV];

    const uint32_t head = blockIdx.x % a.nq, tile = blockIdx.x / a.nq;
    ItemCtx c;
    locate<QT>(a, tile, c);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int kvh = head / a.group;
    const T *P = reinterpret_cast<const T *>(a.qkv);
    const int W = (int)a.window;

    const int tq = c.q_lo + wave * 32 + li;
    const bool qvalid = tq < c.q_hi;
    const int wq0 = c.q_lo + wave * 32, wq1 = min(wq0 + 32, c.q_hi);

    // this lane's query, channels (hd/2)*hf .. +hd/2 (its half of each dot product)
    using QF = typename std::conditional<F16, f16x8, f32x4>::type;
    constexpr int NQ = HD / 2 / CE;
    QF qf[NQ];
    {
        const T *qp = P + (size_t)row_of(c.it, qvalid ? tq : c.q_lo) * a.ld + a.q_col + head * HD + (HD / 2) * hf;
#pragma unroll
        for (int j = 0; j < NQ; j++) qf[j] = qvalid ? *reinterpret_cast<const QF *>(qp + CE * j) : QF{};
    }

    QF rk[NKC];
    QF rv[F16 ? 2 * NVC : NVC];
    auto gload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < NKC; i++) {
            const int f = tid + NT * i, key = f / (HD / CE), ch = (f % (HD / CE)) * CE;
            const int t = kb + key;
            rk[i] = (f < KU && t < c.k_hi) ? *reinterpret_cast<const QF *>(P + (size_t)row_of(c.it, t) * a.ld + a.k_col +
                                                               kvh * HD + ch)
                               : QF{};
        }
        if constexpr (F16) {
            // unit = (key pair p, 8 channels ch..ch+7): rows 2p and 2p+1;
            // consecutive lanes take consecutive pairs
#pragma unroll
            for (int i = 0; i < NVC; i++) {
                const int f = tid + NT * i, p = f % (KB / 2), ch = (f / (KB / 2)) * 8;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int t = kb + 2 * p + h;
                    rv[2 * i + h] = (f < VU && t < c.k_hi) ? *reinterpret_cast<const QF *>(P + (size_t)row_of(c.it, t) * a.ld +
                                                                               a.v_col + kvh * HD + ch)
                                               : QF{};
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NVC; i++) {
                const int f = tid + NT * i, key = f / (HD / CE), ch = (f % (HD / CE)) * CE;
                const int t = kb + key;
                rv[i] = (f < VU && t < c.k_hi) ? *reinterpret_cast<const QF *>(P + (size_t)row_of(c.it, t) * a.ld + a.v_col +
                                                                   kvh * HD + ch)
                                   : QF{};
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NKC; i++) {
            const int f = tid + NT * i, key = f / (HD / CE), ch = (f % (HD / CE)) * CE;
            if (f < KU) *reinterpret_cast<QF *>(&Ks[buf][key][ch]) = rk[i];
        }
        if constexpr (F16) {
#pragma unroll
            for (int i = 0; i < NVC; i++) {
                const int f = tid + NT * i, p = f % (KB / 2), ch = (f / (KB / 2)) * 8;
                if (f < VU) {
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const f16x2 pr = {rv[2 * i][e], rv[2 * i + 1][e]};
                        Vs[buf][ch + e][p] = __builtin_bit_cast(uint32_t, pr);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NVC; i++) {
                const int f = tid + NT * i, key = f / (HD / CE), ch = (f % (HD / CE)) * CE;
                if (f < VU) *reinterpret_cast<f32x4 *>(&Vs[buf][key][ch]) = rv[i];
            }
        }
    };

    f32x16 o[HD / 32];
#pragma unroll
    for (int d = 0; d < HD / 32; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) o[d][r] = 0.0f;
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
        // does any (query, key) pair of this wave x block pass the mask?
        const bool active = wq0 < wq1 && kb < c.k_hi &&
                            (!W || (kb <= wq1 - 1 + W && kb + KB - 1 >= wq0 - W));
        if (active) {
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; r++) s[r] = 0.0f;
            const T *kr = &Ks[buf][li][(HD / 2) * hf];
#pragma unroll
            for (int j = 0; j < NQ; j++) {
                const QF kf = *reinterpret_cast<const QF *>(kr + CE * j);
                if constexpr (F16) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[j], s, 0, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; e++) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e], qf[j][e], s, 0, 0, 0);
                }
            }
            // every pair visible: all 32 queries valid, all keys inside the item
            // and inside every query's window
            const bool full = OPT && wq1 - wq0 == 32 && kb + KB <= c.k_hi &&
                              (!W || (wq1 - 1 - kb <= W && kb + KB - 1 - wq0 <= W));
            float sv[16];
            if (full) {
#pragma unroll
                for (int r = 0; r < 16; r++) sv[r] = s[r] * a.scale_log2;
            } else {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = kb + 8 * (r >> 2) + 4 * hf + (r & 3);
                    const bool vis = qvalid && key < c.k_hi && (!W || abs(tq - key) <= W);
                    sv[r] = vis ? s[r] * a.scale_log2 : -INFINITY;
                }
            }
            float mx = sv[0];
#pragma unroll
            for (int r = 1; r < 16; r++) mx = fmaxf(mx, sv[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx);
            // the output and the running sum are rescaled only when some query's
            // max grew; otherwise the factor would be exactly 1
            if (!OPT || __any(m_new > m_run)) {
                const float alpha = exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
                l_run *= alpha;
#pragma unroll
                for (int d = 0; d < HD / 32; d++)
#pragma unroll
                    for (int r = 0; r < 16; r++) o[d][r] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.0f : m_run;
            float rs = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                sv[r] = exp2f(sv[r] - m_use);
                rs += sv[r];
            }
            l_run += rs + __shfl_xor(rs, 32, 64);
            if constexpr (F16) {
                // B operand: this lane's p for keys 16*s2 + {4hf..4hf+3, 8+4hf..8+4hf+3}
#pragma unroll
                for (int s2 = 0; s2 < 2; s2++) {
                    f16x8 pb;
#pragma unroll
                    for (int e = 0; e < 8; e++) pb[e] = (_Float16)sv[8 * s2 + e];
#pragma unroll
                    for (int d = 0; d < HD / 32; d++) {
                        const uint32_t *vr = &Vs[buf][32 * d + li][8 * s2 + 2 * hf];
                        const uint2 v0 = *reinterpret_cast<const uint2 *>(vr);
                        const uint2 v1 = *reinterpret_cast<const uint2 *>(vr + 4);
                        const uint4 vv = {v0.x, v0.y, v1.x, v1.y};
                        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), pb, o[d], 0, 0, 0);
                    }
                }
            } else {
                // O^T[d][q] += V^T[d][key] P^T[key][q]; step r pairs lane halves' keys
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const float *vr = &Vs[buf][8 * (r >> 2) + 4 * hf + (r & 3)][li];
#pragma unroll
                    for (int d = 0; d < HD / 32; d++)
                        o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * d], sv[r], o[d], 0, 0, 0);
                }
            }
        }
        if (b + 1 < nblk) sstore(buf ^ 1);
        __syncthreads();
    }
    if (qvalid) {
        const float inv = 1.0f / l_run;
        T *out = reinterpret_cast<T *>(a.out) + (size_t)row_of(c.it, tq) * a.ldo + head * HD;
#pragma unroll
        for (int d = 0; d < HD / 32; d++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int ch = 32 * d + 8 * q + 4 * hf;
                const f32x4 v = out_scale(a, head * HD + ch,
                                          f32x4{o[d][4 * q] * inv, o[d][4 * q + 1] * inv,
                                                o[d][4 * q + 2] * inv, o[d][4 * q + 3] * inv});
                if constexpr (F16)
                    st4h(out + ch, v);
                else
                    st4(out + ch, v);
            }
    }
}

// f16 flash attention at head dim 128 with K/V staged by direct global -> LDS
// loads.  Same tiling and softmax as attn_kernel<128, true, ..> (transposed
// scores, a lane per query, lazy rescale, full-block mask fast path); what
// changes is how K and V reach the MFMAs:
//  - a three-stage LDS ring of (K, V) key blocks, each 32 keys x 256 bytes, is
//    filled by global_load_lds_dwordx4 two blocks ahead, with no registers or
//    LDS writes spent on staging and one barrier per block;
//  - V stays row-major (key x channel) and the O^T = V^T P^T operand is read
//    with the transposing ds_read_b64_tr_b16: within each 16-lane group, lane i
//    gets channel C0 + i of four consecutive keys;
//  - K row t keeps 16-byte chunk c at position c ^ (t & 15), V row t at
//    c ^ 4 (t & 3), so fragment reads hit distinct bank groups;
//  - the softmax scale is folded into one FMA per score (p = exp2(s c - m)),
//    and the per-lane partial row sums are combined across the two lane halves
//    once, at the end.
// Keys past the item (in the last block) load a clamped, finite row and are
// masked.  Requires hd = 128 and nq*hd, ld, offsets as attention_items checks.
template <int NW, int MINW>
__global__ __launch_bounds__(64 * NW, MINW) void attn_f16d_kernel(AttnArgs a) {
    constexpr int HD = 128, QT = 32 * NW, NS = 3;
    constexpr int TBYTES = KB * HD * 2;          // one K or V block: 8 KB
    constexpr int SBYTES = 2 * TBYTES;           // a stage: K then V
    constexpr int NI = TBYTES / 1024 / NW;       // load instructions per wave per tile
    constexpr int NDMA = 2 * NI;                 // per wave per stage
    static_assert(TBYTES / 1024 % NW == 0, "waves");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * SBYTES];

    const uint32_t head = blockIdx.x % a.nq, tile = blockIdx.x / a.nq;
    ItemCtx c;
    locate<QT>(a, tile, c);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int kvh = head / a.group;
    const _Float16 *P = reinterpret_cast<const _Float16 *>(a.qkv);
    const int W = (int)a.window;

    const int tq = c.q_lo + wave * 32 + li;
    const bool qvalid = tq < c.q_hi;
    const int wq0 = c.q_lo + wave * 32, wq1 = min(wq0 + 32, c.q_hi);

    f16x8 qf[HD / 16];
    {
        const _Float16 *qp = P + (size_t)row_of(c.it, qvalid ? tq : c.q_lo) * a.ld + a.q_col + head * HD + 64 * hf;
#pragma unroll
        for (int j = 0; j < HD / 16; j++) qf[j] = qvalid ? *reinterpret_cast<const f16x8 *>(qp + 8 * j) : f16x8{};
    }

    // loads: instruction q of this wave covers keys 4 (wave NI + q) .. +3 of the
    // block; lane l takes key + l/16 and LDS position l % 16 of that key row
    const int kl = lane >> 4, pl = lane & 15;
    auto dma = [&](int b) {
        const int kb = c.k_lo + b * KB;
        uint8_t *buf = smem + (b % NS) * SBYTES;
#pragma unroll
        for (int q = 0; q < NI; q++) {
            const int ti = 4 * (wave * NI + q) + kl;
            const int t = min(kb + ti, c.k_hi - 1);
            const _Float16 *row = P + (size_t)row_of(c.it, t) * a.ld + kvh * HD;
            dma16(row + a.k_col + 8 * (pl ^ (ti & 15)), buf + (wave * NI + q) * 1024);
            dma16(row + a.v_col + 8 * (pl ^ (4 * (ti & 3))), buf + TBYTES + (wave * NI + q) * 1024);
        }
    };

    // fragment addresses within a stage: K (key li, chunk 8 hf + j); V^T
    // transposed reads for channel block dblk, key group s2 and half e8
    const uint32_t lds0 = lds_offset(smem);
    const uint32_t krow = lds0 + (uint32_t)li * 256u;
    const int g = lane >> 4, src = lane & 15;
    const uint32_t vrow = lds0 + TBYTES + (uint32_t)(4 * (g >> 1) + (src >> 2)) * 256u + 8u * (src & 1);
    const int vc0 = 2 * (g & 1) + ((src & 3) >> 1);   // chunk within a 32-channel block
    const int vsw = 4 * (src >> 2);                   // row & 3 == src / 4 for every read

    f32x16 o[HD / 32];
#pragma unroll
    for (int d = 0; d < HD / 32; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) o[d][r] = 0.0f;
    float m_run = -INFINITY, l_lane = 0.0f;

    const int nblk = (c.k_hi - c.k_lo + KB - 1) / KB;
    if (nblk > 0) dma(0);
    if (nblk > 1) dma(1);
    for (int b = 0; b < nblk; b++) {
        // block b landed (own loads; block b+1's may still fly), then everyone's;
        // after this barrier no wave reads block b-1's buffer, which takes b+2
        if (b + 1 < nblk)
            vm_wait<NDMA>();
        else
            vm_wait<0>();
        block_barrier();
        if (b + 2 < nblk) dma(b + 2);
        const int kb = c.k_lo + b * KB;
        const bool active = wq0 < wq1 && (!W || (kb <= wq1 - 1 + W && kb + KB - 1 >= wq0 - W));
        if (!active) continue;
        const uint32_t sb = (uint32_t)((b % NS) * SBYTES);

        // LDS reads in flight stay within the 15 the counter holds: K (8) and
        // the first half of V for key group 0 (4), then the rest of group 0
        // during the scores, then group 1 during the first P V products
        u32x4 kf[HD / 16];
#pragma unroll
        for (int j = 0; j < HD / 16; j++) kf[j] = ds_read16(krow + sb + (uint32_t)(((8 * hf + j) ^ (li & 15)) * 16));
        u32x2 vf[HD / 32][2][2];
        auto vread = [&](int d, int s2) {
#pragma unroll
            for (int e8 = 0; e8 < 2; e8++)
                vf[d][s2][e8] = ds_read8_tr16(vrow + sb + (uint32_t)((16 * s2 + 8 * e8) * 256) +
                                              (uint32_t)(((4 * d + vc0) ^ vsw) * 16));
        };
        vread(0, 0);
        vread(1, 0);
        lgkm_wait_n<4>();
#pragma unroll
        for (int j = 0; j < HD / 16; j++) ready(kf[j]);
        vread(2, 0);
        vread(3, 0);

        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; r++) s[r] = 0.0f;
#pragma unroll
        for (int j = 0; j < HD / 16; j++)
            s = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kf[j]), qf[j], s, 0, 0, 0);

        const bool full = wq1 - wq0 == 32 && kb + KB <= c.k_hi &&
                          (!W || (wq1 - 1 - kb <= W && kb + KB - 1 - wq0 <= W));
        if (!full) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int key = kb + 8 * (r >> 2) + 4 * hf + (r & 3);
                const bool vis = qvalid && key < c.k_hi && (!W || abs(tq - key) <= W);
                s[r] = vis ? s[r] : -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; r++) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run)) {
            const float alpha = exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
            l_lane *= alpha;
#pragma unroll
            for (int d = 0; d < HD / 32; d++)
#pragma unroll
                for (int r = 0; r < 16; r++) o[d][r] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            pv[r] = exp2f(fmaf(s[r], a.scale_log2, -m_use));
            l_lane += pv[r];
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) {
            lgkm_wait_n<0>();
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                ready(vf[d][s2][0]);
                ready(vf[d][s2][1]);
            }
            if (s2 == 0)
#pragma unroll
                for (int d = 0; d < HD / 32; d++) vread(d, 1);
            f16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; e++) pb[e] = (_Float16)pv[8 * s2 + e];
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                const u32x4 vv = {vf[d][s2][0][0], vf[d][s2][0][1], vf[d][s2][1][0], vf[d][s2][1][1]};
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), pb, o[d], 0, 0, 0);
            }
        }
    }
    const float l_run = l_lane + __shfl_xor(l_lane, 32, 64);
    if (qvalid) {
        const float inv = 1.0f / l_run;
        _Float16 *out = reinterpret_cast<_Float16 *>(a.out) + (size_t)row_of(c.it, tq) * a.ldo + head * HD;
#pragma unroll
        for (int d = 0; d < HD / 32; d++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int ch = 32 * d + 8 * q + 4 * hf;
                st4h(out + ch, out_scale(a, head * HD + ch,
                                         f32x4{o[d][4 * q] * inv, o[d][4 * q + 1] * inv,
                                               o[d][4 * q + 2] * inv, o[d][4 * q + 3] * inv}));
            }
    }
}


// The attention without a window at hd 128, software-pipelined within each
// wave, with K/V staged as in attn_f16d_kernel (direct global -> LDS loads, a
// ring of four or six stages, the same LDS swizzles) and the per-block overhead cut
// down to the softmax itself:
//  - the loop is unrolled over the LDS stages, so every fragment read is a
//    loop-invariant per-lane address plus an immediate offset (no address
//    arithmetic per block), and the scores of consecutive blocks alternate
//    between two register sets instead of being copied;
//  - a block that lies inside one row range of the item is staged from a
//    wave-uniform row base plus per-lane byte offsets fixed at the start; when
//    every byte offset of the panel fits 31 bits (BUF) these are raw buffer
//    loads with the row base as their scalar offset, so a block's staging
//    costs no address arithmetic in vector registers (2-5% faster on the DiT
//    item tables than 64-bit per-lane addresses, the same bits);
//  - the row sum adds the f16 probabilities that the P V product consumes, two
//    at a time (v_dot2_f32_f16 with ones, f32 accumulation), so numerator and
//    denominator see the same rounded p;
//  - the row max takes three scores per instruction (v_maximum3, no input
//    quieting);
//  - the running max moves only when a block's max passes it by more than 8
//    (in log2 units), and then to that block's max: p = 2^(s c - m) stays at
//    most 256 (exact in f16's range), the output is rescaled only on such a
//    move, and the quotient o / l does not depend on where m sits.
// Step b: the row max of block b's scores; the first half of block b's V
// fragments is read while the K fragments of block b+1 (read at the end of
// step b-1) land; the scores of block b+1 (a dependent MFMA chain) run
// interleaved with the exponentials of block b, each MFMA waiting only for its
// own K fragment (4% on the 1056-row DiT table, where one wave per SIMD leaves
// the read latency exposed); then the second half of V is read and the first
// half of P V issued.
// The step's one barrier comes after the wave's last LDS read of stage b, and
// behind it the freed stage takes block b+4, block b+2's K fragments are read
// and the second half of P V is issued: those MFMAs and the K reads overlap
// the next step's row max instead of waiting on a fragment read at its top
// (2-4% faster than reading K at the top of the step, the same bits).  With
// PAIR (8-wave blocks, one per CU) the ring has six stages and the barrier
// comes after odd blocks only: blocks b+1 .. b+3 have landed by then and the
// stages of blocks b-2 and b-1 take blocks b+4 and b+5, so each load still
// has two steps to land and the block synchronises half as often (1% on the
// 8448-row DiT table and the long-sequence steady state, the same bits).  The
// LDS holds the stages' K blocks, then their V blocks.  Keys
// past the item occur only in the last block and are masked there; rows past
// the item's queries are computed on clamped data and never stored; the last
// step's scores of a block past the end come from a stale stage and are never
// used.
template <int NW, int MINW, bool BUF, bool PAIR>
__global__ __launch_bounds__(64 * NW, MINW) void attn_f16s_kernel(AttnArgs a) {
    constexpr int HD = 128, QT = 32 * NW, NS = PAIR ? 6 : 4;
    constexpr int TBYTES = KB * HD * 2;   // one K or V block: 8 KB
    constexpr int SBYTES = 2 * TBYTES;    // a stage's K and V blocks
    constexpr int VREG = NS * TBYTES;     // the stages' K blocks, then from VREG their V blocks
    constexpr int NI = TBYTES / 1024 / NW;
    constexpr int NDMA = 2 * NI;
    static_assert(TBYTES / 1024 % NW == 0, "waves");
    static_assert(VREG <= 65536, "immediate LDS offsets");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * SBYTES];

    const uint32_t head = blockIdx.x % a.nq, tile = blockIdx.x / a.nq;
    ItemCtx c;
    locate<QT>(a, tile, c);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int kvh = head / a.group;
    const _Float16 *P = reinterpret_cast<const _Float16 *>(a.qkv);

    const int tq = c.q_lo + wave * 32 + li;
    const bool qvalid = tq < c.q_hi;
    const bool wactive = c.q_lo + wave * 32 < c.q_hi;  // waves without queries only join the barriers

    f16x8 qf[HD / 16];
    {
        const _Float16 *qp = P + (size_t)row_of(c.it, qvalid ? tq : c.q_lo) * a.ld + a.q_col + head * HD + 64 * hf;
#pragma unroll
        for (int j = 0; j < HD / 16; j++) qf[j] = *reinterpret_cast<const f16x8 *>(qp + 8 * j);
        vm_wait<0>();
#pragma unroll
        for (int j = 0; j < HD / 16; j++) ready(qf[j]);
    }

    // staging: instruction q of this wave covers keys 4 (wave NI + q) .. +3 of a
    // block; lane l takes key + l/16 and LDS position l % 16 of that key row,
    // which holds chunk (l%16) ^ (key & 15) of K and (l%16) ^ 4 (key & 3) of V
    const int kl = lane >> 4, pl = lane & 15;
    uint32_t kso[NI], vso[NI];  // byte offsets from the block's first row
#pragma unroll
    for (int q = 0; q < NI; q++) {
        const uint32_t ti = 4 * (wave * NI + q) + kl;
        const uint32_t r = ti * a.ld + kvh * HD;
        kso[q] = 2 * (r + a.k_col + 8 * (pl ^ (ti & 15)));
        vso[q] = 2 * (r + a.v_col + 8 * (pl ^ (4 * (ti & 3))));
    }
    const int na = (int)c.it.na;
    const __amdgpu_buffer_rsrc_t pres = raw_buffer(P);
    auto dma = [&](auto st, int b) {
        uint8_t *buf = smem + decltype(st)::value * TBYTES;
        const int kb = c.k_lo + b * KB;
        if (kb + KB <= c.k_hi && (kb + KB <= na || kb >= na)) {
            const int r0 = kb < na ? (int)c.it.r0a + kb : (int)c.it.r0b + (kb - na);
            if constexpr (BUF) {
                const uint32_t soff = (uint32_t)r0 * a.ld * 2u;
#pragma unroll
                for (int q = 0; q < NI; q++) {
                    buffer_dma16(pres, buf + (wave * NI + q) * 1024, kso[q], soff);
                    buffer_dma16(pres, buf + VREG + (wave * NI + q) * 1024, vso[q], soff);
                }
            } else {
                const char *base = reinterpret_cast<const char *>(P + (size_t)r0 * a.ld);
#pragma unroll
                for (int q = 0; q < NI; q++) {
                    dma16(base + kso[q], buf + (wave * NI + q) * 1024);
                    dma16(base + vso[q], buf + VREG + (wave * NI + q) * 1024);
                }
            }
        } else {
            // the block crosses into the second row range or past the item:
            // rows per lane, keys past the item clamped to its last row (masked)
#pragma unroll
            for (int q = 0; q < NI; q++) {
                const int ti = 4 * (wave * NI + q) + kl;
                const int t = min(kb + ti, c.k_hi - 1);
                const char *base = reinterpret_cast<const char *>(P + ((ptrdiff_t)row_of(c.it, t) - ti) * a.ld);
                dma16(base + kso[q], buf + (wave * NI + q) * 1024);
                dma16(base + vso[q], buf + VREG + (wave * NI + q) * 1024);
            }
        }
    };

    // fragment addresses (stage 0): K row li, chunk 8 hf + j; V^T transposed
    // reads of channel block d (key group and half are immediates)
    const uint32_t lds0 = lds_offset(smem);
    uint32_t kaddr[HD / 16], vaddr[HD / 32];
#pragma unroll
    for (int j = 0; j < HD / 16; j++) kaddr[j] = lds0 + (uint32_t)li * 256u + (uint32_t)(((8 * hf + j) ^ (li & 15)) * 16);
    {
        const int g = lane >> 4, src = lane & 15;
        const uint32_t vrow = lds0 + VREG + (uint32_t)(4 * (g >> 1) + (src >> 2)) * 256u + 8u * (src & 1);
        const int vc0 = 2 * (g & 1) + ((src & 3) >> 1), vsw = 4 * (src >> 2);
#pragma unroll
        for (int d = 0; d < HD / 32; d++) vaddr[d] = vrow + (uint32_t)(((4 * d + vc0) ^ vsw) * 16);
    }
    u32x4 kf[HD / 16];
    u32x2 vf[HD / 32][2][2];
    auto vread = [&](auto st, int d, auto s2c) {
        constexpr int s2 = decltype(s2c)::value;
        constexpr int off = decltype(st)::value * TBYTES + 16 * s2 * 256;
        vf[d][s2][0] = ds_read8_tr16_at<off>(vaddr[d]);
        vf[d][s2][1] = ds_read8_tr16_at<off + 8 * 256>(vaddr[d]);
    };

    auto kread_to = [&](auto st, u32x4 (&k)[HD / 16]) {
        constexpr int off = decltype(st)::value * TBYTES;
#pragma unroll
        for (int j = 0; j < HD / 16; j++) k[j] = ds_read16_at<off>(kaddr[j]);
    };

    f32x16 o[HD / 32];
#pragma unroll
    for (int d = 0; d < HD / 32; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) o[d][r] = 0.0f;
    float m_run = -INFINITY, l_lane = 0.0f;
    const float cs = a.scale_log2;
    // the scalar load of the scale lands here, on every path into the loop: a
    // load still pending at the loop head makes the compiler wait for every LDS
    // read in flight (lgkmcnt(0)) at the scale's first use in each step
    asm volatile("" ::"s"(cs));
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    const int nblk = (c.k_hi - c.k_lo + KB - 1) / KB;
    if (nblk > 0) dma(IC<0>{}, 0);
    if (nblk > 1) dma(IC<1>{}, 1);
    if (nblk > 2) dma(IC<2>{}, 2);
    if (nblk > 3) dma(IC<3>{}, 3);
    if constexpr (PAIR) {
        if (nblk > 4) dma(IC<4>{}, 4);
    }
    {
        // landed before the first barrier: blocks 0 and 1, and with PAIR
        // block 2 too (no barrier follows step 0)
        const int fly = PAIR ? max(0, min(5, nblk) - 3) : max(0, min(NS, nblk) - 2);
        if (fly >= 2)
            vm_wait<2 * NDMA>();
        else if (fly == 1)
            vm_wait<NDMA>();
        else
            vm_wait<0>();
    }
    block_barrier();
    f32x16 sA, sB;
#pragma unroll
    for (int r = 0; r < 16; r++) sA[r] = 0.0f;
    if (wactive && nblk > 0) {
        kread_to(IC<0>{}, kf);
        lgkm_wait_n<0>();
#pragma unroll
        for (int j = 0; j < HD / 16; j++) {
            ready(kf[j]);
            sA = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kf[j]), qf[j], sA, 0, 0, 0);
        }
        if (nblk > 1) kread_to(IC<1>{}, kf);
    }

    // block b (stage st): scores in s_cur, block b+1's K fragments in flight in
    // kf; leaves block b+1's scores in s_nx and block b+2's K in flight
    auto step = [&](auto st, int b, f32x16 &s_cur, f32x16 &s_nx) {
        constexpr int S = decltype(st)::value;
        f16x8 pb[2];
        if (wactive) {
            const int kb = c.k_lo + b * KB;
            if (kb + KB > c.k_hi) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = kb + 8 * (r >> 2) + 4 * hf + (r & 3);
                    s_cur[r] = key < c.k_hi ? s_cur[r] : -INFINITY;
                }
            }
            // row max (v_maximum3: no input quieting; a NaN score gives a NaN
            // max, which reaches the output)
            float mx = __builtin_elementwise_maximum(s_cur[0], s_cur[1]);
#pragma unroll
            for (int r = 2; r < 16; r++) mx = __builtin_elementwise_maximum(mx, s_cur[r]);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            // the running max moves (to this block's max) only when it is
            // passed by more than 8; the output and the row sum follow it then
            const float mb = mx * cs;
            const bool up = mb > m_run + 8.0f;
            if (__any(up)) {
                const float m_new = up ? mb : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_lane *= alpha;
#pragma unroll
                for (int d = 0; d < HD / 32; d++)
#pragma unroll
                    for (int r = 0; r < 16; r++) o[d][r] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.0f : m_run;

            // the first half of block b's V fragments; then the scores of
            // block b+1 fragment by fragment as its K reads land (DS reads
            // complete in order: K fragment j has landed once at most 15 - j
            // reads are in flight), each MFMA behind a pair of block b's
            // exponentials, which need no fragment
            vread(st, 0, IC<0>{});
            vread(st, 1, IC<0>{});
            vread(st, 2, IC<0>{});
            vread(st, 3, IC<0>{});
#pragma unroll
            for (int r = 0; r < 16; r++) s_nx[r] = 0.0f;
            float rs = 0.0f;
            auto group = [&](auto jc) {
                constexpr int j = decltype(jc)::value, s2 = j / 4, e = 2 * (j % 4);
                const f16x2 pr = {(_Float16)__builtin_amdgcn_exp2f(fmaf(s_cur[8 * s2 + e], cs, -m_use)),
                                  (_Float16)__builtin_amdgcn_exp2f(fmaf(s_cur[8 * s2 + e + 1], cs, -m_use))};
                pb[s2][e] = pr[0];
                pb[s2][e + 1] = pr[1];
                rs = __builtin_amdgcn_fdot2(pr, ones, rs, false);
                __builtin_amdgcn_sched_barrier(0);
                lgkm_wait_n<15 - j>();
                ready(kf[j]);
                s_nx = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kf[j]), qf[j], s_nx, 0, 0, 0);
            };
            group(IC<0>{});
            group(IC<1>{});
            group(IC<2>{});
            group(IC<3>{});
            group(IC<4>{});
            group(IC<5>{});
            group(IC<6>{});
            group(IC<7>{});
            l_lane += rs;
            vread(st, 0, IC<1>{});
            vread(st, 1, IC<1>{});
            vread(st, 2, IC<1>{});
            vread(st, 3, IC<1>{});
            lgkm_wait_n<8>();  // the first half of V landed
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                ready(vf[d][0][0]);
                ready(vf[d][0][1]);
            }
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                const u32x4 vv = {vf[d][0][0][0], vf[d][0][0][1], vf[d][0][1][0], vf[d][0][1][1]};
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), pb[0], o[d], 0, 0, 0);
            }
            lgkm_wait_n<0>();
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                ready(vf[d][1][0]);
                ready(vf[d][1][1]);
            }
        }
        // every wave: stage b+2 landed (b+3 may fly) and this wave's reads of
        // stage b done; after the barrier stage b+2 is readable everywhere and
        // stage b's buffer takes block b+4
        if constexpr (PAIR) {
            // one barrier per two blocks, after odd blocks: blocks b+1 .. b+3
            // landed (everything issued so far) and every wave done with the
            // stages of blocks b-2 and b-1, which take blocks b+4 and b+5
            if constexpr (S & 1) {
                vm_wait<0>();
                block_barrier();
                if (b + 4 < nblk) dma(IC<(S + 4) % NS>{}, b + 4);
                if (b + 5 < nblk) dma(IC<(S + 5) % NS>{}, b + 5);
            }
        } else {
            if (b + 3 < nblk)
                vm_wait<NDMA>();
            else
                vm_wait<0>();
            block_barrier();
            if (b + 4 < nblk) dma(IC<S>{}, b + 4);
        }
        if (!wactive) return;
        // into the registers block b+1's score MFMAs read (issued long before)
        if (b + 2 < nblk) kread_to(IC<(S + 2) % NS>{}, kf);
#pragma unroll
        for (int d = 0; d < HD / 32; d++) {
            const u32x4 vv = {vf[d][1][0][0], vf[d][1][0][1], vf[d][1][1][0], vf[d][1][1][1]};
            o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), pb[1], o[d], 0, 0, 0);
        }
    };
    for (int b = 0; b < nblk; b += NS) {
        step(IC<0>{}, b, sA, sB);
        if (b + 1 >= nblk) break;
        step(IC<1>{}, b + 1, sB, sA);
        if (b + 2 >= nblk) break;
        step(IC<2>{}, b + 2, sA, sB);
        if (b + 3 >= nblk) break;
        step(IC<3>{}, b + 3, sB, sA);
        if constexpr (PAIR) {
            if (b + 4 >= nblk) break;
            step(IC<4>{}, b + 4, sA, sB);
            if (b + 5 >= nblk) break;
            step(IC<5>{}, b + 5, sB, sA);
        }
    }
    const float l_run = l_lane + __shfl_xor(l_lane, 32, 64);
    if (qvalid) {
        const float inv = 1.0f / l_run;
        _Float16 *out = reinterpret_cast<_Float16 *>(a.out) + (size_t)row_of(c.it, tq) * a.ldo + head * HD;
#pragma unroll
        for (int d = 0; d < HD / 32; d++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int ch = 32 * d + 8 * q + 4 * hf;
                st4h(out + ch, out_scale(a, head * HD + ch,
                                         f32x4{o[d][4 * q] * inv, o[d][4 * q + 1] * inv,
                                               o[d][4 * q + 2] * inv, o[d][4 * q + 3] * inv}));
            }
    }
}

// f16 flash attention at head dim 128 for short items, with each query's keys
// split two ways inside the block.  An item of 1056 rows has 33 groups of 32
// queries per head: 990 waves of 32 queries for 30 heads on 1024 SIMDs, one
// wave per SIMD with nothing to hide its latencies.  Here a block of four waves
// takes 64 queries of one item and one head: waves 0 and 1 (part 0) run the
// first ceil(n/2) of the item's n key blocks for their 32 queries each, waves
// 2 and 3 (part 1) the rest, and at the end part 1 hands its unnormalised
// output, running max and row sums to part 0 through the LDS.  The result is
// part 0's sums plus part 1's, each rescaled to the larger of the two running
// maxima: the split follows the item's length alone, so an item gets the same
// bits in any batch.
// Each part has its own two-stage K ring and two-stage V ring (32 KB; 64 KB a
// block, so two blocks share a CU and each SIMD holds two waves).  Step b of a
// part: the row max of block b; V(b) read from its stage; the scores of block
// b+1 interleaved with block b's exponentials (as in attn_f16s_kernel); the
// first half of P V; one barrier, behind which the freed stages take K(b+3)
// and V(b+2), K(b+2) is read into registers and the second half of P V is
// issued.  A load has one step to land.
template <bool BUF>
__global__ __launch_bounds__(256, 2) void attn_f16k_kernel(AttnArgs a) {
    constexpr int HD = 128, QT = 64;
    constexpr int TBYTES = KB * HD * 2;    // one K or V block: 8 KB
    constexpr int PBYTES = 4 * TBYTES;     // a part's K stages 0, 1, then its V stages 0, 1
    constexpr int NI = TBYTES / 1024 / 2;  // load instructions per wave per K or V block
    constexpr int XW = HD / 32 * 16 + 2;   // floats a lane hands over: o, running max, row sum
    static_assert(2 * XW * 64 * 4 <= 2 * PBYTES, "hand-over fits the ring");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * PBYTES];

    const uint32_t head = blockIdx.x % a.nq, tile = blockIdx.x / a.nq;
    ItemCtx c;
    locate<QT>(a, tile, c);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: the part's values stay scalar
    const int qg = wave & 1, part = wave >> 1;
    const int li = lane & 31, hf = lane >> 5;
    const int kvh = head / a.group;
    const _Float16 *P = reinterpret_cast<const _Float16 *>(a.qkv);

    const int tq = c.q_lo + qg * 32 + li;
    const bool qvalid = tq < c.q_hi;
    const bool wactive = c.q_lo + qg * 32 < c.q_hi;  // waves without queries only join the barriers

    // this part's key blocks: [g0, g0 + nmine) of the item's nblk
    const int nblk = (c.k_hi - c.k_lo + KB - 1) / KB;
    const int n0 = (nblk + 1) / 2;
    const int g0 = part ? n0 : 0;
    const int nmine = part ? nblk - n0 : n0;
    uint8_t *const pbuf = smem + part * PBYTES;

    f16x8 qf[HD / 16];
    {
        const _Float16 *qp = P + (size_t)row_of(c.it, qvalid ? tq : c.q_lo) * a.ld + a.q_col + head * HD + 64 * hf;
#pragma unroll
        for (int j = 0; j < HD / 16; j++) qf[j] = *reinterpret_cast<const f16x8 *>(qp + 8 * j);
        vm_wait<0>();
#pragma unroll
        for (int j = 0; j < HD / 16; j++) ready(qf[j]);
    }

    // staging (as attn_f16s_kernel, over the part's two waves): instruction q
    // of this wave covers keys 4 (qg NI + q) .. +3 of a block
    const int kl = lane >> 4, pl = lane & 15;
    uint32_t kso[NI], vso[NI];
#pragma unroll
    for (int q = 0; q < NI; q++) {
        const uint32_t ti = 4 * (qg * NI + q) + kl;
        const uint32_t r = ti * a.ld + kvh * HD;
        kso[q] = 2 * (r + a.k_col + 8 * (pl ^ (ti & 15)));
        vso[q] = 2 * (r + a.v_col + 8 * (pl ^ (4 * (ti & 3))));
    }
    const int na = (int)c.it.na;
    const __amdgpu_buffer_rsrc_t pres = raw_buffer(P);
    // key block b of the item (K with V = false) into the 8 KB at buf
    auto dma = [&](uint8_t *buf, bool v, int b) {
        const int kb = c.k_lo + b * KB;
        if (kb + KB <= c.k_hi && (kb + KB <= na || kb >= na)) {
            const int r0 = kb < na ? (int)c.it.r0a + kb : (int)c.it.r0b + (kb - na);
            if constexpr (BUF) {
                const uint32_t soff = (uint32_t)r0 * a.ld * 2u;
#pragma unroll
                for (int q = 0; q < NI; q++) buffer_dma16(pres, buf + (qg * NI + q) * 1024, v ? vso[q] : kso[q], soff);
            } else {
                const char *base = reinterpret_cast<const char *>(P + (size_t)r0 * a.ld);
#pragma unroll
                for (int q = 0; q < NI; q++) dma16(base + (v ? vso[q] : kso[q]), buf + (qg * NI + q) * 1024);
            }
        } else {
            // the block crosses into the second row range or past the item:
            // rows per lane, keys past the item clamped to its last row (masked)
#pragma unroll
            for (int q = 0; q < NI; q++) {
                const int ti = 4 * (qg * NI + q) + kl;
                const int t = min(kb + ti, c.k_hi - 1);
                const char *base = reinterpret_cast<const char *>(P + ((ptrdiff_t)row_of(c.it, t) - ti) * a.ld);
                dma16(base + (v ? vso[q] : kso[q]), buf + (qg * NI + q) * 1024);
            }
        }
    };
    auto dmaK = [&](auto st, int b) { dma(pbuf + decltype(st)::value * TBYTES, false, b); };
    auto dmaV = [&](auto st, int b) { dma(pbuf + (2 + decltype(st)::value) * TBYTES, true, b); };

    // fragment addresses in the part's ring (as attn_f16s_kernel)
    const uint32_t lds0 = lds_offset(pbuf);
    uint32_t kaddr[HD / 16], vaddr[HD / 32];
#pragma unroll
    for (int j = 0; j < HD / 16; j++) kaddr[j] = lds0 + (uint32_t)li * 256u + (uint32_t)(((8 * hf + j) ^ (li & 15)) * 16);
    {
        const int g = lane >> 4, src = lane & 15;
        const uint32_t vrow = lds0 + 2 * TBYTES + (uint32_t)(4 * (g >> 1) + (src >> 2)) * 256u + 8u * (src & 1);
        const int vc0 = 2 * (g & 1) + ((src & 3) >> 1), vsw = 4 * (src >> 2);
#pragma unroll
        for (int d = 0; d < HD / 32; d++) vaddr[d] = vrow + (uint32_t)(((4 * d + vc0) ^ vsw) * 16);
    }
    u32x4 kf[HD / 16];
    u32x2 vf[HD / 32][2][2];
    auto vread = [&](auto st, int d, auto s2c) {
        constexpr int s2 = decltype(s2c)::value;
        constexpr int off = decltype(st)::value * TBYTES + 16 * s2 * 256;
        vf[d][s2][0] = ds_read8_tr16_at<off>(vaddr[d]);
        vf[d][s2][1] = ds_read8_tr16_at<off + 8 * 256>(vaddr[d]);
    };
    auto kread_to = [&](auto st, u32x4 (&k)[HD / 16]) {
        constexpr int off = decltype(st)::value * TBYTES;
#pragma unroll
        for (int j = 0; j < HD / 16; j++) k[j] = ds_read16_at<off>(kaddr[j]);
    };

    f32x16 o[HD / 32];
#pragma unroll
    for (int d = 0; d < HD / 32; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) o[d][r] = 0.0f;
    float m_run = -INFINITY, l_lane = 0.0f;
    const float cs = a.scale_log2;
    // the scalar load of the scale lands here, on every path into the loop: a
    // load still pending at the loop head makes the compiler wait for every LDS
    // read in flight (lgkmcnt(0)) at the scale's first use in each step
    asm volatile("" ::"s"(cs));
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    // K(0), V(0), K(1); after K(0) is read everywhere, K(2) and V(1)
    if (nmine > 0) {
        dmaK(IC<0>{}, g0);
        dmaV(IC<0>{}, g0);
    }
    if (nmine > 1) dmaK(IC<1>{}, g0 + 1);
    vm_wait<0>();
    block_barrier();
    f32x16 sA, sB;
#pragma unroll
    for (int r = 0; r < 16; r++) sA[r] = 0.0f;
    if (wactive && nmine > 0) {
        kread_to(IC<0>{}, kf);
        lgkm_wait_n<0>();
#pragma unroll
        for (int j = 0; j < HD / 16; j++) {
            ready(kf[j]);
            sA = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kf[j]), qf[j], sA, 0, 0, 0);
        }
        if (nmine > 1) kread_to(IC<1>{}, kf);
    }
    block_barrier();
    if (nmine > 2) dmaK(IC<0>{}, g0 + 2);
    if (nmine > 1) dmaV(IC<1>{}, g0 + 1);

    // part block b (K and V stage S = b % 2): scores in s_cur, block b+1's K
    // fragments in flight in kf; leaves block b+1's scores in s_nx and block
    // b+2's K in flight
    auto step = [&](auto st, int b, f32x16 &s_cur, f32x16 &s_nx) {
        constexpr int S = decltype(st)::value;
        f16x8 pb[2];
        const bool act = wactive && b < nmine;
        if (act) {
            const int kb = c.k_lo + (g0 + b) * KB;
            if (kb + KB > c.k_hi) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = kb + 8 * (r >> 2) + 4 * hf + (r & 3);
                    s_cur[r] = key < c.k_hi ? s_cur[r] : -INFINITY;
                }
            }
            float mx = __builtin_elementwise_maximum(s_cur[0], s_cur[1]);
#pragma unroll
            for (int r = 2; r < 16; r++) mx = __builtin_elementwise_maximum(mx, s_cur[r]);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float mb = mx * cs;
            const bool up = mb > m_run + 8.0f;
            if (__any(up)) {
                const float m_new = up ? mb : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_lane *= alpha;
#pragma unroll
                for (int d = 0; d < HD / 32; d++)
#pragma unroll
                    for (int r = 0; r < 16; r++) o[d][r] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.0f : m_run;

            vread(st, 0, IC<0>{});
            vread(st, 1, IC<0>{});
            vread(st, 2, IC<0>{});
            vread(st, 3, IC<0>{});
#pragma unroll
            for (int r = 0; r < 16; r++) s_nx[r] = 0.0f;
            float rs = 0.0f;
            // K fragment j of block b+1 has landed once at most 15 - j reads
            // are in flight (its 8 reads, then V's 8; DS reads complete in order)
            auto group = [&](auto jc) {
                constexpr int j = decltype(jc)::value, s2 = j / 4, e = 2 * (j % 4);
                const f16x2 pr = {(_Float16)__builtin_amdgcn_exp2f(fmaf(s_cur[8 * s2 + e], cs, -m_use)),
                                  (_Float16)__builtin_amdgcn_exp2f(fmaf(s_cur[8 * s2 + e + 1], cs, -m_use))};
                pb[s2][e] = pr[0];
                pb[s2][e + 1] = pr[1];
                rs = __builtin_amdgcn_fdot2(pr, ones, rs, false);
                __builtin_amdgcn_sched_barrier(0);
                lgkm_wait_n<15 - j>();
                ready(kf[j]);
                s_nx = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kf[j]), qf[j], s_nx, 0, 0, 0);
            };
            group(IC<0>{});
            group(IC<1>{});
            group(IC<2>{});
            group(IC<3>{});
            group(IC<4>{});
            group(IC<5>{});
            group(IC<6>{});
            group(IC<7>{});
            l_lane += rs;
            vread(st, 0, IC<1>{});
            vread(st, 1, IC<1>{});
            vread(st, 2, IC<1>{});
            vread(st, 3, IC<1>{});
            lgkm_wait_n<8>();  // the first half of V landed
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                ready(vf[d][0][0]);
                ready(vf[d][0][1]);
            }
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                const u32x4 vv = {vf[d][0][0][0], vf[d][0][0][1], vf[d][0][1][0], vf[d][0][1][1]};
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), pb[0], o[d], 0, 0, 0);
            }
            lgkm_wait_n<0>();
#pragma unroll
            for (int d = 0; d < HD / 32; d++) {
                ready(vf[d][1][0]);
                ready(vf[d][1][1]);
            }
        }
        // every wave: K(b+2) and V(b+1) landed and this wave's reads of K(b+1)
        // and V(b) done; behind the barrier K stage S + 1 takes K(b+3) and V
        // stage S takes V(b+2)
        vm_wait<0>();
        block_barrier();
        if (b + 3 < nmine) dmaK(IC<(S + 1) % 2>{}, g0 + b + 3);
        if (b + 2 < nmine) dmaV(st, g0 + b + 2);
        if (!act) return;
        if (b + 2 < nmine) kread_to(st, kf);
#pragma unroll
        for (int d = 0; d < HD / 32; d++) {
            const u32x4 vv = {vf[d][1][0][0], vf[d][1][0][1], vf[d][1][1][0], vf[d][1][1][1]};
            o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), pb[1], o[d], 0, 0, 0);
        }
    };
    // both parts take n0 steps (the barriers); part 1 idles through the last
    // one when nblk is odd
    for (int b = 0; b < n0; b += 2) {
        step(IC<0>{}, b, sA, sB);
        if (b + 1 >= n0) break;
        step(IC<1>{}, b + 1, sB, sA);
    }

    // hand-over (ordinary LDS stores and loads, so barriers with fences): no
    // read of the ring is pending after the last step's barrier (its K read
    // needs b + 2 < nmine)
    __syncthreads();
    float *const xch = reinterpret_cast<float *>(smem) + qg * XW * 64 + lane;
    if (part == 1) {
#pragma unroll
        for (int d = 0; d < HD / 32; d++)
#pragma unroll
            for (int r = 0; r < 16; r++) xch[(16 * d + r) * 64] = o[d][r];
        xch[(XW - 2) * 64] = m_run;
        xch[(XW - 1) * 64] = l_lane;
    }
    __syncthreads();
    if (part == 1) return;
    const float m1 = xch[(XW - 2) * 64], l1 = xch[(XW - 1) * 64];
    const float mm = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    const float l_m = l_lane * a0 + l1 * a1;
    const float l_run = l_m + __shfl_xor(l_m, 32, 64);
    if (qvalid) {
        const float inv = 1.0f / l_run;
        _Float16 *out = reinterpret_cast<_Float16 *>(a.out) + (size_t)row_of(c.it, tq) * a.ldo + head * HD;
#pragma unroll
        for (int d = 0; d < HD / 32; d++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int ch = 32 * d + 8 * q + 4 * hf;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * q + e;
                    v[e] = (o[d][r] * a0 + xch[(16 * d + r) * 64] * a1) * inv;
                }
                st4h(out + ch, out_scale(a, head * HD + ch, v));
            }
    }
}

// Tiles of the launch for QT queries per block (fills tile0, ntiles): q-tiles
// times key splits per item.  Only the f32 kernel reads the split fields; the
// host gives every item of an f16 launch nsplit = 1.
inline uint32_t plan_tiles(AttnArgs &a, int QT) {
    uint32_t tiles = 0;
    for (uint32_t i = 0; i < a.nitems; i++) {
        a.items[i].tile0 = tiles;
        tiles += (a.items[i].na + a.items[i].nb + QT - 1) / QT * a.items[i].nsplit;
    }
    a.ntiles = tiles;
    return tiles;
}

template <int NW, int MINW>
hipError_t launch_f16d(AttnArgs a, hipStream_t s) {
    const uint32_t tiles = plan_tiles(a, 32 * NW);
    if (!tiles) return hipSuccess;
    hipLaunchKernelGGL((attn_f16d_kernel<NW, MINW>), dim3(tiles * a.nq), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

template <int NW, int MINW>
hipError_t launch_f16s(AttnArgs a, hipStream_t s) {
    const uint32_t tiles = plan_tiles(a, 32 * NW);
    if (!tiles) return hipSuccess;
    constexpr bool PAIR = NW == 8;
    if ((uint64_t)a.rows * a.ld * 2u <= 0x7fffffffu)
        hipLaunchKernelGGL((attn_f16s_kernel<NW, MINW, true, PAIR>), dim3(tiles * a.nq), dim3(64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((attn_f16s_kernel<NW, MINW, false, PAIR>), dim3(tiles * a.nq), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

inline hipError_t launch_f16k(AttnArgs a, hipStream_t s) {
    const uint32_t tiles = plan_tiles(a, 64);
    if (!tiles) return hipSuccess;
    if ((uint64_t)a.rows * a.ld * 2u <= 0x7fffffffu)
        hipLaunchKernelGGL((attn_f16k_kernel<true>), dim3(tiles * a.nq), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((attn_f16k_kernel<false>), dim3(tiles * a.nq), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int HD, bool F16, int NW, int MINW, bool OPT>
hipError_t launch(AttnArgs a, hipStream_t s) {
    const uint32_t tiles = plan_tiles(a, 32 * NW);
    if (!tiles) return hipSuccess;
    hipLaunchKernelGGL((attn_kernel<HD, F16, NW, MINW, OPT>), dim3(tiles * a.nq), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

}  // namespace attn
}  // namespace enc
