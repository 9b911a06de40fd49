// Row ops of the encoder block on gfx950: HBM-bound, one wavefront per row.
//
// What they compute:
//  - RMSNorm y = x w / sqrt(mean(x^2) + eps), gain multiplying directly:
//    egemma2.rs (cortiq-engine 0.8.39), `Prog::rms`.
//  - LayerNorm with bias, population variance: vision_encoder_gpu.rs (cera
//    0.2.4), `VitGpuOps::layernorm`.
//  - post-norm residual fused with the next pre-norm, h += rms(t) w_post;
//    a = rms(h) w_next: egemma2.rs `Prog::add_norm`; zimage.rs (cortiq-engine
//    0.7.6) `Enc::rowop`.
//  - q/k RMSNorm per head then RoPE rotate_half within `sec` channels:
//    egemma2.rs `Prog::qkv` / `EgQkv`; zimage.rs `PQk`.
//  - gated activations gelu_tanh(g) u (egemma2.rs `Prog::gelu`) and
//    silu(g) u (zimage.rs `PSw`).
//  - mean pool of each item's rows: egemma2.rs, final norm + pool of
//    `TextGpu::forward`.
//
// Layout: a row is held in registers as NV float4 per lane (lane-strided so a
// wave's loads of one float4 slot cover 1 KiB contiguous), reduced with a
// 64-lane butterfly.  The row statistics come from the same inline functions
// in every kernel, so a fused add_norm produces exactly the bits a separate
// rms_norm of the updated residual would.
#include <math.h>

#include <algorithm>

#include "dev.h"
#include "kern.h"

namespace enc {

namespace {

template <int NV>
struct Row {
    f32x4 v[NV];
};

template <int NV>
__device__ __forceinline__ void load_row(Row<NV> &r, const float *x, int d, int lane) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int c = (i * 64 + lane) * 4;
        r.v[i] = c < d ? ld4(x + c) : f32x4{0, 0, 0, 0};
    }
}

template <int NV>
__device__ __forceinline__ void store_row(const Row<NV> &r, void *y, bool f16, int d, int lane) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int c = (i * 64 + lane) * 4;
        if (c < d) {
            if (f16)
                st4h(reinterpret_cast<_Float16 *>(y) + c, r.v[i]);
            else
                st4(reinterpret_cast<float *>(y) + c, r.v[i]);
        }
    }
}

// 1 / sqrt(mean(x^2) + eps) of a register-resident row
template <int NV>
__device__ __forceinline__ float rms_inv(const Row<NV> &r, int d, float eps) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; i++)
#pragma unroll
        for (int e = 0; e < 4; e++) ss = fmaf(r.v[i][e], r.v[i][e], ss);
    ss = wave_sum(ss);
    return 1.0f / sqrtf(ss / (float)d + eps);
}

template <int NV>
__device__ __forceinline__ Row<NV> rms_apply(const Row<NV> &r, float inv, const float *w, int d,
                                             int lane) {
    Row<NV> y;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int c = (i * 64 + lane) * 4;
        const f32x4 wv = c < d ? ld4(w + c) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; e++) y.v[i][e] = r.v[i][e] * inv * wv[e];
    }
    return y;
}

template <int NV, bool F16>
__global__ __launch_bounds__(256) void rms_norm_kernel(NormArgs a) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= (int)a.rows) return;
    Row<NV> r;
    load_row(r, a.x + (size_t)row * a.ldx, a.d, lane);
#pragma unroll
    for (int i = 0; i < NV; i++) r.v[i] *= a.pre;  // exact when pre == 1
    const float inv = rms_inv(r, a.d, a.eps);
    Row<NV> y = rms_apply(r, inv, a.w, a.d, lane);
    if (F16)
        store_row(y, reinterpret_cast<_Float16 *>(a.y) + (size_t)row * a.ldy, true, a.d, lane);
    else
        store_row(y, reinterpret_cast<float *>(a.y) + (size_t)row * a.ldy, false, a.d, lane);
}

template <int NV, bool F16>
__global__ __launch_bounds__(256) void layer_norm_kernel(NormArgs a) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= (int)a.rows) return;
    Row<NV> r;
    load_row(r, a.x + (size_t)row * a.ldx, a.d, lane);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; i++)
#pragma unroll
        for (int e = 0; e < 4; e++) s += r.v[i][e];
    const float mean = wave_sum(s) / (float)a.d;
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int c = (i * 64 + lane) * 4;
        if (c < (int)a.d)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float z = r.v[i][e] - mean;
                ss = fmaf(z, z, ss);
            }
    }
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)a.d + a.eps);
    Row<NV> y;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int c = (i * 64 + lane) * 4;
        const f32x4 wv = c < (int)a.d ? ld4(a.w + c) : f32x4{0, 0, 0, 0};
        const f32x4 bv = (a.b && c < (int)a.d) ? ld4(a.b + c) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; e++) y.v[i][e] = (r.v[i][e] - mean) * inv * wv[e] + bv[e];
    }
    if (F16)
        store_row(y, reinterpret_cast<_Float16 *>(a.y) + (size_t)row * a.ldy, true, a.d, lane);
    else
        store_row(y, reinterpret_cast<float *>(a.y) + (size_t)row * a.ldy, false, a.d, lane);
}

// y[c] *= v[c] (+ add) for the row slots of this lane
template <int NV>
__device__ __forceinline__ void mul_cols(Row<NV> &y, const float *v, float add, int d, int lane) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int c = (i * 64 + lane) * 4;
        const f32x4 m = c < d ? ld4(v + c) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; e++) y.v[i][e] *= m[e] + add;
    }
}

template <int NV, bool F16>
__global__ __launch_bounds__(256) void add_norm_kernel(AddNormArgs a) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= (int)a.rows) return;
    const size_t off = (size_t)row * a.d;
    Row<NV> h;
    load_row(h, a.h + off, a.d, lane);
    if (a.t) {
        Row<NV> t;
        load_row(t, a.t + off, a.d, lane);
        const float inv_t = rms_inv(t, a.d, a.eps);
        Row<NV> tn = rms_apply(t, inv_t, a.w_post, a.d, lane);
        if (a.gate) mul_cols(tn, a.gate, 0.0f, a.d, lane);
#pragma unroll
        for (int i = 0; i < NV; i++) h.v[i] = (h.v[i] + tn.v[i]) * a.post;  // exact when post == 1
        store_row(h, a.h + off, false, a.d, lane);
    }
    if (a.w_next) {
        const float inv_h = rms_inv(h, a.d, a.eps);
        Row<NV> y = rms_apply(h, inv_h, a.w_next, a.d, lane);
        if (a.scale) mul_cols(y, a.scale, 1.0f, a.d, lane);  // adaLN: times (1 + s)
        // copy z = y col_z oscale.  A column row is loaded whole before the
        // first store: loads placed after stores the compiler cannot prove
        // disjoint would each wait for the one before (h is dead by now, so
        // the extra register row raises no peak).  The copies with and
        // without a column row take separate store loops, so the stores of
        // the plain copy carry no wait for column loads.
        auto put = [&](size_t zo, const Row<NV> &v) {
            if (F16)
                store_row(v, reinterpret_cast<_Float16 *>(a.a) + zo, true, a.d, lane);
            else
                store_row(v, reinterpret_cast<float *>(a.a) + zo, false, a.d, lane);
        };
        for (uint32_t z = 0; z < a.nout; z++) {
            const float *col = a.col[z];
            const size_t zo = off + z * a.a_stride;
            Row<NV> v;
            if (col) {
                load_row(v, col, a.d, lane);
#pragma unroll
                for (int i = 0; i < NV; i++)
#pragma unroll
                    for (int e = 0; e < 4; e++) v.v[i][e] = y.v[i][e] * v.v[i][e] * a.oscale;
            } else {
#pragma unroll
                for (int i = 0; i < NV; i++)
#pragma unroll
                    for (int e = 0; e < 4; e++) v.v[i][e] = y.v[i][e] * a.oscale;  // a power of two: exact
            }
            put(zo, v);
        }
    }
}

// A row's nq q heads and nkv k heads (and, with v_norm, its nkv v heads:
// weightless RMS, no rotation) are split into groups of a few passes, one wave
// per (row, group).  A head is held by
// LH = hd / VE lanes, each owning VE consecutive channels (one 16-byte vector:
// 4 f32 or 8 f16), so a wave covers 64 / LH heads per pass with fully
// coalesced loads.  The per-head RMS is a butterfly inside the LH-lane group;
// the rotate_half partner of channel c (c +- S/2) sits (S/2)/VE lanes away, in
// the same vector slot.  A lane's channels are the same in every head, so its
// norm gains and cos/sin are loaded once; the next pass's vector is loaded
// before the current one is processed.
template <int HD, bool F16>
__device__ __forceinline__ void qk_load(const QkArgs &a, uint32_t row, uint32_t col, int c0, bool valid,
                                        float (&x)[F16 ? 8 : 4]) {
    constexpr int VE = F16 ? 8 : 4;
    if (!valid) {
#pragma unroll
        for (int e = 0; e < VE; e++) x[e] = 0.0f;
    } else if (F16) {
        const f16x8 v = *reinterpret_cast<const f16x8 *>(
            reinterpret_cast<const _Float16 *>(a.panel) + (size_t)row * a.ld + col + c0);
#pragma unroll
        for (int e = 0; e < VE; e++) x[e] = (float)v[e % 8];
    } else {
        const f32x4 v = ld4(reinterpret_cast<const float *>(a.panel) + (size_t)row * a.ld + col + c0);
#pragma unroll
        for (int e = 0; e < VE; e++) x[e] = v[e % 4];
    }
}

template <int HD, bool F16>
__device__ __forceinline__ void qk_store(const QkArgs &a, uint32_t row, uint32_t col, int c0,
                                         const float (&x)[F16 ? 8 : 4]) {
    constexpr int VE = F16 ? 8 : 4;
    if (F16) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] = (_Float16)x[e % VE];
        *reinterpret_cast<f16x8 *>(reinterpret_cast<_Float16 *>(a.panel) + (size_t)row * a.ld + col + c0) = v;
    } else {
        st4(reinterpret_cast<float *>(a.panel) + (size_t)row * a.ld + col + c0,
            f32x4{x[0], x[1 % VE], x[2 % VE], x[3 % VE]});
    }
}

// The launch splits a row's passes into gridDim.y groups only when rows alone
// give fewer waves than this (extra groups reload the gains and cos/sin, which
// costs at large row counts).  Every head is normed and rotated by one wave
// whatever the grouping, so the grouping changes no bit.
constexpr uint32_t kQkWaveTarget = 8192;

template <int HD, bool F16>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(QkArgs a) {
    constexpr int VE = F16 ? 8 : 4;
    constexpr int LH = HD / VE;   // lanes per head
    constexpr int HP = 64 / LH;   // heads per pass
    const uint32_t row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.rows) return;
    const int hsub = lane / LH, c0 = (lane % LH) * VE;
    const int S = a.sections ? HD / (int)a.sections : HD, half = S / 2;
    const int s_idx = c0 / S, i0 = c0 % S;
    const bool first = i0 < half;
    const int ti = s_idx * half + (first ? i0 : i0 - half);
    const int pmask = half / VE;  // partner lane distance (power of two)
    float cs[VE], sn[VE], wq[VE], wk[VE];
    if (a.sections) {
        const float *cp = a.cos + (size_t)row * (HD / 2) + ti;
        const float *sp = a.sin + (size_t)row * (HD / 2) + ti;
#pragma unroll
        for (int e = 0; e < VE; e++) {
            cs[e] = cp[e];
            sn[e] = sp[e];
        }
    }
#pragma unroll
    for (int e = 0; e < VE; e++) {
        wq[e] = a.qw[c0 + e];
        wk[e] = a.kw[c0 + e];
    }
    // heads in order: q, k, then (v_norm) v; group g of HP heads is one pass
    const uint32_t nqk = a.nq + a.nkv, heads = nqk + (a.v_norm ? a.nkv : 0);
    auto col_of = [&](uint32_t hh) -> uint32_t {
        return hh < a.nq ? a.q_col + hh * HD
                         : hh < nqk ? a.k_col + (hh - a.nq) * HD : a.v_col + (hh - nqk) * HD;
    };
    // this wave's heads: group blockIdx.y of gridDim.y, whole passes each
    const uint32_t npass = (heads + HP - 1) / HP, gp = (npass + gridDim.y - 1) / gridDim.y;
    const uint32_t hbeg = blockIdx.y * gp * HP, hend = min(heads, hbeg + gp * HP);
    float xn[VE];
    qk_load<HD, F16>(a, row, col_of(hbeg + hsub), c0, hbeg + hsub < hend, xn);
    for (uint32_t h0 = hbeg; h0 < hend; h0 += HP) {
        const uint32_t hh = h0 + hsub;
        const bool valid = hh < hend, isv = hh >= nqk;
        float x[VE];
#pragma unroll
        for (int e = 0; e < VE; e++) x[e] = xn[e];
        if (h0 + HP < hend) qk_load<HD, F16>(a, row, col_of(hh + HP), c0, hh + HP < hend, xn);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < VE; e++) ss = fmaf(x[e], x[e], ss);
#pragma unroll
        for (int o = LH / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
        const float inv = 1.0f / sqrtf(ss / (float)HD + a.eps);
        const bool isq = hh < a.nq;
#pragma unroll
        for (int e = 0; e < VE; e++) x[e] = isv ? x[e] * inv : x[e] * inv * (isq ? wq[e] : wk[e]);
        if (a.sections) {
            // every lane takes part in the exchange; v heads keep their value
            float y[VE];
#pragma unroll
            for (int e = 0; e < VE; e++) {
                const float xp = __shfl_xor(x[e], pmask, 64);
                y[e] = first ? x[e] * cs[e] - xp * sn[e] : x[e] * cs[e] + xp * sn[e];
            }
            if (!isv)
#pragma unroll
                for (int e = 0; e < VE; e++) x[e] = y[e];
        }
        if (valid) qk_store<HD, F16>(a, row, col_of(hh), c0, x);
    }
}

template <bool F16>
__global__ __launch_bounds__(256) void gated_act_kernel(ActArgs a) {
    const uint32_t q = a.ff / 4;
    const size_t total = (size_t)a.rows * q;
    for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * 256) {
        const size_t r = idx / q;
        const uint32_t c = (uint32_t)(idx % q) * 4;
        const f32x4 g = ld4(a.g + r * a.ldg + c), u = ld4(a.u + r * a.ldu + c);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = (a.kind == 1 ? gelu_tanh(g[e]) : silu(g[e])) * u[e];
        if (a.ocol) {
            const f32x4 m = ld4(a.ocol + c);
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] *= m[e];
        }
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] *= a.oscale;
        if (F16)
            st4h(reinterpret_cast<_Float16 *>(a.out) + r * a.ldo + c, o);
        else
            st4(reinterpret_cast<float *>(a.out) + r * a.ldo + c, o);
    }
}

// out[i][j] = mean over item i's rows of a[r][j].  A block takes one item and
// 64 columns; wave w of 16 sums rows t = w, w+16, ... in that order (lane =
// column, coalesced 256-byte loads, eight rows in flight per lane), and the 16
// partial sums are added in wave order: deterministic, and independent of the
// other items.
__global__ __launch_bounds__(1024) void mean_pool_kernel(PoolArgs a) {
    constexpr int NWV = 16, U = 8;  // waves per block; rows in flight per lane
    __shared__ float part[NWV][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t j = blockIdx.x * 64 + lane;
    // items beyond the grid's y extent (65 535) are taken in grid-stride order
    for (uint32_t i = blockIdx.y; i < a.nitems; i += gridDim.y) {
        const AttnItemK it = a.items[i];
        const uint32_t L = it.na + it.nb;
        float s = 0.0f;
        if (j < a.d) {
            // wave w sums rows w, w + 16, w + 32, ... in that order, U loads at a time
            for (uint32_t t0 = wave; t0 < L; t0 += NWV * U) {
                float v[U];
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const uint32_t t = t0 + NWV * u;
                    const uint32_t r = t < it.na ? it.r0a + t : it.r0b + (t - it.na);
                    v[u] = t < L ? a.a[(size_t)r * a.d + j] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < U; u++)
                    if (t0 + NWV * u < L) s += v[u];
            }
        }
        part[wave][lane] = s;
        __syncthreads();
        if (wave == 0 && j < a.d) {
            float tot = part[0][lane];
#pragma unroll
            for (int w = 1; w < NWV; w++) tot += part[w][lane];
            a.out[(size_t)i * a.d + j] = tot / (float)L;
        }
        __syncthreads();
    }
}

// Max |x| of a half buffer: pass 1 (blocks of 256) writes one maximum per
// block, pass 2 (one block) reduces them.  Max is order-free: deterministic.
__global__ __launch_bounds__(256) void amax_part_kernel(AmaxArgs a) {
    __shared__ float red[4];
    float m = 0.0f;
    const uint64_t n8 = a.n / 8;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (uint64_t)gridDim.x * 256) {
        const f16x8 v = reinterpret_cast<const f16x8 *>(a.x)[i];
#pragma unroll
        for (int e = 0; e < 8; e++) m = fmaxf(m, fabsf((float)v[e]));
    }
    for (uint64_t i = n8 * 8 + (uint64_t)blockIdx.x * 256 + threadIdx.x; i < a.n; i += (uint64_t)gridDim.x * 256)
        m = fmaxf(m, fabsf((float)a.x[i]));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) a.part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void amax_final_kernel(AmaxArgs a) {
    __shared__ float red[4];
    float m = 0.0f;
    for (uint32_t i = threadIdx.x; i < a.blocks; i += 256) m = fmaxf(m, a.part[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) *a.out = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

}  // namespace

// NV = ceil(d / 256) float4 slots per lane, d <= 4096.
#define ENC_NV_SWITCH(nv, CALL)                                                                  \
    switch (nv) {                                                                                \
    case 1: CALL(1); break;                                                                      \
    case 2: CALL(2); break;                                                                      \
    case 3: CALL(3); break;                                                                      \
    case 4: CALL(4); break;                                                                      \
    case 5: CALL(5); break;                                                                      \
    case 6: CALL(6); break;                                                                      \
    case 7: CALL(7); break;                                                                      \
    case 8: CALL(8); break;                                                                      \
    case 9: CALL(9); break;                                                                      \
    case 10: CALL(10); break;                                                                    \
    case 11: CALL(11); break;                                                                    \
    case 12: CALL(12); break;                                                                    \
    case 13: CALL(13); break;                                                                    \
    case 14: CALL(14); break;                                                                    \
    case 15: CALL(15); break;                                                                    \
    case 16: CALL(16); break;                                                                    \
    default: return hipErrorInvalidValue;                                                        \
    }

hipError_t launch_rms_norm(const NormArgs &a, bool f16, hipStream_t s) {
    if (!a.rows) return hipSuccess;
    const dim3 grid((a.rows + 3) / 4);
#define L(N)                                                                                     \
    if (f16) hipLaunchKernelGGL((rms_norm_kernel<N, true>), grid, dim3(256), 0, s, a);           \
    else hipLaunchKernelGGL((rms_norm_kernel<N, false>), grid, dim3(256), 0, s, a);
    ENC_NV_SWITCH((a.d + 255) / 256, L)
#undef L
    return hipGetLastError();
}

hipError_t launch_layer_norm(const NormArgs &a, bool f16, hipStream_t s) {
    if (!a.rows) return hipSuccess;
    const dim3 grid((a.rows + 3) / 4);
#define L(N)                                                                                     \
    if (f16) hipLaunchKernelGGL((layer_norm_kernel<N, true>), grid, dim3(256), 0, s, a);         \
    else hipLaunchKernelGGL((layer_norm_kernel<N, false>), grid, dim3(256), 0, s, a);
    ENC_NV_SWITCH((a.d + 255) / 256, L)
#undef L
    return hipGetLastError();
}

hipError_t launch_add_norm(const AddNormArgs &a, bool f16, hipStream_t s) {
    if (!a.rows) return hipSuccess;
    const dim3 grid((a.rows + 3) / 4);
#define L(N)                                                                                     \
    if (f16) hipLaunchKernelGGL((add_norm_kernel<N, true>), grid, dim3(256), 0, s, a);           \
    else hipLaunchKernelGGL((add_norm_kernel<N, false>), grid, dim3(256), 0, s, a);
    ENC_NV_SWITCH((a.d + 255) / 256, L)
#undef L
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const QkArgs &a, bool f16, hipStream_t s) {
    if (!a.rows || !(a.nq + a.nkv)) return hipSuccess;
    const uint32_t heads = a.nq + a.nkv + (a.v_norm ? a.nkv : 0);
    const uint32_t hp = 64 / (a.hd / (f16 ? 8 : 4));  // heads per pass
    const uint32_t npass = (heads + hp - 1) / hp;
    const uint32_t want = std::min(npass, std::max(1u, (kQkWaveTarget + a.rows - 1) / a.rows));
    const uint32_t gp = (npass + want - 1) / want;  // passes per group; no group is empty
    const dim3 grid((a.rows + 3) / 4, (npass + gp - 1) / gp);
    if (a.hd == 64) {
        if (f16) hipLaunchKernelGGL((qk_norm_rope_kernel<64, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((qk_norm_rope_kernel<64, false>), grid, dim3(256), 0, s, a);
    } else {
        if (f16) hipLaunchKernelGGL((qk_norm_rope_kernel<128, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((qk_norm_rope_kernel<128, false>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gated_act(const ActArgs &a, bool f16, hipStream_t s) {
    const size_t total = (size_t)a.rows * (a.ff / 4);
    if (!total) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 256 * 64);
    if (f16) hipLaunchKernelGGL(gated_act_kernel<true>, dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gated_act_kernel<false>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_amax_f16(const AmaxArgs &a, hipStream_t s) {
    if (!a.n || !a.blocks) return hipErrorInvalidValue;
    hipLaunchKernelGGL(amax_part_kernel, dim3(a.blocks), dim3(256), 0, s, a);
    hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_mean_pool(const PoolArgs &a, hipStream_t s) {
    if (!a.nitems || !a.d) return hipSuccess;
    hipLaunchKernelGGL(mean_pool_kernel, dim3((a.d + 63) / 64, a.nitems < 65535u ? a.nitems : 65535u), dim3(1024),
                       0, s, a);
    return hipGetLastError();
}

}  // namespace enc
