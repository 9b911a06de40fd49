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

template <int NV, bool F16>
__global__ __launch_bounds__(256) void add_norm_kernel(AddNormArgs a) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= (int)a.rows) return;
    const size_t off = (size_t)row * a.d;
    Row<NV> t, h;
    load_row(t, a.t + off, a.d, lane);
    load_row(h, a.h + off, a.d, lane);
    const float inv_t = rms_inv(t, a.d, a.eps);
    const Row<NV> tn = rms_apply(t, inv_t, a.w_post, a.d, lane);
#pragma unroll
    for (int i = 0; i < NV; i++) h.v[i] += tn.v[i];
    store_row(h, a.h + off, false, a.d, lane);
    if (a.w_next) {
        const float inv_h = rms_inv(h, a.d, a.eps);
        const Row<NV> y = rms_apply(h, inv_h, a.w_next, a.d, lane);
        if (F16)
            store_row(y, reinterpret_cast<_Float16 *>(a.a) + off, true, a.d, lane);
        else
            store_row(y, reinterpret_cast<float *>(a.a) + off, false, a.d, lane);
    }
}

// One wave per (row, head) over the nq q heads then the nkv k heads; lane owns
// E = hd/64 consecutive channels.  The rotate_half partner of channel c is
// c +- S/2, held by lane ^ (S/2/E) in the same slot.
template <int HD, bool F16>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(QkArgs a) {
    constexpr int E = HD / 64;
    const uint32_t heads = a.nq + a.nkv;
    const uint32_t unit = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (unit >= a.rows * heads) return;
    const uint32_t row = unit / heads, hh = unit % heads;
    const bool isq = hh < a.nq;
    const uint32_t col = isq ? a.q_col + hh * HD : a.k_col + (hh - a.nq) * HD;
    const float *w = isq ? a.qw : a.kw;
    const int c0 = lane * E;
    float x[E];
    if (F16) {
        const _Float16 *p = reinterpret_cast<const _Float16 *>(a.panel) + (size_t)row * a.ld + col + c0;
#pragma unroll
        for (int e = 0; e < E; e++) x[e] = (float)p[e];
    } else {
        const float *p = reinterpret_cast<const float *>(a.panel) + (size_t)row * a.ld + col + c0;
#pragma unroll
        for (int e = 0; e < E; e++) x[e] = p[e];
    }
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < E; e++) ss = fmaf(x[e], x[e], ss);
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)HD + a.eps);
#pragma unroll
    for (int e = 0; e < E; e++) x[e] = x[e] * inv * w[c0 + e];
    if (a.sections) {
        const int S = HD / (int)a.sections, half = S / 2;
        const int mask = half / E;
        const float *cs = a.cos + (size_t)row * (HD / 2);
        const float *sn = a.sin + (size_t)row * (HD / 2);
        float y[E];
#pragma unroll
        for (int e = 0; e < E; e++) {
            const float xp = __shfl_xor(x[e], mask, 64);
            const int c = c0 + e, s = c / S, i = c % S;
            const bool first = i < half;
            const int ti = s * half + (first ? i : i - half);
            const float cv = cs[ti], sv = sn[ti];
            y[e] = first ? x[e] * cv - xp * sv : x[e] * cv + xp * sv;
        }
#pragma unroll
        for (int e = 0; e < E; e++) x[e] = y[e];
    }
    if (F16) {
        _Float16 *p = reinterpret_cast<_Float16 *>(a.panel) + (size_t)row * a.ld + col + c0;
#pragma unroll
        for (int e = 0; e < E; e++) p[e] = (_Float16)x[e];
    } else {
        float *p = reinterpret_cast<float *>(a.panel) + (size_t)row * a.ld + col + c0;
#pragma unroll
        for (int e = 0; e < E; e++) p[e] = x[e];
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
        if (F16)
            st4h(reinterpret_cast<_Float16 *>(a.out) + r * a.ldo + c, o);
        else
            st4(reinterpret_cast<float *>(a.out) + r * a.ldo + c, o);
    }
}

// out[i][j] = mean over item i's rows of a[r][j]; one thread per column, rows
// summed in order (deterministic).
__global__ __launch_bounds__(256) void mean_pool_kernel(PoolArgs a) {
    const uint32_t j = blockIdx.x * 256 + threadIdx.x, i = blockIdx.y;
    if (j >= a.d || i >= a.nitems) return;
    const AttnItemK it = a.items[i];
    float s = 0.0f;
    for (uint32_t t = 0; t < it.na; t++) s += a.a[(size_t)(it.r0a + t) * a.d + j];
    for (uint32_t t = 0; t < it.nb; t++) s += a.a[(size_t)(it.r0b + t) * a.d + j];
    a.out[(size_t)i * a.d + j] = s / (float)(it.na + it.nb);
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
    const size_t units = (size_t)a.rows * (a.nq + a.nkv);
    if (!units) return hipSuccess;
    const dim3 grid((unsigned)((units + 3) / 4));
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

hipError_t launch_mean_pool(const PoolArgs &a, hipStream_t s) {
    if (!a.nitems || !a.d) return hipSuccess;
    hipLaunchKernelGGL(mean_pool_kernel, dim3((a.d + 255) / 256, a.nitems), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace enc
