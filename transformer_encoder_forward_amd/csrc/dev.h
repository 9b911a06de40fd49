// Device-side helpers for gfx950 (CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace enc {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Butterfly sum over the 64 lanes; every lane ends with the same bits (each
// lane adds the same pairs, only commuted).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// tanh(u) = sign(u) (1 - e) / (1 + e), e = exp(-2|u|): no cancellation for
// small |u| beyond the f32 rounding of e.  The divisor lies in (1, 2], so the
// quotient is taken as a product with the hardware reciprocal (within 1 ulp)
// instead of the IEEE division sequence.
__device__ __forceinline__ float tanh_f32(float u) {
    float e = __expf(-2.0f * fabsf(u));
    float t = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    return copysignf(t, u);
}

// GELU, tanh approximation: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
__device__ __forceinline__ float gelu_tanh(float x) {
    const float c = 0.7978845608028654f;
    return 0.5f * x * (1.0f + tanh_f32(c * (x + 0.044715f * x * x * x)));
}

// silu(x) = x / (1 + exp(-x)); the divisor lies in (1, inf].  Up to 2^126 the
// hardware reciprocal is within 1 ulp; beyond (x below about -87.3) the
// reciprocal is subnormal and may flush to 0, so silu gives -0 where the exact
// value is under 2^-120 in magnitude (and 0 at inf, as the division gives).
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }

__device__ __forceinline__ f32x4 ld4h(const _Float16 *p) {
    f16x4 h = *reinterpret_cast<const f16x4 *>(p);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
__device__ __forceinline__ void st4h(_Float16 *p, f32x4 v) {
    f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<f16x4 *>(p) = h;
}

// ---- LDS staging by direct global -> LDS loads, and LDS reads the compiler
// does not track.  A global_load_lds_dwordx4 writes 64 lanes x 16 bytes to 1 KB
// of consecutive LDS from the wave-uniform address it is given.  The compiler
// would wait for every such load in flight before any LDS read it can see, so
// kernels that keep loads in flight across their reads issue those reads in
// inline assembly and wait for them with explicit counters.
#define ENC_GLOBAL(p) ((const void __attribute__((address_space(1))) *)(p))
#define ENC_SHARED(p) ((void __attribute__((address_space(3))) *)(p))

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)ENC_SHARED(const_cast<void *>(p));
}

// A direct load through a raw buffer: 16 bytes per lane from byte voff +
// soff of the buffer into 1 KB of LDS at the wave-uniform lds.  The stage
// offset soff and the LDS address stay in scalar registers.  (The host pass
// of a kernel template does not take this builtin; only the device pass
// compiles the call.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ void buffer_dma16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ENC_SHARED(lds), 16, voff, soff, 0, 0);
#else
    (void)r, (void)lds, (void)voff, (void)soff;
#endif
}

__device__ __forceinline__ void dma16(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(ENC_GLOBAL(src), ENC_SHARED(lds_wave_base), 16, 0, 0);
}

__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// LDS reads at a base address plus an immediate byte offset (0..65535).
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16_at(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset");
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
    return v;
}

// N reads at OFF, OFF + STRIDE, ... into d[0..N).
template <int OFF, int STRIDE, int N>
__device__ __forceinline__ void ds_read16_run(u32x4 *d, uint32_t addr) {
    if constexpr (N > 0) {
        d[0] = ds_read16_at<OFF>(addr);
        ds_read16_run<OFF + STRIDE, STRIDE, N - 1>(d + 1, addr);
    }
}

// Transposing 64-bit read of 16-bit data: within each group of 16 lanes, lane i
// receives element i % 4 of the four 64-bit rows addressed by lanes i/4 + 4e,
// e = 0..3 (the layout measured on gfx950).
__device__ __forceinline__ u32x2 ds_read8_tr16(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

template <int OFF>
__device__ __forceinline__ u32x2 ds_read8_tr16_at(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset");
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
    return v;
}

// A compile-time integer as a value (stage indices of unrolled loops).
template <int V>
using IC = std::integral_constant<int, V>;

// Wait until at most N LDS reads (of this wave) are in flight.  The registers
// the reads filled are then passed through empty asm statements (see `ready`):
// volatile asm keeps its order, so no use of them moves above the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait_n() {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
template <typename T>
__device__ __forceinline__ void ready(T &v) {
    asm volatile("" : "+v"(v));
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    // s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt low bits
    // [3:0] and high bits [15:14], expcnt [6:4], lgkmcnt [11:8] at maximum)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace enc
