// MFMA issue-rate probe: 4 independent 32x32 accumulators per wave, operands
// in registers (random, rotating), no memory traffic inside the loop.  The measured rate is the
// ceiling the GEMM and attention kernels are compared with next to the
// datasheet peak (zimage.rs, cortiq-engine 0.7.6, `bench_mma_peak`: a pure
// simdgroup-MMA loop with 16 independent accumulators).
#include "dev.h"
#include "kern.h"

namespace enc {

namespace {

// Operands differ per lane and per MFMA (four operand pairs in rotation), so the
// multipliers switch the way they do on real data: with constant operands the
// chip draws less power and holds a higher clock than any GEMM can.
__device__ __forceinline__ uint32_t xorshift(uint32_t &h) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return h;
}

__global__ __launch_bounds__(256) void peak_f32_kernel(float *out, uint32_t iters, float seed) {
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][r] = 0.0f;
    uint32_t h = (threadIdx.x + 1) * 2654435761u ^ (blockIdx.x * 40503u + 12345u);
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        a[i] = seed * (float)((int)(xorshift(h) % 255u) - 127);
        b[i] = seed * (float)((int)(xorshift(h) % 255u) - 127);
    }
    for (uint32_t it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[(i + j) & 3], b[i], acc[i], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[i][r];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void peak_f16_kernel(float *out, uint32_t iters, float seed) {
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][r] = 0.0f;
    uint32_t h = (threadIdx.x + 1) * 2654435761u ^ (blockIdx.x * 40503u + 12345u);
    f16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            a[i][e] = (_Float16)(seed * (float)((int)(xorshift(h) % 255u) - 127));
            b[i][e] = (_Float16)(seed * (float)((int)(xorshift(h) % 255u) - 127));
        }
    for (uint32_t it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(i + j) & 3], b[i], acc[i], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[i][r];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// flops of one launch: blocks * 4 waves * iters * 16 MFMAs * (32*32*K*2)
hipError_t launch_mfma_peak(bool f16, uint32_t blocks, uint32_t iters, float *out, hipStream_t s) {
    if (f16)
        hipLaunchKernelGGL(peak_f16_kernel, dim3(blocks), dim3(256), 0, s, out, iters, 1.0f / 64);
    else
        hipLaunchKernelGGL(peak_f32_kernel, dim3(blocks), dim3(256), 0, s, out, iters, 1.0f / 64);
    return hipGetLastError();
}

}  // namespace enc
