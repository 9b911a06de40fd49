// Item-table batched GEMM Y = epi(alpha * X W^T) on gfx950 MFMA.
//
// What it computes: egemma2.rs (cortiq-engine 0.8.39), module doc "GEMM" and
// `EgMm` (one item per grid z: q/k/v in one launch, gate/up in another);
// zimage.rs (cortiq-engine 0.7.6), module doc "The chain" and `PMm` (int8
// weight rows used exactly as half, per-output-row scale in an f32 epilogue).
//
// Design for CDNA4 (not the pages' 64x64 simdgroup tile): a 256-thread block
// owns a 128 x 128 output tile; its 4 waves form a 2 x 2 grid of 64 x 64 wave
// tiles, each 2 x 2 MFMA 32x32 accumulator blocks.  X and W tiles are staged
// through double-buffered LDS with one barrier per K stage; the next stage's
// global loads are issued before the current stage's MFMAs.  Inside a stage a
// lane's two halves own disjoint K sub-ranges, so every fragment read is a run
// of contiguous LDS words (ds_read_b128).  The K order of every output element
// depends only on K, never on the row count, so packed and separate batches
// give the same bits.
//  - f32 path: v_mfma_f32_32x32x2_f32, K stage 32.
//  - int8 path: W tiles are widened int8 -> f16 (exact) while being staged,
//    X is f16; v_mfma_f32_32x32x16_f16, K stage 64, f32 accumulation.
// Blocks are renumbered so that each XCD (round-robin block dispatch) owns a
// contiguous run of tiles, which share X row blocks and W panels in its L2.
#include "dev.h"
#include "kern.h"

namespace enc {

namespace {

constexpr int BM = kGemmBM, BN = kGemmBN;

__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t G) {
    uint32_t x = b & 7u, j = b >> 3, q = G >> 3, r = G & 7u;
    return x * q + min(x, r) + j;
}

struct TileCtx {
    GemmItemK it;
    const void *w;
    const float *rs;
    const float *bias;
    int row0, col0;
};

__device__ __forceinline__ bool locate(const GemmArgs &a, TileCtx &t) {
    uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
    if (tile >= a.total_tiles) return false;
    int sel = 0;
#pragma unroll
    for (int i = 1; i < kMaxGemmItems; i++)
        if (i < (int)a.nitems && tile >= a.items[i].tile0) sel = i;
    t.it = a.items[0];
#pragma unroll
    for (int i = 1; i < kMaxGemmItems; i++)
        if (sel == i) t.it = a.items[i];
    t.w = a.w[0];
    t.rs = a.rs[0];
    t.bias = a.bias[0];
#pragma unroll
    for (int s = 1; s < kMaxGemmItems; s++)
        if ((int)t.it.slot == s) {
            t.w = a.w[s];
            t.rs = a.rs[s];
            t.bias = a.bias[s];
        }
    uint32_t local = tile - t.it.tile0;
    t.row0 = (int)(local / t.it.tiles_m) * BM;
    t.col0 = (int)(local % t.it.tiles_m) * BN;
    return true;
}

// Epilogue for one 32x32 accumulator block: D[i][j] of lane l, register r sits
// at i = 8*(r/4) + 4*(l/32) + r%4, j = l%32.
template <bool I8>
__device__ __forceinline__ void store_block(const GemmArgs &a, const TileCtx &t, const f32x16 &acc,
                                            int rbase, int cbase, int lane) {
    const int li = lane & 31, hf = lane >> 5;
    const int c = cbase + li;
    if (c >= (int)t.it.m) return;
    float mul = a.alpha;
    if (I8) mul *= t.rs[c];
    const float b = t.bias ? t.bias[c] : 0.0f;
    const bool f16 = a.flags & 1u, accum = a.flags & 2u, gelu = a.flags & 4u;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int row = rbase + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (row >= (int)t.it.n) continue;
        float v = acc[r] * mul + b;
        if (gelu) v = gelu_tanh(v);
        const size_t off = t.it.y_off + (size_t)row * t.it.ldy + c;
        if (f16) {
            reinterpret_cast<_Float16 *>(a.y)[off] = (_Float16)v;
        } else {
            float *y = reinterpret_cast<float *>(a.y) + off;
            *y = accum ? *y + v : v;
        }
    }
}

// ------------------------------------------------------------------- f32 path

constexpr int BK32 = 32;
constexpr int LDS32 = BK32 + 4;  // padded row, floats

__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) float As[2][BM][LDS32];
    __shared__ __attribute__((aligned(16))) float Bs[2][BN][LDS32];
    TileCtx t;
    if (!locate(a, t)) return;
    const int n = t.it.n, m = t.it.m, K = t.it.k;
    const float *X = reinterpret_cast<const float *>(a.x) + t.it.x_off;
    const float *W = reinterpret_cast<const float *>(t.w);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5, wr = wave >> 1, wc = wave & 1;

    // global -> register staging: thread loads 4 float4 of each tile
    f32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int f = tid + 256 * i, r = f >> 3, c = (f & 7) * 4;
            const int gk = k0 + c, gr = t.row0 + r, gc = t.col0 + r;
            ra[i] = (gr < n && gk < K) ? ld4(X + (size_t)gr * t.it.ldx + gk) : f32x4{0, 0, 0, 0};
            rb[i] = (gc < m && gk < K) ? ld4(W + (size_t)gc * K + gk) : f32x4{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int f = tid + 256 * i, r = f >> 3, c = (f & 7) * 4;
            st4(&As[buf][r][c], ra[i]);
            st4(&Bs[buf][r][c], rb[i]);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nst = (K + BK32 - 1) / BK32;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int s = 0; s < nst; s++) {
        const int buf = s & 1;
        if (s + 1 < nst) gload((s + 1) * BK32);
        // lane half hf owns k = 16*hf + 0..15 of this stage
        f32x4 fa[2][4], fb[2][4];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                fa[i][q] = ld4(&As[buf][wr * 64 + i * 32 + li][16 * hf + 4 * q]);
                fb[i][q] = ld4(&Bs[buf][wc * 64 + i * 32 + li][16 * hf + 4 * q]);
            }
#pragma unroll
        for (int kk = 0; kk < 16; kk++)
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        fa[i][kk >> 2][kk & 3], fb[j][kk >> 2][kk & 3], acc[i][j], 0, 0, 0);
        if (s + 1 < nst) sstore(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            store_block<false>(a, t, acc[i][j], t.row0 + wr * 64 + i * 32, t.col0 + wc * 64 + j * 32,
                               lane);
}

// ------------------------------------------------------------ int8 x f16 path

constexpr int BK16 = 64;
constexpr int LDS16 = BK16 + 8;  // padded row, halves

// 16 int8 -> 16 f16, exact.
__device__ __forceinline__ void widen16(const int32_t w[4], f16x8 &lo, f16x8 &hi) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
        lo[e] = (_Float16)(float)(int8_t)(w[e >> 2] >> (8 * (e & 3)));
        hi[e] = (_Float16)(float)(int8_t)(w[2 + (e >> 2)] >> (8 * (e & 3)));
    }
}

__global__ __launch_bounds__(256, 2) void gemm_i8f16_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM][LDS16];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN][LDS16];
    TileCtx t;
    if (!locate(a, t)) return;
    const int n = t.it.n, m = t.it.m, K = t.it.k;
    const _Float16 *X = reinterpret_cast<const _Float16 *>(a.x) + t.it.x_off;
    const int8_t *W = reinterpret_cast<const int8_t *>(t.w);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5, wr = wave >> 1, wc = wave & 1;

    // X tile: 128 rows x 64 halves = 1024 chunks of 8 halves, 4 per thread.
    // W tile: 128 rows x 64 int8 = 512 chunks of 16 bytes, 2 per thread.
    f16x8 ra[4];
    int32_t rb[2][4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int f = tid + 256 * i, r = f >> 3, c = (f & 7) * 8;
            const int gk = k0 + c, gr = t.row0 + r;
            if (gr < n && gk < K)
                ra[i] = *reinterpret_cast<const f16x8 *>(X + (size_t)gr * t.it.ldx + gk);
            else
                ra[i] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int f = tid + 256 * i, r = f >> 2, c = (f & 3) * 16;
            const int gk = k0 + c, gc = t.col0 + r;
            if (gc < m && gk < K) {
                const int32_t *p = reinterpret_cast<const int32_t *>(W + (size_t)gc * K + gk);
                rb[i][0] = p[0];
                rb[i][1] = p[1];
                rb[i][2] = p[2];
                rb[i][3] = p[3];
            } else {
                rb[i][0] = rb[i][1] = rb[i][2] = rb[i][3] = 0;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int f = tid + 256 * i, r = f >> 3, c = (f & 7) * 8;
            *reinterpret_cast<f16x8 *>(&As[buf][r][c]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int f = tid + 256 * i, r = f >> 2, c = (f & 3) * 16;
            f16x8 lo, hi;
            widen16(rb[i], lo, hi);
            *reinterpret_cast<f16x8 *>(&Bs[buf][r][c]) = lo;
            *reinterpret_cast<f16x8 *>(&Bs[buf][r][c + 8]) = hi;
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nst = (K + BK16 - 1) / BK16;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int s = 0; s < nst; s++) {
        const int buf = s & 1;
        if (s + 1 < nst) gload((s + 1) * BK16);
        // lane half hf owns k = 32*hf + 0..31 of this stage, 8 per MFMA step
        f16x8 fa[2][4], fb[2][4];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                fa[i][q] = *reinterpret_cast<const f16x8 *>(&As[buf][wr * 64 + i * 32 + li][32 * hf + 8 * q]);
                fb[i][q] = *reinterpret_cast<const f16x8 *>(&Bs[buf][wc * 64 + i * 32 + li][32 * hf + 8 * q]);
            }
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i][q], fb[j][q], acc[i][j],
                                                                       0, 0, 0);
        if (s + 1 < nst) sstore(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            store_block<true>(a, t, acc[i][j], t.row0 + wr * 64 + i * 32, t.col0 + wc * 64 + j * 32,
                              lane);
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s) {
    if (a.total_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(a.total_tiles), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_i8f16(const GemmArgs &a, hipStream_t s) {
    if (a.total_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_i8f16_kernel, dim3(a.total_tiles), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace enc
