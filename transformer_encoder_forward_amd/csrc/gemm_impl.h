// Item-table batched GEMM Y = epi(alpha * X W^T) on gfx950 MFMA: the kernel
// template (the launcher in gemm.hip picks the instantiation per shape).
//
// What it computes: egemma2.rs (cortiq-engine 0.8.39), module doc "GEMM" and
// `EgMm` (one item per grid z: q/k/v in one launch, gate/up in another);
// zimage.rs (cortiq-engine 0.7.6), module doc "The chain" and `PMm` (int8
// weight rows used exactly as half, per-output-row scale in an f32 epilogue).
//
// Design for CDNA4: a block of WGM x WGN waves owns a BM x BN output tile; each
// wave owns (BM/WGM) x (BN/WGN) = FM x FN accumulator blocks of 32 x 32.  X and
// W tiles of BK columns reach LDS either through registers (gemm_kernel,
// gemm_kernel_v2, gemm_gated_kernel: double-buffered, the next stage's global
// loads issued before the current stage's MFMAs) or by direct global -> LDS
// loads into a ring of stages (gemm_f32d_kernel, gemm_q8d_kernel); one barrier
// per K stage.  Inside a stage, lane half h owns the contiguous K run
// [h*BK/2, (h+1)*BK/2), so every fragment read is a run of ds_read_b128.
// The K order of an output element depends only on K and the instantiation,
// never on the row count or the row's position, so packed and separate
// batches give the same bits.
//  - f32: v_mfma_f32_32x32x2_f32 (one k per lane half per step).
//  - int8 x f16: W tiles are widened int8 -> f16 (exact) while being staged
//    through registers, or per fragment when W sits in LDS as int8; X is f16;
//    v_mfma_f32_32x32x16_f16 (8 k per lane half per step), f32 accumulation.
// Tiles are renumbered so that each XCD (blocks are dispatched round robin
// over the 8 XCDs) owns a contiguous run, and inside an item the run walks
// groups of GR row tiles column by column, so a group's X rows and the W
// columns in flight stay in that XCD's L2.
#pragma once
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "dev.h"
#include "kern.h"

namespace enc {
namespace gemm {

// Compute units of the current device (queried once per device).
inline int device_cus() {
    constexpr int kDevs = 64;
    static std::atomic<int> cache[kDevs];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const bool cached = dev >= 0 && dev < kDevs;
    if (cached) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (cached) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

constexpr int GR = 8;  // row tiles per L2 group

__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t G) {
    const uint32_t x = b & 7u, j = b >> 3, q = G >> 3, r = G & 7u;
    return x * q + min(x, r) + j;
}

struct TileCtx {
    GemmItemK it;
    const void *w;
    const float *rs;
    const float *bias;
    int row0, col0;
};

// Item, weights and tile origin of linear tile `tile` (< a.total_tiles);
// G row tiles per L2 group.
template <int BM, int BN, int G = GR>
__device__ __forceinline__ void locate_tile(const GemmArgs &a, uint32_t tile, TileCtx &t, int cols_per_tile) {
    // uniform by construction; stated, so that the item lookup below stays a
    // scalar load of the argument block (a per-lane index would copy the
    // whole block to scratch)
    tile = __builtin_amdgcn_readfirstlane(tile);
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
    // item-local tile -> (row tile, col tile): groups of GR row tiles, each
    // group walked column by column (row tile fastest)
    const uint32_t local = tile - t.it.tile0;
    const uint32_t tiles_n = (t.it.n + BM - 1) / BM, tm = t.it.tiles_m;
    const uint32_t g = local / (G * tm), in_g = local % (G * tm);
    const uint32_t rows_g = min((uint32_t)G, tiles_n - g * G);
    t.row0 = (int)((g * G + in_g % rows_g) * BM);
    t.col0 = (int)((in_g / rows_g) * cols_per_tile);
}

// The tile of this block in a launch of one block per tile: consecutive
// blocks go to the eight XCDs in turn, so block b takes tile xcd_remap(b) and
// each XCD works through one contiguous run of tiles (shared rows and columns
// stay in its L2).
template <int BM, int BN, int G = GR>
__device__ __forceinline__ bool locate(const GemmArgs &a, TileCtx &t, int cols_per_tile = BN) {
    const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
    if (tile >= a.total_tiles) return false;
    locate_tile<BM, BN, G>(a, tile, t, cols_per_tile);
    return true;
}

// Gated epilogue flags (internal copies of the public ENC_EPI_GATE_* bits).
constexpr uint32_t kGateGelu = 8u, kGateSilu = 16u;

template <bool I8>
struct Elem;
template <>
struct Elem<false> {
    using T = float;
    using V = f32x4;  // 16-byte LDS / global chunk
    static constexpr int CE = 4;
    static constexpr int KSTEP = 2;  // k per MFMA (both lane halves)
};
template <>
struct Elem<true> {
    using T = _Float16;
    using V = f16x8;
    static constexpr int CE = 8;
    static constexpr int KSTEP = 16;
};

// 16 int8 -> 16 f16, exact: byte b, biased to b + 128 in [1, 255], is the low
// mantissa of the half 1024 + (b + 128) (bits 0x6400 | byte); subtracting 1152
// leaves b.  Two packed halves per 32-bit op.
__device__ __forceinline__ void widen16(const int32_t w[4], f16x8 &lo, f16x8 &hi) {
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t u = (uint32_t)w[i] ^ 0x80808080u;
        // bytes (0, 1) and (2, 3) of u as the low bytes of two halves each
        o[2 * i] = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);
        o[2 * i + 1] = __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u);
    }
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f16x2 a = __builtin_bit_cast(f16x2, o[i]) - bias;
        f16x2 b = __builtin_bit_cast(f16x2, o[4 + i]) - bias;
        lo[2 * i] = a[0];
        lo[2 * i + 1] = a[1];
        hi[2 * i] = b[0];
        hi[2 * i + 1] = b[1];
    }
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
    const float oc = a.ycol ? a.ycol[c] : 1.0f;
    const bool f16 = a.flags & 1u, accum = a.flags & 2u, gelu = a.flags & 4u;
    const size_t base = t.it.y_off + c;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int row = rbase + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (row >= (int)t.it.n) continue;
        float v = acc[r] * mul + b;
        if (gelu) v = gelu_tanh(v);
        v = v * oc * a.yscale;  // exact when both are 1
        const size_t off = base + (size_t)row * t.it.ldy;
        if (f16) {
            reinterpret_cast<_Float16 *>(a.y)[off] = (_Float16)v;
        } else {
            float *y = reinterpret_cast<float *>(a.y) + off;
            *y = accum ? *y + v : v;
        }
    }
}

// Epilogue of a wave's FM x FN accumulator blocks of an int8-path tile (not
// gated), rows rbase0 + 32 i + ..., columns cbase0 + 32 j + ...: the values of
// store_block, with the launch's flags resolved once.  The common cases (f16 or
// f32 output, no accumulation, no GELU, no column field and a unit output
// scale) take a loop without per-value flag tests, row checks only in a tile
// that crosses n, and 32-bit element offsets from a scalar base; v * 1 * 1
// is v exactly, so they give store_block's bits.
template <typename T, int FM, int FN>
__device__ __forceinline__ void store_plain(const GemmArgs &a, const TileCtx &t, const f32x16 (&acc)[FM][FN],
                                            int rbase0, int cbase0, int lane) {
    const int li = lane & 31, hf = lane >> 5;
    const int n = (int)t.it.n;
    const uint32_t ldy = t.it.ldy;
#pragma unroll
    for (int j = 0; j < FN; j++) {
        const int c = cbase0 + 32 * j + li;
        if (c >= (int)t.it.m) continue;
        const float mul = a.alpha * t.rs[c];
        const float b = t.bias ? t.bias[c] : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int rbase = rbase0 + 32 * i;
            T *ytile = reinterpret_cast<T *>(a.y) + t.it.y_off + (size_t)rbase * ldy;  // uniform
            const uint32_t lo = (uint32_t)(4 * hf) * ldy + (uint32_t)c;
            // (v is materialised in f32 before the conversion, as store_block
            // has it, rather than fused into a mixed-precision fma)
            if (rbase + 32 <= n) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    float v = acc[i][j][r] * mul + b;
                    asm("" : "+v"(v));
                    ytile[lo + (uint32_t)(8 * (r >> 2) + (r & 3)) * ldy] = (T)v;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int dr = 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (rbase + dr >= n) continue;
                    float v = acc[i][j][r] * mul + b;
                    asm("" : "+v"(v));
                    ytile[lo + (uint32_t)(8 * (r >> 2) + (r & 3)) * ldy] = (T)v;
                }
            }
        }
    }
}

template <int FM, int FN>
__device__ __forceinline__ void store_tile_i8(const GemmArgs &a, const TileCtx &t, const f32x16 (&acc)[FM][FN],
                                              int rbase0, int cbase0, int lane) {
    const bool f16 = a.flags & 1u, accum = a.flags & 2u, gelu = a.flags & 4u;
    if (!accum && !gelu && !a.ycol && a.yscale == 1.0f) {
        if (f16)
            store_plain<_Float16>(a, t, acc, rbase0, cbase0, lane);
        else
            store_plain<float>(a, t, acc, rbase0, cbase0, lane);
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) store_block<true>(a, t, acc[i][j], rbase0 + i * 32, cbase0 + j * 32, lane);
}

template <int BM, int BN, int BK, int WGM, int WGN, bool I8, int MINB>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_kernel(GemmArgs a) {
    using E = Elem<I8>;
    using T = typename E::T;
    using V = typename E::V;
    constexpr int NT = 64 * WGM * WGN;
    constexpr int CE = E::CE;
    constexpr int LDS = BK + CE;  // padded row (elements): rows 16 bytes apart in bank phase
    constexpr int FM = BM / WGM / 32, FN = BN / WGN / 32;
    constexpr int HK = BK / 2;            // k per lane half per stage
    constexpr int NV = HK / CE;           // 16-byte fragment chunks per lane per block
    constexpr int NSTEP = BK / E::KSTEP;  // MFMA k-steps per stage
    constexpr int A_CH = BM * BK / CE / NT;        // X chunks per thread per stage
    constexpr int B_CH = I8 ? BN * BK / 16 / NT : BN * BK / CE / NT;
    static_assert(FM >= 1 && FN >= 1 && BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "tile");
    static_assert(BM * BK % (CE * NT) == 0 && (I8 ? BN * BK % (16 * NT) : BN * BK % (CE * NT)) == 0,
                  "loads");
    static_assert(HK % CE == 0, "fragments");

    __shared__ __attribute__((aligned(16))) T As[2][BM][LDS];
    __shared__ __attribute__((aligned(16))) T Bs[2][BN][LDS];
    TileCtx t;
    if (!locate<BM, BN>(a, t)) return;
    const int n = t.it.n, m = t.it.m, K = t.it.k;
    const T *X = reinterpret_cast<const T *>(a.x) + t.it.x_off;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int wr = wave / WGN, wc = wave % WGN;

    V ra[A_CH];
    using BReg = typename std::conditional<I8, int32_t, V>::type;
    constexpr int BRW = I8 ? 4 : 1;  // register words per B chunk
    BReg rb[B_CH][BRW];

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
            const int gk = k0 + c, gr = t.row0 + r;
            if (gr < n && gk < K)
                ra[i] = *reinterpret_cast<const V *>(X + (size_t)gr * t.it.ldx + gk);
            else
                ra[i] = V{};
        }
        if constexpr (I8) {
            const int8_t *W = reinterpret_cast<const int8_t *>(t.w);
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / 16), c = (f % (BK / 16)) * 16;
                const int gk = k0 + c, gc = t.col0 + r;
                if (gc < m && gk < K) {
                    const int32_t *p = reinterpret_cast<const int32_t *>(W + (size_t)gc * K + gk);
#pragma unroll
                    for (int q = 0; q < 4; q++) rb[i][q] = p[q];
                } else {
#pragma unroll
                    for (int q = 0; q < 4; q++) rb[i][q] = 0;
                }
            }
        } else {
            const float *W = reinterpret_cast<const float *>(t.w);
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
                const int gk = k0 + c, gc = t.col0 + r;
                rb[i][0] = (gc < m && gk < K) ? *reinterpret_cast<const V *>(W + (size_t)gc * K + gk) : V{};
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
            *reinterpret_cast<V *>(&As[buf][r][c]) = ra[i];
        }
        if constexpr (I8) {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / 16), c = (f % (BK / 16)) * 16;
                f16x8 lo, hi;
                widen16(rb[i], lo, hi);
                *reinterpret_cast<f16x8 *>(&Bs[buf][r][c]) = lo;
                *reinterpret_cast<f16x8 *>(&Bs[buf][r][c + 8]) = hi;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
                *reinterpret_cast<V *>(&Bs[buf][r][c]) = rb[i][0];
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nst = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int s = 0; s < nst; s++) {
        const int buf = s & 1;
        if (s + 1 < nst) gload((s + 1) * BK);
        V fa[FM][NV], fb[FN][NV];
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int q = 0; q < NV; q++)
                fa[i][q] = *reinterpret_cast<const V *>(&As[buf][wr * (BM / WGM) + i * 32 + li][HK * hf + CE * q]);
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int q = 0; q < NV; q++)
                fb[j][q] = *reinterpret_cast<const V *>(&Bs[buf][wc * (BN / WGN) + j * 32 + li][HK * hf + CE * q]);
#pragma unroll
        for (int kk = 0; kk < NSTEP; kk++)
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    if constexpr (I8)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i][kk], fb[j][kk], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][kk / 4][kk % 4], fb[j][kk / 4][kk % 4],
                                                                        acc[i][j], 0, 0, 0);
                }
        if (s + 1 < nst) sstore(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            store_block<I8>(a, t, acc[i][j], t.row0 + wr * (BM / WGM) + i * 32, t.col0 + wc * (BN / WGN) + j * 32,
                            lane);
}

// Tiles of the item table for a BM x BN instantiation (fills tiles_m, tile0).
inline uint32_t plan_tiles(GemmArgs &g, int BM, int BN) {
    uint32_t tiles = 0;
    for (uint32_t i = 0; i < g.nitems; i++) {
        GemmItemK &k = g.items[i];
        k.tiles_m = (k.m + BN - 1) / BN;
        k.tile0 = tiles;
        tiles += k.tiles_m * ((k.n + BM - 1) / BM);
    }
    for (uint32_t i = g.nitems; i < (uint32_t)kMaxGemmItems; i++) g.items[i].tile0 = 0xffffffffu;
    g.total_tiles = tiles;
    return tiles;
}

template <int BM, int BN, int BK, int WGM, int WGN, bool I8, int MINB>
hipError_t launch(GemmArgs g, hipStream_t s) {
    const uint32_t tiles = plan_tiles(g, BM, BN);
    if (!tiles) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WGM, WGN, I8, MINB>), dim3(tiles), dim3(64 * WGM * WGN), 0, s, g);
    return hipGetLastError();
}

// Deeper-pipelined schedule of the same tile: global loads run two K stages
// ahead (a ring of two register sets, loop unrolled by two so the ring index
// is static), and inside a stage the fragments of k-step kk+1 are read from
// LDS while the MFMAs of k-step kk run.  Same K order per output as
// gemm_kernel, so results are bit-identical between the two schedules.
template <int BM, int BN, int BK, int WGM, int WGN, bool I8, int MINB>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_kernel_v2(GemmArgs a) {
    using E = Elem<I8>;
    using T = typename E::T;
    using V = typename E::V;
    constexpr int NT = 64 * WGM * WGN;
    constexpr int CE = E::CE;
    constexpr int LDS = BK + CE;
    constexpr int FM = BM / WGM / 32, FN = BN / WGN / 32;
    constexpr int HK = BK / 2;
    constexpr int NSTEP = BK / E::KSTEP;
    constexpr int A_CH = BM * BK / CE / NT;
    constexpr int B_CH = I8 ? BN * BK / 16 / NT : BN * BK / CE / NT;
    // fragment of one k-step: f16 -> one V (8 halves); f32 -> one float
    using F = typename std::conditional<I8, f16x8, float>::type;
    static_assert(FM >= 1 && FN >= 1, "tile");
    static_assert(BM * BK % (CE * NT) == 0 && (I8 ? BN * BK % (16 * NT) : BN * BK % (CE * NT)) == 0,
                  "loads");

    __shared__ __attribute__((aligned(16))) T As[2][BM][LDS];
    __shared__ __attribute__((aligned(16))) T Bs[2][BN][LDS];
    TileCtx t;
    if (!locate<BM, BN>(a, t)) return;
    const int n = t.it.n, m = t.it.m, K = t.it.k;
    const T *X = reinterpret_cast<const T *>(a.x) + t.it.x_off;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int wr = wave / WGN, wc = wave % WGN;

    using BReg = typename std::conditional<I8, int32_t, V>::type;
    constexpr int BRW = I8 ? 4 : 1;
    V ra[2][A_CH];
    BReg rb[2][B_CH][BRW];

    auto gload = [&](int k0, V (&RA)[A_CH], BReg (&RB)[B_CH][BRW]) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
            const int gk = k0 + c, gr = t.row0 + r;
            if (gr < n && gk < K)
                RA[i] = *reinterpret_cast<const V *>(X + (size_t)gr * t.it.ldx + gk);
            else
                RA[i] = V{};
        }
        if constexpr (I8) {
            const int8_t *W = reinterpret_cast<const int8_t *>(t.w);
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / 16), c = (f % (BK / 16)) * 16;
                const int gk = k0 + c, gc = t.col0 + r;
                if (gc < m && gk < K) {
                    const int32_t *p = reinterpret_cast<const int32_t *>(W + (size_t)gc * K + gk);
#pragma unroll
                    for (int q = 0; q < 4; q++) RB[i][q] = p[q];
                } else {
#pragma unroll
                    for (int q = 0; q < 4; q++) RB[i][q] = 0;
                }
            }
        } else {
            const float *W = reinterpret_cast<const float *>(t.w);
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
                const int gk = k0 + c, gc = t.col0 + r;
                RB[i][0] = (gc < m && gk < K) ? *reinterpret_cast<const V *>(W + (size_t)gc * K + gk) : V{};
            }
        }
    };
    auto sstore = [&](int buf, const V (&RA)[A_CH], const BReg (&RB)[B_CH][BRW]) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
            *reinterpret_cast<V *>(&As[buf][r][c]) = RA[i];
        }
        if constexpr (I8) {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / 16), c = (f % (BK / 16)) * 16;
                f16x8 lo, hi;
                widen16(RB[i], lo, hi);
                *reinterpret_cast<f16x8 *>(&Bs[buf][r][c]) = lo;
                *reinterpret_cast<f16x8 *>(&Bs[buf][r][c + 8]) = hi;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
                *reinterpret_cast<V *>(&Bs[buf][r][c]) = RB[i][0];
            }
        }
    };
    // fragment of k-step kk for accumulator row block i / column block j
    auto frag_a = [&](int buf, int i, int kk) -> F {
        const T *p = &As[buf][wr * (BM / WGM) + i * 32 + li][HK * hf];
        if constexpr (I8) return *reinterpret_cast<const f16x8 *>(p + 8 * kk);
        else return p[kk];
    };
    auto frag_b = [&](int buf, int j, int kk) -> F {
        const T *p = &Bs[buf][wc * (BN / WGN) + j * 32 + li][HK * hf];
        if constexpr (I8) return *reinterpret_cast<const f16x8 *>(p + 8 * kk);
        else return p[kk];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    auto compute = [&](int buf) {
        F fa[2][FM], fb[2][FN];
#pragma unroll
        for (int i = 0; i < FM; i++) fa[0][i] = frag_a(buf, i, 0);
#pragma unroll
        for (int j = 0; j < FN; j++) fb[0][j] = frag_b(buf, j, 0);
#pragma unroll
        for (int kk = 0; kk < NSTEP; kk++) {
            const int cur = kk & 1, nxt = cur ^ 1;
            if (kk + 1 < NSTEP) {
#pragma unroll
                for (int i = 0; i < FM; i++) fa[nxt][i] = frag_a(buf, i, kk + 1);
#pragma unroll
                for (int j = 0; j < FN; j++) fb[nxt][j] = frag_b(buf, j, kk + 1);
            }
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    if constexpr (I8)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
                }
        }
    };

    const int nst = (K + BK - 1) / BK;
    gload(0, ra[0], rb[0]);
    if (nst > 1) gload(BK, ra[1], rb[1]);
    sstore(0, ra[0], rb[0]);
    __syncthreads();
    // stage s computes on LDS buf s&1; register set s&1 is free once stage s
    // has been written to LDS, so it receives stage s+2
    for (int s = 0; s < nst; s += 2) {
        if (s + 2 < nst) gload((s + 2) * BK, ra[0], rb[0]);
        compute(0);
        if (s + 1 < nst) sstore(1, ra[1], rb[1]);
        __syncthreads();
        if (s + 1 >= nst) break;
        if (s + 3 < nst) gload((s + 3) * BK, ra[1], rb[1]);
        compute(1);
        if (s + 2 < nst) sstore(0, ra[0], rb[0]);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            store_block<I8>(a, t, acc[i][j], t.row0 + wr * (BM / WGM) + i * 32, t.col0 + wc * (BN / WGN) + j * 32,
                            lane);
}

template <int BM, int BN, int BK, int WGM, int WGN, bool I8, int MINB>
hipError_t launch_v2(GemmArgs g, hipStream_t s) {
    const uint32_t tiles = plan_tiles(g, BM, BN);
    if (!tiles) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel_v2<BM, BN, BK, WGM, WGN, I8, MINB>), dim3(tiles), dim3(64 * WGM * WGN), 0, s, g);
    return hipGetLastError();
}

// Gated MLP GEMM: Y[i][j] = act(alpha * gate_ij) * (alpha * up_ij), act =
// gelu_tanh or silu, gate from weight slot s and up from slot s+1 (int8 path:
// each times its own row scale).  Each wave's two 32-column accumulator blocks
// are the gate and the up projections of the same 32 output columns, so the
// product is formed in registers: the gate|up pair is never written out.  The
// block tile covers BN/2 output columns; K order as gemm_kernel.
template <int BM, int BN, int BK, int WGM, bool I8, int MINB>
__global__ __launch_bounds__(64 * WGM * (BN / 64), MINB) void gemm_gated_kernel(GemmArgs a) {
    constexpr int WGN = BN / 64;  // waves along N, each 32 gate + 32 up columns
    using E = Elem<I8>;
    using T = typename E::T;
    using V = typename E::V;
    constexpr int NT = 64 * WGM * WGN;
    constexpr int CE = E::CE;
    constexpr int LDS = BK + CE;
    constexpr int FM = BM / WGM / 32, FN = 2;
    constexpr int HK = BK / 2;
    constexpr int NV = HK / CE;
    constexpr int NSTEP = BK / E::KSTEP;
    constexpr int A_CH = BM * BK / CE / NT;
    constexpr int B_CH = I8 ? BN * BK / 16 / NT : BN * BK / CE / NT;
    static_assert(FM >= 1 && BN % 64 == 0, "tile");
    static_assert(BM * BK % (CE * NT) == 0 && (I8 ? BN * BK % (16 * NT) : BN * BK % (CE * NT)) == 0,
                  "loads");

    __shared__ __attribute__((aligned(16))) T As[2][BM][LDS];
    __shared__ __attribute__((aligned(16))) T Bs[2][BN][LDS];
    TileCtx t;
    if (!locate<BM, BN>(a, t, BN / 2)) return;
    // gate = slot s, up = slot s + 1
    const void *wg = t.w, *wu = a.w[1];
    const float *rg = t.rs, *ru = a.rs[1];
#pragma unroll
    for (int s2 = 1; s2 < kMaxGemmItems; s2++)
        if ((int)t.it.slot + 1 == s2) {
            wu = a.w[s2];
            ru = a.rs[s2];
        }
    const int n = t.it.n, m = t.it.m, K = t.it.k;
    const T *X = reinterpret_cast<const T *>(a.x) + t.it.x_off;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int wr = wave / WGN, wc = wave % WGN;

    // B tile row r holds weight row col0 + (r/64)*32 + r%32 of the gate
    // ((r/32) even) or up ((r/32) odd) matrix
    auto brow = [&](int r, const void *&w) -> int {
        w = ((r >> 5) & 1) ? wu : wg;
        return t.col0 + (r >> 6) * 32 + (r & 31);
    };

    V ra[A_CH];
    using BReg = typename std::conditional<I8, int32_t, V>::type;
    constexpr int BRW = I8 ? 4 : 1;
    BReg rb[B_CH][BRW];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
            const int gk = k0 + c, gr = t.row0 + r;
            if (gr < n && gk < K)
                ra[i] = *reinterpret_cast<const V *>(X + (size_t)gr * t.it.ldx + gk);
            else
                ra[i] = V{};
        }
        if constexpr (I8) {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / 16), c = (f % (BK / 16)) * 16;
                const void *w;
                const int gc = brow(r, w), gk = k0 + c;
                if (gc < m && gk < K) {
                    const int32_t *p = reinterpret_cast<const int32_t *>(reinterpret_cast<const int8_t *>(w) +
                                                                         (size_t)gc * K + gk);
#pragma unroll
                    for (int q = 0; q < 4; q++) rb[i][q] = p[q];
                } else {
#pragma unroll
                    for (int q = 0; q < 4; q++) rb[i][q] = 0;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
                const void *w;
                const int gc = brow(r, w), gk = k0 + c;
                rb[i][0] = (gc < m && gk < K)
                               ? *reinterpret_cast<const V *>(reinterpret_cast<const float *>(w) + (size_t)gc * K + gk)
                               : V{};
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
            *reinterpret_cast<V *>(&As[buf][r][c]) = ra[i];
        }
        if constexpr (I8) {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / 16), c = (f % (BK / 16)) * 16;
                f16x8 lo, hi;
                widen16(rb[i], lo, hi);
                *reinterpret_cast<f16x8 *>(&Bs[buf][r][c]) = lo;
                *reinterpret_cast<f16x8 *>(&Bs[buf][r][c + 8]) = hi;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_CH; i++) {
                const int f = tid + NT * i, r = f / (BK / CE), c = (f % (BK / CE)) * CE;
                *reinterpret_cast<V *>(&Bs[buf][r][c]) = rb[i][0];
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nst = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int s = 0; s < nst; s++) {
        const int buf = s & 1;
        if (s + 1 < nst) gload((s + 1) * BK);
        V fa[FM][NV], fb[FN][NV];
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int q = 0; q < NV; q++)
                fa[i][q] = *reinterpret_cast<const V *>(&As[buf][wr * (BM / WGM) + i * 32 + li][HK * hf + CE * q]);
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int q = 0; q < NV; q++)
                fb[j][q] = *reinterpret_cast<const V *>(&Bs[buf][wc * 64 + j * 32 + li][HK * hf + CE * q]);
#pragma unroll
        for (int kk = 0; kk < NSTEP; kk++)
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    if constexpr (I8)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i][kk], fb[j][kk], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][kk / 4][kk % 4], fb[j][kk / 4][kk % 4],
                                                                        acc[i][j], 0, 0, 0);
                }
        if (s + 1 < nst) sstore(buf ^ 1);
        __syncthreads();
    }
    // epilogue: lane holds gate and up of the same (row, column)
    const int c = t.col0 + wc * 32 + li;
    if (c >= m) return;
    float mg = a.alpha, mu = a.alpha;
    if (I8) {
        mg *= rg[c];
        mu *= ru[c];
    }
    const bool f16 = a.flags & 1u, gelu = a.flags & kGateGelu;
    const float oc = a.ycol ? a.ycol[c] : 1.0f;
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int row = t.row0 + wr * (BM / WGM) + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (row >= n) continue;
            const float g = acc[i][0][r] * mg, u = acc[i][1][r] * mu;
            const float v = (gelu ? gelu_tanh(g) : silu(g)) * u * oc * a.yscale;
            const size_t off = t.it.y_off + (size_t)row * t.it.ldy + c;
            if (f16)
                reinterpret_cast<_Float16 *>(a.y)[off] = (_Float16)v;
            else
                reinterpret_cast<float *>(a.y)[off] = v;
        }
}

template <int BM, int BN, int BK, int WGM, bool I8, int MINB>
hipError_t launch_gated(GemmArgs g, hipStream_t s) {
    const uint32_t tiles = plan_tiles(g, BM, BN / 2);
    if (!tiles) return hipSuccess;
    hipLaunchKernelGGL((gemm_gated_kernel<BM, BN, BK, WGM, I8, MINB>), dim3(tiles), dim3(64 * WGM * (BN / 64)), 0, s,
                       g);
    return hipGetLastError();
}

// 8 int8 (two 32-bit words) -> 8 f16, exact (the widen16 construction).
__device__ __forceinline__ f16x8 widen8(uint32_t w0, uint32_t w1) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u0, 0x05010400u)) - bias;
    const f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u0, 0x05030402u)) - bias;
    const f16x2 c = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u1, 0x05010400u)) - bias;
    const f16x2 d = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u1, 0x05030402u)) - bias;
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The same 8 values by the signed-byte conversion: v_cvt_f16_i16 reads one
// byte of its operand sign-extended (SDWA) and writes one half of its result
// word, so each value costs one instruction; exact, the same bits as widen8.
__device__ __forceinline__ f16x8 widen8s(uint32_t w0, uint32_t w1) {
    uint32_t d0, d1, d2, d3;
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(d0) : "v"(w0));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1"
        : "+v"(d0)
        : "v"(w0));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(d1) : "v"(w0));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
        : "+v"(d1)
        : "v"(w0));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(d2) : "v"(w1));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1"
        : "+v"(d2)
        : "v"(w1));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(d3) : "v"(w1));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
        : "+v"(d3)
        : "v"(w1));
    return __builtin_bit_cast(f16x8, u32x4{d0, d1, d2, d3});
}

// ---------------------------------------------------------------------------
// int8 x f16 GEMM fed by direct global -> LDS loads (raw buffer loads with
// the LDS as destination, buffer_load_dwordx4 ... lds).
//
// BM x BN block tile, WGM x WGN waves, each wave (BM/WGM) x (BN/WGN) outputs
// (FM x FN accumulator blocks of 32 x 32), W kept as int8 in LDS and widened
// per fragment (widen8s: one signed-byte conversion per value).  Three LDS
// stages of 64 K each: the loads of stage s+3 are issued as soon as every wave
// has finished reading stage s, so two stages of loads are in flight while
// one is computed, and no register holds staged data.  The loads are raw
// buffer loads whose per-lane offsets are fixed for the tile and whose k
// offset and LDS destination sit in scalar registers: a load costs no vector
// instruction.  The epilogue resolves the launch's flags once per tile
// (store_tile_i8).  Measured on the 8448-row DiT shapes against per-value
// flag tests, global_load_lds with per-lane 64-bit addresses and the
// byte-permute widening, these three took the GEMMs from 1050-1140 to
// 1110-1180 TFLOP/s with the same bits.  The large-problem instantiation is 256 x 256 with 8 waves (128 x 64
// each, one block per CU, 48 KB per stage); 128-row tiles serve launches with
// too few 256-row tiles to spread over the CUs.
//
// A load instruction writes 64 lanes x 16 bytes to 1 KB of consecutive LDS, so
// the LDS tiles are swizzled instead of padded: X row r (128 bytes = 8 chunks
// of 8 halves) keeps chunk c at position c ^ ((r >> 1) & 7); W row r (64 bytes
// = 4 chunks of 16 int8) keeps chunk c at position c ^ ((r >> 2) & 3).  Every
// 16 consecutive lanes of a fragment read then hit 16 distinct bank groups.
//
// The compiler cannot tell LDS reads apart from the in-flight LDS-bound loads
// and would wait for all of them before every read, so the fragment reads are
// issued as ds_read_b128 in inline assembly and their completion is awaited
// explicitly (lgkmcnt), each fragment register then passed through an empty
// asm statement so that no use moves above the wait.
//
// Same K order as gemm_kernel<.., 64, .., true, ..>: stage 64, lane half h
// owns k in [32h, 32h + 32), k-step kk the 8 values at 32h + 8kk.  Requires
// K % 64 == 0.  Rows past n and columns past m load clamped (finite) rows and
// are never stored.  Gated: each wave column holds 32 gate and 32 up rows of
// the same 32 output columns (BN / WGN == 64).
template <int FM, int FN>
__device__ __forceinline__ void frag_ready(u32x4 (&a)[FM], u32x4 (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; i++) ready(a[i]);
#pragma unroll
    for (int j = 0; j < FN; j++) ready(b[j]);
}

// Wait until at most k stages of NDMA loads each are in flight, 0 <= k <= KMAX.
template <int NDMA, int KMAX>
__device__ __forceinline__ void vm_wait_stages(int k) {
    if constexpr (KMAX > 0) {
        if (k >= KMAX) {
            vm_wait<KMAX * NDMA>();
            return;
        }
        vm_wait_stages<NDMA, KMAX - 1>(k);
    } else {
        vm_wait<0>();
    }
}

template <int BM, int BN, int WGM, int WGN, int MINB, bool GATED, int NS = 3>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_q8d_kernel(GemmArgs a) {
    constexpr int NW = WGM * WGN, BK = 64;
    static_assert(NS >= 2 && NS <= 8, "stages");
    constexpr int FM = BM / WGM / 32, FN = BN / WGN / 32;
    constexpr int A_BYTES = BM * BK * 2, S_BYTES = A_BYTES + BN * BK;
    constexpr int AL = A_BYTES / 1024 / NW, BL = BN * BK / 1024 / NW;  // loads per wave per stage
    constexpr int NDMA = AL + BL;
    static_assert(AL >= 1 && BL >= 1 && AL * 1024 * NW == A_BYTES && BL * 1024 * NW == BN * BK, "loads");
    static_assert(FM >= 1 && FN >= 1 && (!GATED || BN / WGN == 64), "tile");
    static_assert(NS * S_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * S_BYTES];

    // groups of four row tiles: an XCD's 32 concurrent tiles are 4 row tiles by
    // 8 column tiles, whose X slabs (two bytes per value) and W slabs (one)
    // together stream least from beyond the L2 (8448 rows: 16-21% fewer bytes
    // fetched per launch than groups of eight, and 0-1% faster)
    TileCtx t;
    if (!locate<BM, BN, 4>(a, t, GATED ? BN / 2 : BN)) return;
    const int8_t *wg = reinterpret_cast<const int8_t *>(t.w), *wu = wg;
    const float *rg = t.rs, *ru = t.rs;
    if constexpr (GATED) {
        wu = reinterpret_cast<const int8_t *>(a.w[1]);
        ru = a.rs[1];
#pragma unroll
        for (int s2 = 1; s2 < kMaxGemmItems; s2++)
            if ((int)t.it.slot + 1 == s2) {
                wu = reinterpret_cast<const int8_t *>(a.w[s2]);
                ru = a.rs[s2];
            }
    }
    const int n = t.it.n, m = t.it.m, K = t.it.k;
    const _Float16 *X = reinterpret_cast<const _Float16 *>(a.x) + t.it.x_off;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 31, hf = lane >> 5;
    const int wr = wave / WGN, wc = wave % WGN;

    // sources of this lane's load instructions (k offset added per stage):
    // X load q of this wave covers tile rows 8 (AL wave + q) .. + 7, W load q
    // covers W rows 16 (BL wave + q) .. + 15
    const _Float16 *asrc[AL];
#pragma unroll
    for (int q = 0; q < AL; q++) {
        const int r = 8 * (AL * wave + q) + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
        asrc[q] = X + (size_t)min(t.row0 + r, n - 1) * t.it.ldx + 8 * c;
    }
    const int8_t *bsrc[BL];
#pragma unroll
    for (int q = 0; q < BL; q++) {
        const int r = 16 * (BL * wave + q) + (lane >> 2), c = (lane & 3) ^ ((r >> 2) & 3);
        const int8_t *w = wg;
        int col = t.col0 + r;
        if constexpr (GATED) {
            w = ((r >> 5) & 1) ? wu : wg;
            col = t.col0 + (r >> 6) * 32 + (r & 31);
        }
        bsrc[q] = w + (size_t)min(col, m - 1) * K + 16 * c;
    }
    // the loads as raw buffer loads: per-lane byte offsets fixed for the
    // tile, the stage's k offset and the LDS destination in scalar registers,
    // so a load costs no vector instruction (the launcher checks that the
    // offsets fit 32 bits).  Gated: each W load's 16 rows lie in one matrix.
    const __amdgpu_buffer_rsrc_t xres = raw_buffer(X), wres[2] = {raw_buffer(wg), raw_buffer(wu)};
    uint32_t aoff[AL], boff[BL];
#pragma unroll
    for (int q = 0; q < AL; q++) aoff[q] = (uint32_t)((const char *)asrc[q] - (const char *)X);
#pragma unroll
    for (int q = 0; q < BL; q++) {
        const int r = 16 * (BL * wave + q);
        boff[q] = (uint32_t)((const char *)bsrc[q] - (const char *)(((r >> 5) & 1) && GATED ? wu : wg));
    }
    auto dma = [&](auto b, int s) {  // stage s into buffer b = s % NS
        uint8_t *buf = smem;
        if constexpr (std::is_integral_v<decltype(b)>)
            buf += b * S_BYTES;
        else
            buf += decltype(b)::value * S_BYTES;
        const int k0 = s * BK;
#pragma unroll
        for (int q = 0; q < AL; q++) buffer_dma16(xres, buf + (AL * wave + q) * 1024, aoff[q], 2 * k0);
#pragma unroll
        for (int q = 0; q < BL; q++)
            buffer_dma16(wres[GATED ? (((BL * wave + q) >> 1) & 1) : 0], buf + A_BYTES + (BL * wave + q) * 1024,
                         boff[q], k0);
    };

    // fragment addresses: X row wr*(BM/WGM) + 32 i + li, chunk 4 hf + kk; W
    // row wc*(BN/WGN) + 32 j + li, chunk 2 hf + p (p = kk / 2, one read per two
    // k-steps).  A read group is one per-lane base plus the stage offset (one
    // add) and immediates for i / j.
    const uint32_t lds0 = lds_offset(smem);
    const uint32_t arow = lds0 + (uint32_t)(wr * (BM / WGM) + li) * 128u;
    const uint32_t brow = lds0 + A_BYTES + (uint32_t)(wc * (BN / WGN) + li) * 64u;
    const int sa = (li >> 1) & 7, sb = (li >> 2) & 3;
    uint32_t abase[4], bbase[2];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) abase[kk] = arow + (uint32_t)(((4 * hf + kk) ^ sa) * 16);
#pragma unroll
    for (int p = 0; p < 2; p++) bbase[p] = brow + (uint32_t)(((2 * hf + p) ^ sb) * 16);

    u32x4 fa0[FM], fa1[FM], fb0[FN], fb1[FN];
    // buffer b: a run-time index (one add per read group), or a compile-time
    // one (IC) whose offset is the reads' immediate where it fits the field
    auto read_a = [&](u32x4 (&d)[FM], auto b, int kk) {
        if constexpr (std::is_integral_v<decltype(b)>) {
            ds_read16_run<0, 4096, FM>(d, abase[kk] + (uint32_t)(b * S_BYTES));
        } else {
            constexpr int OFF = decltype(b)::value * S_BYTES;
            if constexpr (OFF + (FM - 1) * 4096 < 65536)
                ds_read16_run<OFF, 4096, FM>(d, abase[kk]);
            else
                ds_read16_run<0, 4096, FM>(d, abase[kk] + (uint32_t)OFF);
        }
    };
    auto read_b = [&](u32x4 (&d)[FN], auto b, int p) {
        if constexpr (std::is_integral_v<decltype(b)>) {
            ds_read16_run<0, 2048, FN>(d, bbase[p] + (uint32_t)(b * S_BYTES));
        } else {
            constexpr int OFF = decltype(b)::value * S_BYTES;
            if constexpr (OFF + (FN - 1) * 2048 < 65536)
                ds_read16_run<OFF, 2048, FN>(d, bbase[p]);
            else
                ds_read16_run<0, 2048, FN>(d, bbase[p] + (uint32_t)OFF);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
    auto mma = [&](const u32x4 (&fa)[FM], const u32x4 (&fb)[FN], int half) {
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const f16x8 b = widen8s(fb[j][2 * half], fb[j][2 * half + 1]);
#pragma unroll
            for (int i = 0; i < FM; i++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fa[i]), b, acc[i][j], 0,
                                                                   0, 0);
        }
    };

    auto mma_w = [&](const u32x4 (&fa)[FM], const f16x8 &b, int j) {
#pragma unroll
        for (int i = 0; i < FM; i++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fa[i]), b, acc[i][j], 0, 0, 0);
    };

    const int nst = K / BK;
    // the first min(NS, nst) stages; stage 0 awaited, the others may fly
#pragma unroll
    for (int s0 = 0; s0 < NS; s0++)
        if (s0 < nst) dma(s0, s0);
    vm_wait_stages<NDMA, NS - 1>(min(NS, nst) - 1);
    block_barrier();
    read_a(fa0, IC<0>{}, 0);
    read_b(fb0, IC<0>{}, 0);
    // stage s in buffer b = s % NS: a run-time index, or for tiles of at most
    // four accumulator blocks per wave and rings of at most three stages a
    // compile-time one, the loop unrolled over the NS buffers (no index
    // arithmetic per stage: the 1056-row output and down projections' 64 x 256
    // tiles 6-10% faster; larger tiles or rings run out of registers unrolled)
    auto stage = [&](auto b, int s) {
        read_a(fa1, b, 1);
        lgkm_wait_n<FM>();  // fa0, fb0 landed (fa1 may still be in flight)
        frag_ready(fa0, fb0);
        mma(fa0, fb0, 0);
        read_a(fa0, b, 2);
        read_b(fb1, b, 1);
        lgkm_wait_n<FM + FN>();  // fa1 landed
        frag_ready(fa1, fb0);
        mma(fa1, fb0, 1);
        read_a(fa1, b, 3);
        lgkm_wait_n<FM>();  // fa0, fb1 landed
        frag_ready(fa0, fb1);
        mma(fa0, fb1, 0);
        // stage s+1 landed (own loads; stages s+2 .. s+NS-1 may fly), own
        // reads of buffer b done; after the barrier every wave's are, so b
        // takes stage s+NS
        vm_wait_stages<NDMA, NS - 2>(min(NS - 2, nst - s - 2));
        lgkm_wait_n<0>();
        frag_ready(fa1, fb1);
        // the last k-step's W fragments are widened before the barrier and
        // its MFMAs issued first behind it, ahead of the loads and the next
        // stage's reads, so the MFMA pipe restarts as soon as the barrier
        // opens (1.5-2% on the 8448-row DiT shapes, the same bits)
        f16x8 wb[FN];
#pragma unroll
        for (int j = 0; j < FN; j++) wb[j] = widen8s(fb1[j][2], fb1[j][3]);
        __builtin_amdgcn_sched_barrier(0);
        block_barrier();
        mma_w(fa1, wb[0], 0);
        __builtin_amdgcn_sched_barrier(0);
        if (s + NS < nst) dma(b, s + NS);
        if (s + 1 < nst) {
            if constexpr (std::is_integral_v<decltype(b)>) {
                read_a(fa0, (s + 1) % NS, 0);
                read_b(fb0, (s + 1) % NS, 0);
            } else {
                read_a(fa0, IC<(decltype(b)::value + 1) % NS>{}, 0);
                read_b(fb0, IC<(decltype(b)::value + 1) % NS>{}, 0);
            }
        }
#pragma unroll
        for (int j = 1; j < FN; j++) mma_w(fa1, wb[j], j);
    };
    if constexpr (FM * FN <= 4 && NS <= 3) {
        for (int s0 = 0; s0 < nst; s0 += NS) {
            stage(IC<0>{}, s0);
            if constexpr (NS > 1) { if (s0 + 1 >= nst) break; stage(IC<1>{}, s0 + 1); }
            if constexpr (NS > 2) { if (s0 + 2 >= nst) break; stage(IC<2>{}, s0 + 2); }
            if constexpr (NS > 3) { if (s0 + 3 >= nst) break; stage(IC<3>{}, s0 + 3); }
            if constexpr (NS > 4) { if (s0 + 4 >= nst) break; stage(IC<4>{}, s0 + 4); }
            if constexpr (NS > 5) { if (s0 + 5 >= nst) break; stage(IC<5>{}, s0 + 5); }
            if constexpr (NS > 6) { if (s0 + 6 >= nst) break; stage(IC<6>{}, s0 + 6); }
            if constexpr (NS > 7) { if (s0 + 7 >= nst) break; stage(IC<7>{}, s0 + 7); }
        }
    } else {
        for (int s = 0; s < nst; s++) stage(s % NS, s);
    }

    if constexpr (!GATED) {
        store_tile_i8<FM, FN>(a, t, acc, t.row0 + wr * (BM / WGM), t.col0 + wc * (BN / WGN), lane);
    } else if ((a.flags & 1u) && !(a.flags & kGateGelu) && !a.ycol && a.yscale == 1.0f) {
        // SwiGLU into f16 without a column field or guard: silu(g) u (times
        // 1 and 1 elsewhere, the same bits), flags resolved once
        const int c = t.col0 + wc * 32 + li;
        if (c < m) {
            const float mg = a.alpha * rg[c], mu = a.alpha * ru[c];
            const uint32_t ldy = t.it.ldy;
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int rbase = t.row0 + wr * (BM / WGM) + i * 32;
                _Float16 *ytile = reinterpret_cast<_Float16 *>(a.y) + t.it.y_off + (size_t)rbase * ldy;
                const uint32_t lo = (uint32_t)(4 * hf) * ldy + (uint32_t)c;
                const bool full = rbase + 32 <= n;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    if (!full && rbase + 8 * (r >> 2) + 4 * hf + (r & 3) >= n) continue;
                    const float g = acc[i][0][r] * mg, u = acc[i][1][r] * mu;
                    float v = silu(g) * u;
                    asm("" : "+v"(v));
                    ytile[lo + (uint32_t)(8 * (r >> 2) + (r & 3)) * ldy] = (_Float16)v;
                }
            }
        }
    } else {
        const bool f16 = a.flags & 1u, gelu = a.flags & kGateGelu;
        const int c = t.col0 + wc * 32 + li;
        if (c < m) {
            const float mg = a.alpha * rg[c], mu = a.alpha * ru[c];
            const float oc = a.ycol ? a.ycol[c] : 1.0f;
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int row = t.row0 + wr * (BM / WGM) + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (row >= n) continue;
                    const float g = acc[i][0][r] * mg, u = acc[i][1][r] * mu;
                    const float v = (gelu ? gelu_tanh(g) : silu(g)) * u * oc * a.yscale;
                    const size_t off = t.it.y_off + (size_t)row * t.it.ldy + c;
                    if (f16)
                        reinterpret_cast<_Float16 *>(a.y)[off] = (_Float16)v;
                    else
                        reinterpret_cast<float *>(a.y)[off] = v;
                }
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int MINB, bool GATED, int NS = 3>
hipError_t launch_q8d(GemmArgs g, hipStream_t s) {
    const uint32_t tiles = plan_tiles(g, BM, GATED ? BN / 2 : BN);
    if (!tiles) return hipSuccess;
    hipLaunchKernelGGL((gemm_q8d_kernel<BM, BN, WGM, WGN, MINB, GATED, NS>), dim3(tiles), dim3(64 * WGM * WGN), 0, s,
                       g);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// f32 GEMM fed by direct global -> LDS loads, the counterpart of
// gemm_q8d_kernel for the FP32 path.  NS (3, or 2 for tiles whose stage is too
// large for three) LDS stages of 32 K each: the loads of stage s+NS are issued
// once every wave has finished reading stage s, and no register holds staged
// data.  X and W rows are 32 floats (128 bytes = 8
// chunks of 4 floats); row r keeps chunk c at position c ^ ((r >> 1) & 7), so
// the 16 consecutive lanes of a fragment read hit 16 distinct bank groups.
// Fragments are read with ds_read_b128 in inline assembly (one per-lane base
// per chunk, the stage and the 32-row block as immediates or one add) and
// awaited explicitly, as in the int8 kernel.
//
// Same K order as gemm_kernel<.., 32, .., false, ..>: stage 32, lane half h
// owns k in [16h, 16h + 16), k-step kk pairs k = kk (half 0) with 16 + kk
// (half 1); so every f32 instantiation gives the same bits.  Requires K % 32
// == 0.  Rows past n and columns past m load clamped (finite) rows and are
// never stored.  Gated: each wave column holds 32 gate and 32 up rows of the
// same 32 output columns (BN / WGN == 64); the epilogue forms act(g) * u.
//
// KS > 1 splits K inside the block: the block holds KS groups of WGM x WGN
// waves, group g sums k in [g K/KS, (g+1) K/KS) through a ring of its own, and
// at the end groups 1 .. KS-1 pass their sums through the LDS to group 0,
// which adds them in increasing g and stores.  An output is then
// ((s_0 + s_1) + ...) + s_{KS-1} with each s_g summed in the order above, the
// same for every row, so packed and separate batches stay bit-identical as
// long as KS depends only on the weight shape (see launch_gemm_f32).  One
// block per tile, plain epilogue only.
//
// The launch's argument block read in place (constant memory, scalar loads).
// A per-tile lookup in a loop through the by-value kernel argument makes the
// compiler keep a private copy of the whole block in scratch; the kernels
// that look up more than one tile read the table through this reference.
__device__ __forceinline__ const GemmArgs &kernarg_gemm() {
    return *(const GemmArgs *)__builtin_amdgcn_kernarg_segment_ptr();
}

// Per-lane sources of a tile's direct loads (k offset added per stage): load q
// of wave w covers tile rows 8 (L w + q) .. + 7, lane l row + l/8, position
// l%8 holding chunk (l%8) ^ ((row >> 1) & 7).  Rows past n and columns past m
// are clamped to the last one (finite, never stored).
template <int AL, int BL, bool GATED>
__device__ __forceinline__ void f32d_sources(const float *x, const float *wg, const float *wu, const TileCtx &tc,
                                             int wave, int lane, const float *(&asrc)[AL],
                                             const float *(&bsrc)[BL]) {
    const int n = tc.it.n, m = tc.it.m, K = tc.it.k;
    const float *X = x + tc.it.x_off;
#pragma unroll
    for (int q = 0; q < AL; q++) {
        const int r = 8 * (AL * wave + q) + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
        asrc[q] = X + (size_t)min(tc.row0 + r, n - 1) * tc.it.ldx + 4 * c;
    }
#pragma unroll
    for (int q = 0; q < BL; q++) {
        const int r = 8 * (BL * wave + q) + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
        const float *w = wg;
        int col = tc.col0 + r;
        if constexpr (GATED) {
            w = ((r >> 5) & 1) ? wu : wg;
            col = tc.col0 + (r >> 6) * 32 + (r & 31);
        }
        bsrc[q] = w + (size_t)min(col, m - 1) * K + 4 * c;
    }
}

// The up-projection weights and row scales of a gated int8 tile: slot + 1 of
// the tables.
__device__ __forceinline__ const void *gated_up_w(const GemmArgs &a, uint32_t slot) {
    const void *wu = a.w[1];
#pragma unroll
    for (int s2 = 1; s2 < kMaxGemmItems; s2++)
        if ((int)slot + 1 == s2) wu = a.w[s2];
    return wu;
}
__device__ __forceinline__ const float *gated_up_rs(const GemmArgs &a, uint32_t slot) {
    const float *ru = a.rs[1];
#pragma unroll
    for (int s2 = 1; s2 < kMaxGemmItems; s2++)
        if ((int)slot + 1 == s2) ru = a.rs[s2];
    return ru;
}

// The up-projection weights of a gated tile: slot + 1 of the weight table.
__device__ __forceinline__ const float *gated_up(const GemmArgs &a, uint32_t slot) {
    const float *wu = reinterpret_cast<const float *>(a.w[1]);
#pragma unroll
    for (int s2 = 1; s2 < kMaxGemmItems; s2++)
        if ((int)slot + 1 == s2) wu = reinterpret_cast<const float *>(a.w[s2]);
    return wu;
}

template <int BM, int BN, int WGM, int WGN, int MINB, bool GATED, int NS = 3, int KS = 1>
__global__ __launch_bounds__(64 * WGM * WGN * KS, MINB) void gemm_f32d_kernel(GemmArgs a) {
    constexpr int NW = WGM * WGN, BK = 32;
    static_assert(NS == 2 || NS == 3, "stages");
    static_assert(KS == 1 || !GATED, "split K: plain epilogue");
    constexpr bool kPersistent = MINB == 1 && KS == 1;  // one block per CU looping over tiles
    constexpr int FM = BM / WGM / 32, FN = BN / WGN / 32;
    constexpr int A_BYTES = BM * BK * 4, S_BYTES = A_BYTES + BN * BK * 4;
    constexpr int AL = A_BYTES / 1024 / NW, BL = BN * BK * 4 / 1024 / NW;  // loads per wave per stage
    constexpr int NDMA = AL + BL;
    static_assert(AL >= 1 && BL >= 1 && AL * 1024 * NW == A_BYTES && BL * 1024 * NW == BN * BK * 4, "loads");
    static_assert(FM >= 1 && FN >= 1 && (!GATED || BN / WGN == 64), "tile");
    static_assert(KS * NS * S_BYTES <= 160 * 1024, "LDS");
    static_assert(KS == 1 || (KS - 1) * NW * FM * FN * 4096 <= KS * NS * S_BYTES, "split-K exchange");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[KS * NS * S_BYTES];

    // persistent (tiles of one block per CU): block b takes tiles
    // xcd_remap(b + i * gridDim.x), i = 0, 1, ... (a multiple of 8 blocks keeps
    // each block on one XCD's run of tiles)
    const uint32_t T = a.total_tiles;
    uint32_t v = blockIdx.x;
    if (v >= T) return;
    constexpr int CPT = GATED ? BN / 2 : BN;  // output columns per tile
    const GemmArgs &ka = kernarg_gemm();  // the same block as `a`
    TileCtx t;
    locate_tile<BM, BN>(ka, xcd_remap(v, T), t, CPT);
    const int tid = threadIdx.x, lane = tid & 63;
    const int grp = KS > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) / NW : 0;  // K group
    const int wave = (tid >> 6) - grp * NW;                                       // wave in the group
    const int li = lane & 31, hf = lane >> 5;
    const int wr = wave / WGN, wc = wave % WGN;
    uint8_t *const ring = smem + grp * NS * S_BYTES;

    const float *asrc[AL];
    const float *bsrc[BL];
    const float *x = reinterpret_cast<const float *>(a.x);
    int kg0 = 0;  // first k of this group
    auto dma = [&](int s) {
        uint8_t *buf = ring + (s % NS) * S_BYTES;
        const int k0 = kg0 + s * BK;
#pragma unroll
        for (int q = 0; q < AL; q++)
            __builtin_amdgcn_global_load_lds(ENC_GLOBAL(asrc[q] + k0), ENC_SHARED(buf + (AL * wave + q) * 1024), 16,
                                             0, 0);
#pragma unroll
        for (int q = 0; q < BL; q++)
            __builtin_amdgcn_global_load_lds(ENC_GLOBAL(bsrc[q] + k0),
                                             ENC_SHARED(buf + A_BYTES + (BL * wave + q) * 1024), 16, 0, 0);
    };
    // the first min(NS, stages) stages of a tile
    auto prologue = [&](int nst) {
        dma(0);
        if (nst > 1) dma(1);
        if (NS > 2 && nst > 2) dma(2);
    };

    // fragment q (k = 16 hf + 4q .. + 3) of X row wr*(BM/WGM) + 32 i + li and
    // of W row wc*(BN/WGN) + 32 j + li: chunk 4 hf + q; 32 rows = 4096 bytes
    const uint32_t lds0 = lds_offset(ring);
    const uint32_t arow = lds0 + (uint32_t)(wr * (BM / WGM) + li) * 128u;
    const uint32_t brow = lds0 + A_BYTES + (uint32_t)(wc * (BN / WGN) + li) * 128u;
    const int sw = (li >> 1) & 7;
    uint32_t abase[4], bbase[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        abase[q] = arow + (uint32_t)(((4 * hf + q) ^ sw) * 16);
        bbase[q] = brow + (uint32_t)(((4 * hf + q) ^ sw) * 16);
    }
    u32x4 fa0[FM], fa1[FM], fb0[FN], fb1[FN];
    auto read = [&](u32x4 (&da)[FM], u32x4 (&db)[FN], int b, int q) {
        const uint32_t so = (uint32_t)(b * S_BYTES);
        ds_read16_run<0, 4096, FM>(da, abase[q] + so);
        ds_read16_run<0, 4096, FN>(db, bbase[q] + so);
    };

    f32x16 acc[FM][FN];
    // k-steps 4q .. 4q+3 of the stage from fragment q.  (Each element is copied
    // out before the reinterpretation: a bit_cast of a vector element
    // expression compiles to element 0 here.)
    auto mma = [&](const u32x4 (&fa)[FM], const u32x4 (&fb)[FN]) {
#pragma unroll
        for (int e = 0; e < 4; e++)
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    const uint32_t ua = fa[i][e], ub = fb[j][e];
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ua), __uint_as_float(ub),
                                                                    acc[i][j], 0, 0, 0);
                }
    };

    f32d_sources<AL, BL, GATED>(x, reinterpret_cast<const float *>(t.w), GATED ? gated_up(ka, t.it.slot) : nullptr,
                                t, wave, lane, asrc, bsrc);
    int nst = t.it.k / BK / KS;
    kg0 = grp * nst * BK;
    prologue(nst);
    if (NS > 2 && nst > 2)
        vm_wait<2 * NDMA>();
    else if (nst > 1)
        vm_wait<NDMA>();
    else
        vm_wait<0>();
    for (;;) {
        block_barrier();
        read(fa0, fb0, 0, 0);
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
        for (int s = 0; s < nst; s++) {
            const int b = s % NS;
            read(fa1, fb1, b, 1);
            lgkm_wait_n<FM + FN>();  // fragment 0 landed (fragment 1 may still be in flight)
            frag_ready(fa0, fb0);
            mma(fa0, fb0);
            read(fa0, fb0, b, 2);
            lgkm_wait_n<FM + FN>();
            frag_ready(fa1, fb1);
            mma(fa1, fb1);
            read(fa1, fb1, b, 3);
            lgkm_wait_n<FM + FN>();
            frag_ready(fa0, fb0);
            mma(fa0, fb0);
            // stage s+1 landed (own loads; with three stages, s+2's may fly), own
            // reads of buffer b done; after the barrier every wave's are, so b
            // takes stage s+NS
            if (NS > 2 && s + 2 < nst)
                vm_wait<NDMA>();
            else
                vm_wait<0>();
            lgkm_wait_n<0>();
            frag_ready(fa1, fb1);
            block_barrier();
            if (s + NS < nst) dma(s + NS);
            if (s + 1 < nst) read(fa0, fb0, (s + 1) % NS, 0);
            mma(fa1, fb1);
        }

        if constexpr (KS > 1) {
            // groups 1 .. KS-1 hand their sums to group 0 through the LDS (every
            // wave is past its last ring read once the barrier is passed);
            // group 0 adds them in increasing group order
            block_barrier();
            float *xch = reinterpret_cast<float *>(smem);
            auto slot = [&](int g, int i, int j) {  // 16 floats per lane, lane-minor
                return xch + ((((g - 1) * NW + wave) * FM + i) * FN + j) * 1024 + lane;
            };
            if (grp > 0) {
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
#pragma unroll
                        for (int r = 0; r < 16; r++) slot(grp, i, j)[64 * r] = acc[i][j][r];
            }
            block_barrier();
            if (grp == 0) {
                for (int g = 1; g < KS; g++)
#pragma unroll
                    for (int i = 0; i < FM; i++)
#pragma unroll
                        for (int j = 0; j < FN; j++)
#pragma unroll
                            for (int r = 0; r < 16; r++) acc[i][j][r] += slot(g, i, j)[64 * r];
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        store_block<false>(a, t, acc[i][j], t.row0 + wr * (BM / WGM) + i * 32,
                                           t.col0 + wc * (BN / WGN) + j * 32, lane);
            }
        } else if constexpr (!GATED) {
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    store_block<false>(a, t, acc[i][j], t.row0 + wr * (BM / WGM) + i * 32,
                                       t.col0 + wc * (BN / WGN) + j * 32, lane);
        } else {
            // lane holds gate and up of the same (row, column)
            const int c = t.col0 + wc * 32 + li;
            if (c < (int)t.it.m) {
                const float mg = a.alpha, mu = a.alpha;
                const bool f16 = a.flags & 1u, gelu = a.flags & kGateGelu;
                const float oc = a.ycol ? a.ycol[c] : 1.0f;
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int row = t.row0 + wr * (BM / WGM) + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (row >= (int)t.it.n) continue;
                        const float g = acc[i][0][r] * mg, u = acc[i][1][r] * mu;
                        const float val = (gelu ? gelu_tanh(g) : silu(g)) * u * oc * a.yscale;
                        const size_t off = t.it.y_off + (size_t)row * t.it.ldy + c;
                        if (f16)
                            reinterpret_cast<_Float16 *>(a.y)[off] = (_Float16)val;
                        else
                            reinterpret_cast<float *>(a.y)[off] = val;
                    }
            }
        }
        // Every wave has passed the last barrier, so no LDS stage is read any
        // more: once this tile's stores are issued, the next tile's first
        // stages are loaded while they drain.  (Stores first: with the loads
        // issued before them, the compiler waits for every load at the top of
        // each k-step of the next tile.)
        // (only the one-block-per-CU tiles loop; smaller ones run a block per tile)
        const uint32_t vn = v + gridDim.x;
        const bool more = kPersistent && vn < T;
        TileCtx tn;
        int nst_n = 0;
        if (more) {
            locate_tile<BM, BN>(ka, xcd_remap(vn, T), tn, CPT);
            f32d_sources<AL, BL, GATED>(x, reinterpret_cast<const float *>(tn.w),
                                        GATED ? gated_up(ka, tn.it.slot) : nullptr, tn, wave, lane, asrc, bsrc);
            nst_n = tn.it.k / BK;
            prologue(nst_n);
        }

        if (!more) break;
        // the next tile's stages (and this tile's stores) have landed
        vm_wait<0>();
        t = tn;
        v = vn;
        nst = nst_n;
    }
}

template <int BM, int BN, int WGM, int WGN, int MINB, bool GATED, int NS = 3, int KS = 1>
hipError_t launch_f32d(GemmArgs g, hipStream_t s) {
    const uint32_t tiles = plan_tiles(g, BM, GATED ? BN / 2 : BN);
    if (!tiles) return hipSuccess;
    // tiles of one block per CU (MINB 1): one block per CU, each looping over
    // its tiles; smaller tiles: one block per tile, the hardware fills the
    // CUs as blocks end
    const uint32_t slots = MINB == 1 && KS == 1 ? (uint32_t)device_cus() : tiles;
    hipLaunchKernelGGL((gemm_f32d_kernel<BM, BN, WGM, WGN, MINB, GATED, NS, KS>), dim3(std::min(tiles, slots)),
                       dim3(64 * WGM * WGN * KS), 0, s, g);
    return hipGetLastError();
}







}  // namespace gemm
}  // namespace enc
