// Launchers of the item-table GEMM (kernel templates in gemm_impl.h).
//
// The tile shape is chosen per launch from the problem size.  f32: launches
// with about one 256 x 128 tile per CU or more take 256 x 128 tiles (gated: 256
// rows x 128 outputs), smaller ones 64 x 64 (gated: 64 x 64 outputs); with
// K % 32 == 0 the operands reach LDS by direct global -> LDS loads, otherwise
// through registers.  int8 x f16: the kernel fed by
// direct global -> LDS loads (256 x 256 tiles for large launches, 64 x 256 /
// gated 128 x 256 for smaller ones), and otherwise the register-staged
// 128 x 128.
// Every instantiation of one path uses the same K stage and the same lane-half
// K order, so an output element is summed in the same order whatever tile it
// falls in: the choice never changes a result bit, and packed and separate
// batches stay bit-identical.
#include "gemm_impl.h"

namespace enc {

namespace {

// number of BM x BN tiles of the launch (gated items count BN/2 output columns)
uint32_t tiles_of(const GemmArgs &a, int BM, int BN) {
    uint32_t t = 0;
    for (uint32_t i = 0; i < a.nitems; i++)
        t += ((a.items[i].n + BM - 1) / BM) * ((a.items[i].m + BN - 1) / BN);
    return t;
}

constexpr uint32_t kWideF32 = 240;  // about one 256 x 128 tile per CU

}  // namespace

static bool kmul(const GemmArgs &a, uint32_t q) {
    for (uint32_t i = 0; i < a.nitems; i++)
        if (a.items[i].k % q) return false;
    return true;
}

// f32, measured on the 16 057-row text encoder and the 1024-row ViT (min of
// interleaved runs, same-run comparisons):
//  - plain GEMMs with K % 32 == 0 take the direct-to-LDS kernel: 256 x 128
//    tiles of 16 waves (64 x 32 each) beat the register-staged 256 x 128 tile
//    by 8-13% on the text encoder's q/k/v, O and down projections; 64 x 64
//    tiles (4 waves, up to four blocks per CU) beat the register-staged 64 x 64
//    by 4-12% on the ViT's;
//  - gated GEMMs of large launches take the direct-to-LDS 256 x (128 + 128)
//    tile of 16 waves with two 64 KB stages: 6% faster than the register-staged
//    tile of the same shape, which in turn beats 128 x (64 + 64) by 6%; small
//    ones (the 2176-row vision tower) the direct-to-LDS 64 x (64 + 64) tile, 7%
//    faster than the register-staged one.
// Plain f32 items with at most 768 outputs and K >= 3072 (K % 128 == 0; the
// vision towers' down projections) are summed with K split four ways inside
// the block (gemm_f32d_kernel, KS = 4): their launches give few output tiles
// (a 1024-row batch: 192 of 64 x 64 for 256 CUs), and four groups of waves
// per tile hide the latencies one wave per SIMD leaves exposed.  The choice
// follows the item's weight shape alone, so a row gets the same bits in any
// batch; a launch that mixes such items with others is issued as two.
// Measured on the 1024-row ViT's down projection: 69.2 -> 58.2 us (two-way
// split 59.9); the 2176-row vision tower's: unchanged (111.5 us).
static bool f32_split_item(const GemmItemK &it) { return it.m <= 768 && it.k >= 3072 && it.k % 128 == 0; }

static hipError_t launch_gemm_f32_unsplit(const GemmArgs &a, hipStream_t s);

hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s) {
    if (a.flags & (gemm::kGateGelu | gemm::kGateSilu)) return launch_gemm_f32_unsplit(a, s);
    GemmArgs sp = a, un = a;
    sp.nitems = un.nitems = 0;
    for (uint32_t i = 0; i < a.nitems; i++) {
        if (f32_split_item(a.items[i]))
            sp.items[sp.nitems++] = a.items[i];
        else
            un.items[un.nitems++] = a.items[i];
    }
    if (sp.nitems) {
        const hipError_t h = gemm::launch_f32d<64, 64, 2, 2, 1, false, 2, 4>(sp, s);
        if (h != hipSuccess || !un.nitems) return h;
    }
    return launch_gemm_f32_unsplit(un, s);
}

static hipError_t launch_gemm_f32_unsplit(const GemmArgs &a, hipStream_t s) {
    const bool direct = kmul(a, 32);
    if (a.flags & (gemm::kGateGelu | gemm::kGateSilu)) {
        if (tiles_of(a, 256, 128) >= kWideF32)
            return direct ? gemm::launch_f32d<256, 256, 4, 4, 1, true, 2>(a, s)
                          : gemm::launch_gated<256, 256, 32, 4, false, 1>(a, s);
        return direct ? gemm::launch_f32d<64, 128, 2, 2, 4, true>(a, s) : gemm::launch_gated<64, 128, 32, 2, false, 4>(a, s);
    }
    if (tiles_of(a, 256, 128) >= kWideF32)
        return direct ? gemm::launch_f32d<256, 128, 4, 4, 1, false>(a, s) : gemm::launch<256, 128, 32, 4, 2, false, 1>(a, s);
    return direct ? gemm::launch_f32d<64, 64, 2, 2, 4, false>(a, s) : gemm::launch_v2<64, 64, 32, 2, 2, false, 4>(a, s);
}

namespace {

// The direct-to-LDS int8 kernel needs K % 64 == 0.  Plain GEMMs: 256 x 256
// tiles (8 waves of 128 x 64, one block per CU) when the launch has at least
// 384 of them, or at least 256 that the smaller tiles below cannot take in
// one round of two blocks per CU (with 256 to 383 tiles of 256 x 256 the
// second round leaves most CUs idle: 1300 rows' q|k|v ran at 183 us on
// 270 tiles).  Fewer take tiles that fill the CUs in one round of two blocks
// each: 96 x 256 tiles of 4 waves (96 x 64 each: each W fragment widened for
// 96 rows) with a two-stage ring when at most 512 of them cover the launch
// (the 1056-row q|k|v: 495 tiles, 10% faster than 405 tiles of 128 x 256);
// else 128 x 256 tiles of 8 waves (64 x 64 each) with a two-stage ring when
// at most 512 of them do; else 64 x 256 tiles of 8 waves (64 x 32 each; the
// 1056-row output and down projections: 255 tiles, 56% and 48% faster than
// 256 x 256 there).  32 x 256 and 64 x 128 tiles were measured no faster than
// 64 x 256 on the output and down projections, and 8 waves of 64 x 128 in the
// 256 x 256 tile 3% slower than 128 x 64 at 8448 rows.  Gated: 256 x (128 +
// 128) with at least 512 tiles of 256 x 128; else the one of 256, 192 and 128
// rows (one block per CU each; 192 and 128 with four- and five-stage rings,
// the whole LDS) with the fewest rounds of the CUs times rows per tile over
// the tile's relative rate (1, 0.95, 0.8: the larger the wave's row span, the
// fewer widenings per MFMA).  At 1056 rows that is 192 x (128 + 128): 480
// tiles in two rounds, 10% faster than 720 tiles of 128 rows (three rounds),
// which were 6% faster than 400 tiles of 256 rows.  Otherwise (K % 64 != 0,
// or an item too large for the direct loads' 32-bit offsets) the
// register-staged 128 x 128 kernel.  All sum in the same K order, so the
// choice never changes a bit.

}  // namespace

// The direct-load kernel addresses X and W by 32-bit byte offsets from the
// item's X and the weight matrix: both must stay below 2^31.
static bool offsets32(const GemmArgs &a) {
    for (uint32_t i = 0; i < a.nitems; i++) {
        const GemmItemK &it = a.items[i];
        const uint64_t xb = ((uint64_t)(it.n ? it.n - 1 : 0) * it.ldx + it.k) * 2, wb = (uint64_t)it.m * it.k;
        if (xb >= (1ull << 31) || wb >= (1ull << 31)) return false;
    }
    return true;
}

hipError_t launch_gemm_i8f16(const GemmArgs &a, hipStream_t s) {
    const bool gated = a.flags & (gemm::kGateGelu | gemm::kGateSilu);
    if (kmul(a, 64) && offsets32(a)) {
        // the thresholds are in units of the device's CUs (256 on MI355X):
        // one block per CU for the 256-row tiles, two for the smaller ones
        const uint32_t cus = (uint32_t)gemm::device_cus(), kWideTiles = cus, kWideGated = 2 * cus,
                       kSlots = 2 * cus;
        if (gated) {
            if (tiles_of(a, 256, 128) >= kWideGated) {
                // a one-item launch whose last round of 256-row tiles leaves
                // most CUs idle issues the rows of its last 256-row tile as a
                // second launch of 128-row tiles, when rounds x rows / rate
                // (as below) says so
                const GemmItemK &it = a.items[0];
                if (a.nitems == 1 && it.n > 256) {
                    const uint32_t last = it.n - (it.n - 1) / 256 * 256;  // rows of the last row tile
                    const uint32_t ct = (it.m + 127) / 128, t_all = tiles_of(a, 256, 128), t_head = t_all - ct;
                    const uint32_t t_tail = ct * ((last + 127) / 128);
                    const double c_all = (double)((t_all + cus - 1) / cus) * 256;
                    const double c_peel =
                        (double)((t_head + cus - 1) / cus) * 256 + (double)((t_tail + cus - 1) / cus) * 128 / 0.8;
                    if (c_peel < c_all) {
                        GemmArgs head = a, tail = a;
                        head.items[0].n = it.n - last;
                        tail.items[0].n = last;
                        tail.items[0].x_off += (uint64_t)(it.n - last) * it.ldx;
                        tail.items[0].y_off += (uint64_t)(it.n - last) * it.ldy;
                        const hipError_t h = gemm::launch_q8d<256, 256, 2, 4, 1, true>(head, s);
                        if (h != hipSuccess) return h;
                        return gemm::launch_q8d<128, 256, 2, 4, 1, true, 5>(tail, s);
                    }
                }
                return gemm::launch_q8d<256, 256, 2, 4, 1, true>(a, s);
            }
            // one block per CU for every gated tile: rounds of the CUs times
            // the tile's rows over its measured relative rate
            const auto cost = [&](int bm, double rate) {
                return (double)((tiles_of(a, bm, 128) + cus - 1) / cus) * bm / rate;
            };
            const double c256 = cost(256, 1.0), c192 = cost(192, 0.95), c128 = cost(128, 0.8);
            if (c256 <= c192 && c256 <= c128) return gemm::launch_q8d<256, 256, 2, 4, 1, true>(a, s);
            return c192 <= c128 ? gemm::launch_q8d<192, 256, 2, 4, 1, true, 4>(a, s)
                                : gemm::launch_q8d<128, 256, 2, 4, 1, true, 5>(a, s);
        }
        // 256 x 256 unless it leaves most CUs idle in a second round that the
        // two-per-CU 128 x 256 tiles avoid
        const uint32_t t256 = tiles_of(a, 256, 256);
        if (t256 >= kWideTiles && (t256 >= kWideTiles * 3 / 2 || tiles_of(a, 128, 256) > kSlots))
            return gemm::launch_q8d<256, 256, 2, 4, 1, false>(a, s);
        if (tiles_of(a, 64, 256) > kSlots && tiles_of(a, 96, 256) <= kSlots)
            return gemm::launch_q8d<96, 256, 1, 4, 2, false, 2>(a, s);
        if (tiles_of(a, 64, 256) > kSlots && tiles_of(a, 128, 256) <= kSlots)
            return gemm::launch_q8d<128, 256, 2, 4, 2, false, 2>(a, s);
        return gemm::launch_q8d<64, 256, 1, 8, 2, false>(a, s);
    }
    if (gated) return gemm::launch_gated<128, 128, 64, 2, true, 2>(a, s);
    return gemm::launch<128, 128, 64, 2, 2, true, 2>(a, s);
}

}  // namespace enc
