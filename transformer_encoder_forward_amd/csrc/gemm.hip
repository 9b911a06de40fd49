// Launchers of the item-table GEMM (kernel templates in gemm_impl.h).
//
// The tile shape is chosen per launch from the problem size.  f32: large
// problems take 128 x 128 tiles, small ones (too few 128 x 128 tiles to fill
// the 256 CUs twice over) take 64 x 64 tiles.  int8 x f16: large problems take
// the 256 x 256 kernel fed by direct global -> LDS loads, the rest 128 x 128.
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

constexpr uint32_t kBigTiles = 1024;  // >= 4 tiles per CU at 128 x 128

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s) {
    if (a.flags & (gemm::kGateGelu | gemm::kGateSilu)) {
        if (tiles_of(a, 128, 64) >= kBigTiles) return gemm::launch_gated<128, 128, 32, 2, false, 2>(a, s);
        return gemm::launch_gated<64, 128, 32, 2, false, 4>(a, s);
    }
    if (tiles_of(a, 128, 128) >= kBigTiles) return gemm::launch<128, 128, 32, 2, 4, false, 1>(a, s);
    return gemm::launch_v2<64, 64, 32, 2, 2, false, 4>(a, s);
}

namespace {

// The direct-to-LDS kernel (256 x 256 tiles, one block per CU) needs K % 64 == 0
// and enough tiles to occupy most CUs; otherwise 128 x 128 tiles, two blocks
// per CU.  Both sum in the same K order.
bool k64(const GemmArgs &a) {
    for (uint32_t i = 0; i < a.nitems; i++)
        if (a.items[i].k % 64) return false;
    return true;
}

constexpr uint32_t kWideTiles = 200;

}  // namespace

hipError_t launch_gemm_i8f16(const GemmArgs &a, hipStream_t s) {
    const bool gated = a.flags & (gemm::kGateGelu | gemm::kGateSilu);
    if (k64(a) && tiles_of(a, 256, gated ? 128 : 256) >= kWideTiles)
        return gated ? gemm::launch_q8d<true>(a, s) : gemm::launch_q8d<false>(a, s);
    if (gated) return gemm::launch_gated<128, 128, 64, 2, true, 2>(a, s);
    return gemm::launch<128, 128, 64, 2, 2, true, 2>(a, s);
}

}  // namespace enc
