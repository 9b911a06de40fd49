// Launchers of the item-table GEMM (kernel template in gemm_impl.h): the
// instantiation is chosen from the shape alone (never from the row count of a
// particular item), so a row's bits do not depend on how it was batched.
#include "gemm_impl.h"

namespace enc {

hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s) {
    if (a.flags & (gemm::kGateGelu | gemm::kGateSilu)) return gemm::launch_gated<128, 128, 32, 2, false, 2>(a, s);
    return gemm::launch<128, 128, 32, 2, 2, false, 2>(a, s);
}

hipError_t launch_gemm_i8f16(const GemmArgs &a, hipStream_t s) {
    if (a.flags & (gemm::kGateGelu | gemm::kGateSilu)) return gemm::launch_gated<128, 128, 64, 2, true, 2>(a, s);
    return gemm::launch<128, 128, 64, 2, 2, true, 2>(a, s);
}

}  // namespace enc
