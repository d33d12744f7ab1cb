// gemv_ternary.hip - instantiations of the decode GEMV for the ternary format
// (one translation unit per format keeps the builds parallel).
#include "gemv_kernel.hpp"

namespace lowbit {

hipError_t gemv_launch_ternary(const GemvParams& p, const GemvCfg& c, hipStream_t stream) {
    switch (c.wpl) {
        case 4: gemv_launch_wpl<FMT_TERNARY, 4>(p, c, stream); break;
        case 2: gemv_launch_wpl<FMT_TERNARY, 2>(p, c, stream); break;
        case 1: gemv_launch_wpl<FMT_TERNARY, 1>(p, c, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lowbit
