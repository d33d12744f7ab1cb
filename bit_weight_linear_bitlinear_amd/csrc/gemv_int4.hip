// gemv_int4.hip - instantiations of the decode GEMV for the int4 format
// (one translation unit per format keeps the builds parallel).
#include "gemv_kernel.hpp"

namespace lowbit {

hipError_t gemv_launch_int4(const GemvParams& p, const GemvCfg& c, hipStream_t stream) {
    switch (c.wpl) {
        case 4: gemv_launch_wpl<FMT_INT4, 4>(p, c, stream); break;
        case 2: gemv_launch_wpl<FMT_INT4, 2>(p, c, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lowbit
