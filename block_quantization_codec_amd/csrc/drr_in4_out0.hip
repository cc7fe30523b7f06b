// drr_in4_out0.hip - hop kernels for 4-bit inputs and a binary32 sum or average.
#include "drr_kernel.h"

namespace zpp {

hipError_t drr_dispatch_in4_out0(int log2b, const DrrArgs &a) {
    return a.divisor > 0.0f ? by_block<4, 0, true>(log2b, a) : by_block<4, 0, false>(log2b, a);
}

}  // namespace zpp
