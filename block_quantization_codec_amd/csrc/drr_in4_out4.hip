// drr_in4_out4.hip - hop kernels for 4-bit inputs and a 4-bit requantized sum.
#include "drr_kernel.h"

namespace zpp {

hipError_t drr_dispatch_in4_out4(int log2b, const DrrArgs &a) { return by_block<4, 4, false>(log2b, a); }

}  // namespace zpp
