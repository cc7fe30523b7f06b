// drr_in4_out8.hip - hop kernels for 4-bit inputs and a 8-bit requantized sum.
#include "drr_kernel.h"

namespace zpp {

hipError_t drr_dispatch_in4_out8(int log2b, const DrrArgs &a) { return by_block<4, 8, false>(log2b, a); }

}  // namespace zpp
