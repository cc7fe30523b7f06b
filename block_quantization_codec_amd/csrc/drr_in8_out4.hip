// drr_in8_out4.hip - hop kernels for 8-bit inputs and a 4-bit requantized sum.
#include "drr_kernel.h"

namespace zpp {

hipError_t drr_dispatch_in8_out4(int log2b, const DrrArgs &a) { return by_block<8, 4, false>(log2b, a); }

}  // namespace zpp
