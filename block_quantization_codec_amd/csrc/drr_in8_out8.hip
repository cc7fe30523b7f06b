// drr_in8_out8.hip - hop kernels for 8-bit inputs and a 8-bit requantized sum.
#include "drr_kernel.h"

namespace zpp {

hipError_t drr_dispatch_in8_out8(int log2b, const DrrArgs &a) { return by_block<8, 8, false>(log2b, a); }

}  // namespace zpp
