// drr.hip - entry of the hop kernels: picks the unit for the code widths.
//
// Page "Quantized LLM Training at Scale with ZeRO++", section "The Three
// Pillars of ZeRO++", pillar 3 (QGZ): the reduction between the two hops;
// page "ZeRO Stage 2: Gradient Partitioning": the averaged shard. The kernels
// themselves are in drr_kernel.h.
#include "drr_kernel.h"

namespace zpp {

namespace {

hipError_t dispatch(int bits_in, int bits_out, int log2b, const DrrArgs &a) {
    if (bits_in == 8) {
        switch (bits_out) {
        case 0: return drr_dispatch_in8_out0(log2b, a);
        case 4: return drr_dispatch_in8_out4(log2b, a);
        case 8: return drr_dispatch_in8_out8(log2b, a);
        default: return hipErrorInvalidValue;
        }
    }
    switch (bits_out) {
    case 0: return drr_dispatch_in4_out0(log2b, a);
    case 4: return drr_dispatch_in4_out4(log2b, a);
    case 8: return drr_dispatch_in4_out8(log2b, a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_drr(const void *codes_in, int64_t codes_stride, const float *scales_in, int64_t scales_stride,
                      int n_inputs, int bits_in, int64_t numel, int log2b, void *codes_out, float *scales_out,
                      int bits_out, float *sum_out, hipStream_t stream) {
    return dispatch(bits_in, bits_out, log2b,
                    DrrArgs{codes_in, codes_stride, scales_in, scales_stride, n_inputs, numel, codes_out, scales_out,
                            sum_out, 0.0f, stream});
}

hipError_t launch_drr_split(const void *codes_in, int64_t codes_stride, const float *scales_in,
                            int64_t scales_stride, int n_inputs, int bits_in, int64_t numel, int log2b,
                            int64_t keep_begin, int64_t keep_len, void *codes_send, float *scales_send,
                            void *codes_keep, float *scales_keep, int bits_out, hipStream_t stream) {
    DrrArgs a{codes_in, codes_stride, scales_in, scales_stride, n_inputs, numel, codes_send, scales_send,
              nullptr, 0.0f, stream};
    a.keep_begin = keep_begin;
    a.keep_len = keep_len;
    a.codes_keep = codes_keep;
    a.scales_keep = scales_keep;
    return dispatch(bits_in, bits_out, log2b, a);
}

hipError_t launch_drr_average(const void *codes_in, int64_t codes_stride, const float *scales_in,
                              int64_t scales_stride, int n_inputs, int bits_in, int64_t numel, int log2b,
                              int divisor, float *avg_out, hipStream_t stream) {
    return dispatch(bits_in, 0, log2b,
                    DrrArgs{codes_in, codes_stride, scales_in, scales_stride, n_inputs, numel, nullptr, nullptr,
                            avg_out, static_cast<float>(divisor), stream});
}

}  // namespace zpp
