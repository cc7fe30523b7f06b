// zpp_launch.h - internal launchers, one per kernel family. Arguments are
// already validated by the C ABI layer; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zpp {

hipError_t launch_quantize(const void *x, bool f32_in, int64_t numel, int log2b, int bits, void *codes,
                           float *scales, hipStream_t stream);

hipError_t launch_quantize_reordered(const void *x, bool f32_in, int64_t slice_elems, int n_nodes, int gpus_per_node,
                                     int first_slice, int n_slices, int log2b, int bits, void *codes, float *scales,
                                     hipStream_t stream);

hipError_t launch_dequantize(const void *codes, const float *scales, int bits, int64_t numel, int log2b,
                             void *y, bool f32_out, hipStream_t stream);

hipError_t launch_reorder(const void *in, void *out, int64_t slice_bytes, int n_nodes, int gpus_per_node,
                          hipStream_t stream);

hipError_t launch_drr(const void *codes_in, int64_t codes_stride, const float *scales_in, int64_t scales_stride,
                      int n_inputs, int bits_in, int64_t numel, int log2b, void *codes_out, float *scales_out,
                      int bits_out, float *sum_out, hipStream_t stream);

hipError_t launch_drr_split(const void *codes_in, int64_t codes_stride, const float *scales_in,
                            int64_t scales_stride, int n_inputs, int bits_in, int64_t numel, int log2b,
                            int64_t keep_begin, int64_t keep_len, void *codes_send, float *scales_send,
                            void *codes_keep, float *scales_keep, int bits_out, hipStream_t stream);

hipError_t launch_drr_average(const void *codes_in, int64_t codes_stride, const float *scales_in,
                              int64_t scales_stride, int n_inputs, int bits_in, int64_t numel, int log2b,
                              int divisor, float *avg_out, hipStream_t stream);

}  // namespace zpp
