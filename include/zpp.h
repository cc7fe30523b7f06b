/*
 * zpp.h - C ABI of the ZeRO++ block-quantization codec on AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * The library is the per-GPU arithmetic of ZeRO++'s communication reduction:
 * block quantization of weights before the forward all-gather (qwZ), the
 * gather-side dequantization, and the gradient path of qgZ (tensor-slice
 * reordering, one-shot 4-bit quantization, and the dequantize-reduce-
 * requantize step between the two hops of its hierarchical all-to-all).
 * It moves no data between GPUs: the caller's collectives do that.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer (memory the current GPU can
 *   address: hipMalloc'd on it or on a peer it can access, or
 *   hipHostMalloc'd pinned host memory). Ordinary host memory, and another
 *   GPU's memory without peer access, are rejected with ZPP_ERR_POINTER.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *   null stream). The call validates all arguments on the host first; if any
 *   check fails it returns an error code, launches nothing and leaves every
 *   output untouched. Faults during execution surface at the caller's next
 *   synchronization of the stream, as with any HIP kernel. Right before
 *   its launch a call reads and clears the calling thread's pending HIP
 *   error (hipGetLastError), so an error left there by an earlier call does
 *   not survive it; a rejected launch returns ZPP_ERR_LAUNCH and leaves no
 *   error pending. The hop reductions launch once per 2^29 output elements;
 *   if a later launch is rejected, the earlier ones still run, so after
 *   ZPP_ERR_LAUNCH the outputs are unspecified.
 * - The caller allocates and owns every buffer; the library allocates
 *   nothing, keeps no per-call state and may be called from several threads
 *   and streams at once. Outputs must not overlap inputs or each other
 *   (ZPP_ERR_OVERLAP); inputs may overlap each other.
 * - Block quantization layout (structure of arrays): for `numel` elements
 *   and block size B, block b holds elements [b*B, (b+1)*B). `codes` holds
 *   numel*bits/8 bytes: 8-bit codes are two's-complement bytes; 4-bit codes
 *   are two's-complement nibbles, element 2i in the low nibble of byte i.
 *   `scales` holds numel/B binary32 scales s_b (the scale itself, not its
 *   inverse). An element's value is code * s_b.
 * - B is a power of two in [ZPP_MIN_BLOCK, ZPP_MAX_BLOCK]; 0 <= numel <=
 *   ZPP_MAX_NUMEL and numel % B == 0 (callers pad; zero padding changes no
 *   scale and no sum). numel == 0 is a no-op returning ZPP_OK.
 * - Alignment: element data and code pointers 16-byte aligned, scale
 *   pointers 4-byte aligned (ZPP_ERR_ALIGN otherwise).
 *
 * Sources (pages as published, by title and section):
 *   [QWZ] "Quantized LLM Training at Scale with ZeRO++", section "The Three
 *         Pillars of ZeRO++", pillar 1 (QWZ): weights are quantized chunk by
 *         chunk (block quantization) and all-gathered as 8-bit values.
 *   [QGZ] same page and section, pillar 3 (QGZ): one-shot gradient
 *         quantization, two-hop all-to-all (intra-node exchange and
 *         reduction, then inter-node exchange), tensor-slice reordering
 *         before any communication; gradient volume cut to a quarter.
 *   [RS]  "ZeRO Stage 2: Gradient Partitioning": after the reduce-scatter,
 *         GPU i holds the reduced gradient of shard i.
 *   [ZPP2] "ZeRO-1/2/3", section "ZeRO++": quantized weights may be 8- or
 *         4-bit.
 *   [AVG] "ZeRO Stage 2: Gradient Partitioning", the numbered steps of the
 *         stage-2 flow, step 2: the reduce-scatter averages the gradients
 *         over all GPUs, and GPU i keeps the average of shard i.
 * Quantization rule (the pages name block quantization but print no
 * formula; this is the symmetric absmax reading the library implements):
 *   a_b = max |x| over block b;  s_b = a_b / Q rounded once to binary32,
 *   Q = 127 for 8-bit and 7 for 4-bit codes; code = round-half-even of the
 *   correctly rounded binary32 quotient x / s_b, clamped to [-Q, Q];
 *   a block whose scale is 0 gets all-zero codes.
 */
#ifndef ZPP_H
#define ZPP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZPP_ABI_VERSION 2
#define ZPP_MIN_BLOCK 32
#define ZPP_MAX_BLOCK 4096
#define ZPP_MAX_INPUTS 4096
#define ZPP_MAX_DIVISOR 16777216 /* 2^24: every divisor up to it is exact in binary32 */
/* 2^40: the largest element count, input stride (bytes for codes, floats
 * for scales), and reordered buffer (elements, or bytes / 4) accepted; far
 * beyond any GPU's memory, it keeps every byte range of a call exact in
 * 64-bit arithmetic (larger values: ZPP_ERR_ARG). */
#define ZPP_MAX_NUMEL ((int64_t)1 << 40)

typedef enum zpp_status {
    ZPP_OK = 0,
    ZPP_ERR_NULL = 1,        /* a required pointer is NULL                        */
    ZPP_ERR_ARG = 2,         /* size, block, bit width, count or stride invalid   */
    ZPP_ERR_ALIGN = 3,       /* pointer or stride not aligned as required         */
    ZPP_ERR_UNSUPPORTED = 4, /* valid request the library does not implement      */
    ZPP_ERR_LAUNCH = 5,      /* the HIP runtime reported an error for the launch  */
    /* Beyond the five error kinds above, the library tells apart two more
     * argument errors; they come after ZPP_ERR_LAUNCH so that codes 0-5
     * keep their meaning for callers that know only those. */
    ZPP_ERR_OVERLAP = 6,     /* an output overlaps an input or another output     */
    ZPP_ERR_POINTER = 7      /* a pointer is not memory the GPU can address       */
} zpp_status;

typedef enum zpp_dtype {
    ZPP_BF16 = 1, /* bfloat16 */
    ZPP_FP32 = 2  /* IEEE-754 binary32 */
} zpp_dtype;

/* Element types and status codes cross the ABI as int32_t parameters (one of
 * the enumerators above), so that any value a caller passes is well defined
 * and is refused (ZPP_ERR_ARG, or "unknown zpp_status"). */

/*
 * Block-quantize `numel` elements of `x` to `bits`-bit codes and per-block
 * scales. [QWZ] (8-bit weights before the forward all-gather) and [QGZ]
 * (the one-shot 4-bit gradient quantization before the all-to-all).
 *
 *   x        in   numel elements of x_dtype (ZPP_BF16 or ZPP_FP32), 16-B aligned
 *   numel    in   element count, multiple of `block`, <= ZPP_MAX_NUMEL
 *   block    in   block size B (power of two, 32..4096)
 *   bits     in   8 or 4
 *   codes    out  numel*bits/8 bytes, 16-B aligned
 *   scales   out  numel/block floats, 4-B aligned
 *   stream   in   hipStream_t
 * Non-finite inputs are outside the contract (they cannot fault the GPU,
 * but their codes are unspecified).
 */
zpp_status zpp_quantize_blocks(const void *x, int32_t x_dtype, int64_t numel,
                               int32_t block, int32_t bits, void *codes, float *scales,
                               void *stream);

/*
 * Tensor-slice reordering fused into the one-shot quantization [QGZ] (the
 * page lists kernel fusion among the QGZ optimizations): quantizes the
 * reordered view of x (see zpp_reorder_slices) without writing it out.
 * x holds N = n_nodes * gpus_per_node slices of slice_elems elements in
 * their original order; output slice positions
 * [first_slice, first_slice + n_slices) of the reordered buffer are
 * quantized, and their codes and scales are written contiguously, exactly
 * as zpp_quantize_blocks would write them for those slices of the
 * reordered buffer (blocks never straddle slices). Choosing the range lets a
 * caller quantize the chunk it keeps straight into its receive buffer.
 *
 *   x               in   N * slice_elems elements of x_dtype, 16-B aligned
 *   slice_elems     in   multiple of `block`; N * slice_elems <= ZPP_MAX_NUMEL
 *   n_nodes, gpus_per_node  in  >= 1 each, product <= 65535
 *   first_slice, n_slices   in  0 <= first_slice, first_slice + n_slices <= N
 *   block, bits     in   as zpp_quantize_blocks
 *   codes           out  n_slices * slice_elems * bits / 8 bytes, 16-B aligned
 *   scales          out  n_slices * slice_elems / block floats, 4-B aligned
 *   stream          in   hipStream_t
 */
zpp_status zpp_quantize_reordered(const void *x, int32_t x_dtype, int64_t slice_elems, int32_t n_nodes,
                                  int32_t gpus_per_node, int32_t first_slice, int32_t n_slices, int32_t block,
                                  int32_t bits, void *codes, float *scales, void *stream);

/*
 * Rebuild values from codes and scales: y = code * s_b in binary32, then
 * rounded to nearest-even for ZPP_BF16 output. [QWZ] (the receiver of the
 * 8-bit all-gather needs 16-bit weights to compute with) and [ZPP2].
 *
 *   codes    in   numel*bits/8 bytes, 16-B aligned
 *   scales   in   numel/block floats, 4-B aligned
 *   bits     in   8 or 4 (any code value is accepted, including -128 / -8)
 *   numel    in   element count, multiple of `block`, <= ZPP_MAX_NUMEL
 *   block    in   block size B
 *   y        out  numel elements of y_dtype (ZPP_BF16 or ZPP_FP32), 16-B aligned
 *   stream   in   hipStream_t
 */
zpp_status zpp_dequantize_blocks(const void *codes, const float *scales, int32_t bits,
                                 int64_t numel, int32_t block, void *y, int32_t y_dtype,
                                 void *stream);

/*
 * Tensor-slice reordering before the two-hop exchange [QGZ], so that after
 * hop 1 (contiguous chunk j to local rank j) and hop 2 (sub-chunk k of it
 * to node k) every rank holds its own shard [RS]. The buffer is
 * N = n_nodes * gpus_per_node equal slices of `slice_bytes` bytes; ranks
 * are node-major (rank = node * gpus_per_node + local). Output slice
 * position j*n_nodes + k receives input slice k*gpus_per_node + j.
 * Byte-wise: works on any element type, and commutes with block
 * quantization when every slice is a whole number of blocks.
 *
 *   in, out      in/out  N * slice_bytes bytes each, out-of-place
 *   slice_bytes  in      >= 0; any value (vector width adapts to alignment);
 *                        N * slice_bytes <= 4 * ZPP_MAX_NUMEL
 *   n_nodes, gpus_per_node  in  >= 1 each, product <= 65535
 *   stream       in      hipStream_t
 */
zpp_status zpp_reorder_slices(const void *in, void *out, int64_t slice_bytes, int32_t n_nodes,
                              int32_t gpus_per_node, void *stream);

/*
 * The fused hop step of qgZ [QGZ]: dequantize n_inputs received pieces,
 * sum them in binary32 in ascending input order (each product and each sum
 * rounded on its own: no product is fused into the sum), and either
 * requantize the sum for the next hop (hop 1, intra-node reduction) or emit
 * it as binary32 (hop 2, the owner's reduced shard [RS]). It sums; it does
 * not average.
 *
 *   codes_in            in   input r's codes at codes_in + r*codes_stride_bytes
 *   codes_stride_bytes  in   0..ZPP_MAX_NUMEL, multiple of 16
 *   scales_in           in   input r's scales at scales_in + r*scales_stride
 *   scales_stride       in   0..ZPP_MAX_NUMEL, in floats
 *   n_inputs            in   1..ZPP_MAX_INPUTS
 *   bits_in             in   8 or 4
 *   numel, block        in   elements per input (<= ZPP_MAX_NUMEL) and block size B (same B for
 *                            the inputs and the requantized output)
 *   codes_out, scales_out, bits_out
 *                       out  requantized sum (bits_out 8 or 4), or
 *                            NULL, NULL, 0 to skip requantization
 *   sum_out             out  binary32 sum (numel floats, 16-B aligned), or NULL
 *   stream              in   hipStream_t
 * At least one of the two outputs must be requested (ZPP_ERR_ARG).
 * Any code bytes and any finite scales are accepted; the binary32 sum is
 * exact to the contract for all of them. A sum that overflows to infinity
 * (only possible with scales near the binary32 limit) is outside the
 * contract for requantization: that block's codes and scale are unspecified.
 */
zpp_status zpp_dequant_reduce_requant(const void *codes_in, int64_t codes_stride_bytes,
                                      const float *scales_in, int64_t scales_stride,
                                      int32_t n_inputs, int32_t bits_in, int64_t numel,
                                      int32_t block, void *codes_out, float *scales_out,
                                      int32_t bits_out, float *sum_out, void *stream);

/*
 * The hop-1 step of qgZ [QGZ] with its output split the way the next hop
 * needs it: the same binary32 input-order sum as zpp_dequant_reduce_requant,
 * requantized, with the requantized codes and scales of the elements in
 * [keep_begin, keep_begin + keep_elems) written to codes_keep / scales_keep
 * (the piece this GPU keeps for itself in hop 2: its own sub-chunk, which
 * goes straight into its slot of the hop-2 receive buffer), and those of
 * all other elements written to codes_send / scales_send, in element order
 * with the kept window left out (what the inter-node all-to-all sends). One
 * pass over the inputs; both outputs are exactly the corresponding parts of
 * zpp_dequant_reduce_requant's output.
 *
 *   codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs,
 *   bits_in, numel, block   in   as zpp_dequant_reduce_requant
 *   keep_begin, keep_elems  in   the kept window, whole blocks:
 *                                0 <= keep_begin <= keep_begin + keep_elems <= numel
 *   codes_send   out  (numel - keep_elems) * bits_out / 8 bytes, 16-B aligned
 *   scales_send  out  (numel - keep_elems) / block floats, 4-B aligned
 *                     (both may be NULL when keep_elems == numel)
 *   codes_keep   out  keep_elems * bits_out / 8 bytes, 16-B aligned
 *   scales_keep  out  keep_elems / block floats, 4-B aligned
 *                     (both may be NULL when keep_elems == 0)
 *   bits_out     in   8 or 4
 *   stream       in   hipStream_t
 * Errors as zpp_dequant_reduce_requant's, and ZPP_ERR_ARG for a window that
 * is not whole blocks or does not lie inside [0, numel); ZPP_ERR_OVERLAP
 * when any two of the four outputs overlap.
 */
zpp_status zpp_dequant_reduce_requant_split(const void *codes_in, int64_t codes_stride_bytes,
                                            const float *scales_in, int64_t scales_stride,
                                            int32_t n_inputs, int32_t bits_in, int64_t numel,
                                            int32_t block, int64_t keep_begin, int64_t keep_elems,
                                            void *codes_send, float *scales_send, void *codes_keep,
                                            float *scales_keep, int32_t bits_out, void *stream);

/*
 * The final hop of qgZ writing the optimizer-ready shard [QGZ][AVG]: the same
 * input-order binary32 sum as zpp_dequant_reduce_requant, then divided by
 * `divisor`, the number of GPUs whose gradients the sum holds (for the
 * two-hop exchange, n_nodes * gpus_per_node, not n_inputs), with one
 * correctly rounded binary32 division per element. A power-of-two divisor
 * only lowers the exponent (exact unless the result is subnormal).
 *
 *   codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs,
 *   bits_in, numel, block   in   as zpp_dequant_reduce_requant
 *   divisor             in   1..ZPP_MAX_DIVISOR (1 gives the plain sum)
 *   avg_out             out  numel floats, 16-B aligned
 *   stream              in   hipStream_t
 */
zpp_status zpp_dequant_reduce_average(const void *codes_in, int64_t codes_stride_bytes,
                                      const float *scales_in, int64_t scales_stride,
                                      int32_t n_inputs, int32_t bits_in, int64_t numel,
                                      int32_t block, int32_t divisor, float *avg_out, void *stream);

/*
 * Switch the library's HIP-runtime pointer checks on (enabled != 0, the
 * default) or off for the whole process; returns the previous setting (1 or
 * 0). With the checks on, every call asks the HIP runtime, before it
 * launches anything, whether each pointer is memory the current GPU can
 * address (ZPP_ERR_POINTER otherwise) and whether each buffer's byte range
 * lies inside its allocation (ZPP_ERR_ARG otherwise), about 0.2 us of host
 * time per buffer. With them off, those two checks are skipped: the caller
 * guarantees that every pointer it passes is device-addressable and that
 * every buffer is as long as the call's sizes imply, and a call that breaks
 * this faults the GPU instead of returning an error. Every other check (NULL
 * pointers, sizes, block, bit widths, strides, alignment, overlapping
 * outputs) always runs. Safe to call from any thread; calls already past
 * their checks are not affected.
 */
int32_t zpp_set_pointer_checks(int32_t enabled);

/* Static, human-readable name of a status code (a zpp_status value); any
 * other value gives "unknown zpp_status". Never NULL. */
const char *zpp_status_string(int32_t status);

/* ZPP_ABI_VERSION of the loaded library. */
int32_t zpp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZPP_H */
