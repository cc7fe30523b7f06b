/*
 * zpp_oracle.c - plain, slow CPU oracle of the ZeRO++ block-quantization codec.
 *
 * TEST INFRASTRUCTURE ONLY. Tests, the smoke check and the benchmark's CPU
 * baseline may load this; the product library never does, and this file
 * shares no code, header, table or helper with it.
 *
 * Built with the host C compiler: -O2 -ffp-contract=off, no fast-math, SSE
 * single precision (x86-64 default, no x87), so every float operation below
 * is one IEEE-754 binary32 operation rounded to nearest-even, as written.
 *
 * Sources (pages as published; section names as they appear there):
 *   [QWZ]  "Quantized LLM Training at Scale with ZeRO++", section "The Three
 *          Pillars of ZeRO++", pillar 1 (QWZ): the weight tensor is cut into
 *          small chunks and each chunk is quantized on its own (block
 *          quantization), sending 8-bit instead of 16-bit weights.
 *   [QGZ]  same page and section, pillar 3 (QGZ): one-shot quantization of
 *          each GPU's gradient before an all-to-all; a two-hop protocol
 *          (intra-node all-to-all plus reduction, then inter-node all-to-all);
 *          a tensor-slice reordering before any communication so that every
 *          slice ends on its owner; gradient volume cut to a quarter.
 *   [RS]   "ZeRO Stage 2: Gradient Partitioning" (ZeRO Optimization series),
 *          the reduce-scatter step: GPU i ends with the reduced gradient of
 *          parameter shard i.
 *   [ZPP2] "ZeRO-1/2/3" (compassingai concept page), section "ZeRO++":
 *          qwZ weights may be int8 or int4.
 *   [AVG]  "ZeRO Stage 2: Gradient Partitioning", the numbered steps of the
 *          stage-2 flow, step 2: the reduce-scatter averages the gradients
 *          over all GPUs, and GPU i keeps the average for shard i.
 *
 * Readings taken where the pages are silent (each is a choice, not a fact
 * printed on the pages):
 *   - symmetric per-block absmax quantization: a = max|x| over the block,
 *     s = a / Q in binary32 (one correctly rounded division), Q = 127 for
 *     8-bit codes and 7 for 4-bit codes; the code is x / s (correctly
 *     rounded binary32 division), rounded to the nearest integer with ties
 *     to even, then clamped to [-Q, Q]; a block with s == 0 has all codes 0;
 *   - codes and scales are separate arrays; scales are binary32 s (not 1/s);
 *   - 4-bit codes are two's-complement nibbles, element 2i in the low nibble
 *     of byte i; 8-bit codes are two's-complement bytes;
 *   - dequantization is the binary32 product code * scale, and a bfloat16
 *     result is that product rounded to nearest-even;
 *   - the hop reduction sums, in binary32, each input's dequantized value in
 *     ascending input order starting from +0.0f, every product and every
 *     sum rounded on its own (no fused multiply-add); it sums, it does not
 *     average;
 *   - ranks are node-major (rank = node * gpus_per_node + local); hop 1 sends
 *     contiguous chunk j of every buffer to local rank j; hop 2 sends
 *     contiguous sub-chunk k of that chunk to node k.
 *
 * Every routine below is pinned by CPU tests that do not reuse this code:
 * worked examples derived by hand, exact rational checks of each rounding,
 * invariants, a NumPy re-derivation, and a brute-forced two-hop simulation.
 * None is left "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

/* ---- element encodings ------------------------------------------------- */

/* A bfloat16 is the upper half of a binary32: decoding is exact. */
static float bf16_decode(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even (NaN kept quiet). */
static uint16_t bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

static int32_t qmax_of(int32_t bits) { return bits == 8 ? 127 : 7; }

static void code_store(uint8_t *codes, int32_t bits, int64_t i, int32_t q)
{
    if (bits == 8) {
        codes[i] = (uint8_t)(int8_t)q;
        return;
    }
    uint8_t nib = (uint8_t)(q & 0xf);
    uint8_t *byte = &codes[i >> 1];
    if (i & 1)
        *byte = (uint8_t)((*byte & 0x0f) | (nib << 4));
    else
        *byte = (uint8_t)((*byte & 0xf0) | nib);
}

static int32_t code_load(const uint8_t *codes, int32_t bits, int64_t i)
{
    if (bits == 8)
        return (int32_t)(int8_t)codes[i];
    uint8_t byte = codes[i >> 1];
    int32_t nib = (i & 1) ? (byte >> 4) : (byte & 0xf);
    return nib >= 8 ? nib - 16 : nib;
}

static int valid_layout(int64_t numel, int32_t block, int32_t bits)
{
    if (numel < 0 || block < 1 || (bits != 4 && bits != 8))
        return 0;
    if (numel % block != 0)
        return 0;
    if (bits == 4 && (block & 1))
        return 0;
    return 1;
}

/* ---- quantize (QWZ block quantization; QGZ one-shot quantization) ------- */

/* Quantize one block of binary32 values. */
static void quantize_block(const float *x, int64_t n, int32_t bits, uint8_t *codes,
                           int64_t first, float *scale_out)
{
    const int32_t Q = qmax_of(bits);

    /* 1. the block's absolute maximum (max is exact in any order) */
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float m = fabsf(x[i]);
        if (m > a)
            a = m;
    }

    /* 2. the scale: one correctly rounded division by Q */
    float s = a / (float)Q;
    *scale_out = s;

    /* 3. each code: x / s rounded to nearest-even, clamped to [-Q, Q] */
    for (int64_t i = 0; i < n; ++i) {
        int32_t q = 0;
        if (s != 0.0f) {
            float t = x[i] / s;
            float r = rintf(t); /* default rounding mode: nearest, ties to even */
            if (r > (float)Q)
                r = (float)Q;
            if (r < (float)-Q)
                r = (float)-Q;
            q = (int32_t)r;
        }
        code_store(codes, bits, first + i, q);
    }
}

int oracle_quantize_f32(const float *x, int64_t numel, int32_t block, int32_t bits,
                        uint8_t *codes, float *scales)
{
    if (!valid_layout(numel, block, bits))
        return ORACLE_EINVAL;
    for (int64_t b = 0; b < numel / block; ++b)
        quantize_block(x + b * block, block, bits, codes, b * block, &scales[b]);
    return ORACLE_OK;
}

int oracle_quantize_bf16(const uint16_t *x, int64_t numel, int32_t block, int32_t bits,
                         uint8_t *codes, float *scales)
{
    if (!valid_layout(numel, block, bits))
        return ORACLE_EINVAL;
    float *buf = (float *)malloc(sizeof(float) * (size_t)(block > 0 ? block : 1));
    if (!buf)
        return ORACLE_EINVAL;
    for (int64_t b = 0; b < numel / block; ++b) {
        for (int32_t i = 0; i < block; ++i)
            buf[i] = bf16_decode(x[b * block + i]);
        quantize_block(buf, block, bits, codes, b * block, &scales[b]);
    }
    free(buf);
    return ORACLE_OK;
}

/* ---- dequantize (gather side of the QWZ all-gather) --------------------- */

int oracle_dequantize_f32(const uint8_t *codes, const float *scales, int32_t bits,
                          int64_t numel, int32_t block, float *y)
{
    if (!valid_layout(numel, block, bits))
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < numel; ++i)
        y[i] = (float)code_load(codes, bits, i) * scales[i / block];
    return ORACLE_OK;
}

int oracle_dequantize_bf16(const uint8_t *codes, const float *scales, int32_t bits,
                           int64_t numel, int32_t block, uint16_t *y)
{
    if (!valid_layout(numel, block, bits))
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < numel; ++i) {
        float v = (float)code_load(codes, bits, i) * scales[i / block];
        y[i] = bf16_round(v);
    }
    return ORACLE_OK;
}

/* ---- tensor-slice reordering (QGZ) -------------------------------------- */

/*
 * The buffer is N = n_nodes * gpus_per_node equal slices; slice r belongs to
 * rank r, which must end up holding it reduced [RS]. Hop 1 sends contiguous
 * chunk j (n_nodes slices) to local rank j; hop 2 sends sub-chunk k of that
 * chunk (one slice) to node k. So whatever sits at slice position p reaches
 * rank (p % n_nodes) * gpus_per_node + p / n_nodes, and the reorder puts
 * that rank's own slice there.
 */
int oracle_reorder_slices(const uint8_t *in, uint8_t *out, int64_t slice_bytes,
                          int32_t n_nodes, int32_t gpus_per_node)
{
    if (slice_bytes < 0 || n_nodes < 1 || gpus_per_node < 1)
        return ORACLE_EINVAL;
    int64_t n_slices = (int64_t)n_nodes * gpus_per_node;
    for (int64_t p = 0; p < n_slices; ++p) {
        int64_t local = p / n_nodes;      /* hop-1 destination (local rank) */
        int64_t node = p % n_nodes;       /* hop-2 destination (node)       */
        int64_t owner = node * gpus_per_node + local;
        memcpy(out + p * slice_bytes, in + owner * slice_bytes, (size_t)slice_bytes);
    }
    return ORACLE_OK;
}

/* ---- hop reduction (QGZ intra-node reduction; inter-node final sum) ----- */

/*
 * Input r's codes start at codes_in + r * codes_stride_bytes and its scales
 * at scales_in + r * scales_stride (in floats). sum[i] is the binary32 sum,
 * in ascending r, of each input's dequantized element i.
 */
int oracle_dequant_sum(const uint8_t *codes_in, int64_t codes_stride_bytes,
                       const float *scales_in, int64_t scales_stride, int32_t n_inputs,
                       int32_t bits, int64_t numel, int32_t block, float *sum)
{
    if (!valid_layout(numel, block, bits) || n_inputs < 1)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < numel; ++i) {
        float acc = 0.0f;
        for (int32_t r = 0; r < n_inputs; ++r) {
            const uint8_t *c = codes_in + (int64_t)r * codes_stride_bytes;
            const float *s = scales_in + (int64_t)r * scales_stride;
            float v = (float)code_load(c, bits, i) * s[i / block];
            acc = acc + v;
        }
        sum[i] = acc;
    }
    return ORACLE_OK;
}

/*
 * The fused hop step as the oracle sees it: the sum above, then the sum
 * re-quantized block by block (same block size) for the next hop.
 */
int oracle_dequant_reduce_requant(const uint8_t *codes_in, int64_t codes_stride_bytes,
                                  const float *scales_in, int64_t scales_stride,
                                  int32_t n_inputs, int32_t bits_in, int64_t numel,
                                  int32_t block, uint8_t *codes_out, float *scales_out,
                                  int32_t bits_out, float *sum_out)
{
    if (!valid_layout(numel, block, bits_in))
        return ORACLE_EINVAL;
    if (bits_out != 0 && !valid_layout(numel, block, bits_out))
        return ORACLE_EINVAL;
    float *sum = sum_out;
    if (!sum) {
        sum = (float *)malloc(sizeof(float) * (size_t)(numel > 0 ? numel : 1));
        if (!sum)
            return ORACLE_EINVAL;
    }
    int rc = oracle_dequant_sum(codes_in, codes_stride_bytes, scales_in, scales_stride,
                                n_inputs, bits_in, numel, block, sum);
    if (rc == ORACLE_OK && bits_out != 0)
        rc = oracle_quantize_f32(sum, numel, block, bits_out, codes_out, scales_out);
    if (!sum_out)
        free(sum);
    return rc;
}

/*
 * [AVG] The reduce-scatter of ZeRO stage 2 hands GPU i the AVERAGED gradient
 * of shard i. Reading: the average is the binary32 sum above divided by the
 * number of GPUs that contributed (`divisor`, the data-parallel degree, not
 * the number of inputs of this hop), one correctly rounded binary32 division
 * per element.
 */
int oracle_dequant_average(const uint8_t *codes_in, int64_t codes_stride_bytes,
                           const float *scales_in, int64_t scales_stride, int32_t n_inputs,
                           int32_t bits, int64_t numel, int32_t block, int32_t divisor,
                           float *avg)
{
    if (divisor < 1 || divisor > (1 << 24))
        return ORACLE_EINVAL;
    int rc = oracle_dequant_sum(codes_in, codes_stride_bytes, scales_in, scales_stride,
                                n_inputs, bits, numel, block, avg);
    if (rc != ORACLE_OK)
        return rc;
    const float d = (float)divisor; /* exact: divisor <= 2^24 */
    for (int64_t i = 0; i < numel; ++i)
        avg[i] = avg[i] / d;
    return ORACLE_OK;
}

/* ---- element conversions exposed for tests ------------------------------ */

void oracle_bf16_round_array(const float *x, int64_t n, uint16_t *y)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = bf16_round(x[i]);
}

void oracle_bf16_decode_array(const uint16_t *x, int64_t n, float *y)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = bf16_decode(x[i]);
}

int oracle_abi_version(void) { return 1; }
