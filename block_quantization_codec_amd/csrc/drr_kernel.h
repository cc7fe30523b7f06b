// drr_kernel.h - the hop kernel (dequantize -> binary32 reduce -> requantize
// or average) and its launch templates; included by the drr_in*_out*.hip units.
//
// Page "Quantized LLM Training at Scale with ZeRO++", section "The Three
// Pillars of ZeRO++", pillar 3 (QGZ): the two-hop protocol first exchanges
// within the node and reduces what arrived, then exchanges across nodes; the
// page credits kernel fusion among its optimizations. Hop 1 here is
// dequantize + sum + requantize for the next hop; hop 2 is dequantize + sum
// into the owner's binary32 shard (page "ZeRO Stage 2: Gradient
// Partitioning": GPU i keeps shard i, whose optimizer step works in fp32).
//
// Arithmetic contract: for each element, acc = +0; for r = 0..R-1 in order,
// acc = fl(acc + fl(code_r * s_r)), every product and every sum rounded on
// its own, never fused. The averaged variant then divides acc by the number
// of contributing GPUs (one correctly rounded binary32 division): page
// "ZeRO Stage 2: Gradient Partitioning", step 2 of the stage-2 flow, where
// the reduce-scatter hands each GPU the average of its shard. Any code bytes
// and scales are accepted: products use a fused multiply-add shortcut only
// where it is exact (see dequant_dword), and the first sum, written acc = p,
// is made exact by adding +0 to every finished sum (see add_batch).
//
// Layout of the work: a lane owns E consecutive elements of a wave segment of
// 64 E elements: E = 32 (one 16-byte vector of 4-bit codes per input, so
// each load instruction reads one contiguous kilobyte of an input), or E = 8
// for small outputs, which then still spread over every SIMD. Inputs are
// read a batch at a time, all loads of a batch in flight before the batch is
// summed in input order. With E = 32 every batch holds 8 inputs (a last,
// partial one skips its padding), and 4-bit code vectors land in the wave's
// own LDS slots rather than in registers (see consume_lds); with E = 8 the
// next batch's loads are also issued before the current batch is summed.
// Blocks of 4096 elements always take E = 32. The requantized block maximum
// is reduced across the block's lanes with DPP / permlane swaps.
#pragma once

#include "zpp_device.h"
#include "zpp_launch.h"

namespace zpp {

// Arguments of one hop-kernel launch (already validated).
struct DrrArgs {
    const void *codes_in;
    int64_t cstride;
    const float *scales_in;
    int64_t sstride;
    int n_inputs;
    int64_t numel;
    void *codes_out;
    float *scales_out;
    float *sum_out;
    float divisor;
    hipStream_t stream;
    // Keep window: requantized codes and scales of elements [keep_begin,
    // keep_begin + keep_len) go to codes_keep / scales_keep, all others to
    // codes_out / scales_out in order with the window left out (keep_len 0:
    // no window).
    int64_t keep_begin = 0;
    int64_t keep_len = 0;
    void *codes_keep = nullptr;
    float *scales_keep = nullptr;
};

// One launcher per pair of code widths, each in a translation unit of its own
// (the kernels are large; separate units compile in parallel). bits_out 0
// covers the binary32 sum and, when a.divisor > 0, the average.
hipError_t drr_dispatch_in4_out0(int log2b, const DrrArgs &a);
hipError_t drr_dispatch_in4_out4(int log2b, const DrrArgs &a);
hipError_t drr_dispatch_in4_out8(int log2b, const DrrArgs &a);
hipError_t drr_dispatch_in8_out0(int log2b, const DrrArgs &a);
hipError_t drr_dispatch_in8_out4(int log2b, const DrrArgs &a);
hipError_t drr_dispatch_in8_out8(int log2b, const DrrArgs &a);

namespace {

// Inputs per load batch of the wide layout (a 16-byte code vector and one
// scale per input and lane).
#ifndef ZPP_DRR_BATCH
#define ZPP_DRR_BATCH 8
#endif
// Inputs per load batch of the narrow layout (one code dword and one scale
// per input and lane; with the next batch in flight as well, 4 * 8 = 32
// loads, within the 63 a wave can keep outstanding).
#ifndef ZPP_DRR_NARROW_BATCH
#define ZPP_DRR_NARROW_BATCH 8
#endif
// 1: the narrow layout loads each batch while it sums the previous one.
#ifndef ZPP_DRR_NARROW_OVERLAP
#define ZPP_DRR_NARROW_OVERLAP 1
#endif
// Elements per lane of the wide layout (16 or 32).
#ifndef ZPP_DRR_WIDE_E
#define ZPP_DRR_WIDE_E 32
#endif
// 1: with 4-bit inputs the wide layout moves each input's codes into LDS
// with loads that hold no registers (see consume_lds).
#ifndef ZPP_DRR_LDS
#define ZPP_DRR_LDS 1
#endif
// With 4-bit inputs and at most this many of them, the wide (LDS-staged)
// layout is taken from ZPP_DRR_FEW_INPUTS_WAVES waves on, below the general
// threshold: with few inputs the narrow layout's per-lane overhead (factors,
// requantization per 8 elements) outweighs its extra waves once there are
// about two wide waves per SIMD (measured on 2 or 4 inputs: at 1,953 waves
// the wide layout 6-20% faster, at 976 waves 13% slower; with 8 inputs, or
// 8-bit codes, no gain).
#ifndef ZPP_DRR_FEW_INPUTS
#define ZPP_DRR_FEW_INPUTS 4
#endif
#ifndef ZPP_DRR_FEW_INPUTS_WAVES
#define ZPP_DRR_FEW_INPUTS_WAVES 1536
#endif
// 1: hop kernels of the wide layout that write only sums pass them through
// LDS so that every store is contiguous across the wave (see finish_tile):
// twice as fast on 16.8 M-element sums of 32 4-bit inputs, and on 8 8-bit
// ones. The narrow layout stores its own 8 sums per lane: through LDS its
// small launches (32 x 1.95 M elements) ran 2-4% slower.
#ifndef ZPP_DRR_SUM_XPOSE
#define ZPP_DRR_SUM_XPOSE 1
#endif
// Below this many waves of the wide layout, lanes take 8 elements each so
// that small outputs still spread over every SIMD.
#ifndef ZPP_DRR_NARROW_WAVES
#define ZPP_DRR_NARROW_WAVES 4096
#endif

template <int BITS_IN_, int BITS_OUT, int LOG2B_, int E_>
struct DrrGeom {
    static constexpr int BITS_IN = BITS_IN_;
    static constexpr int LOG2B = LOG2B_;
    static constexpr int E = E_;                           // elements per lane per segment
    static constexpr int SEG = kWave * E;                  // elements per wave segment
    static constexpr int B = 1 << LOG2B;
    static constexpr int SPB = B > SEG ? B / SEG : 1;      // segments per block (= per tile)
    static constexpr int L = B >= SEG ? kWave : B / E;     // lanes per block within a segment
    static constexpr int U = SPB;
    static constexpr int TILE = U * SEG;
    static constexpr int ND = E * BITS_IN / 32;            // code dwords per lane per input
    static constexpr int QMAX = BITS_OUT == 8 ? 127 : 7;
    static constexpr int RB = E == 8 ? ZPP_DRR_NARROW_BATCH : ZPP_DRR_BATCH;  // inputs per load batch
    static constexpr bool OVERLAP = E == 8 && ZPP_DRR_NARROW_OVERLAP;           // see consume_overlapped
};

template <int ND>
__device__ __forceinline__ void load_dwords(const uint8_t *p, uint32_t (&d)[ND]) {
    if constexpr (ND == 1) {
        d[0] = ld_stream<uint32_t>(p);
    } else if constexpr (ND == 2) {
        const u32x2 v = ld_stream<u32x2>(p);
        d[0] = v[0];
        d[1] = v[1];
    } else {
#pragma unroll
        for (int j = 0; j < ND / 4; ++j) {
            const u32x4 v = ld_stream<u32x4>(p + 16 * j);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[4 * j + i] = v[i];
        }
    }
}

template <int ND>
__device__ __forceinline__ void store_dwords(uint8_t *p, const uint32_t (&d)[ND]) {
    if constexpr (ND == 1) {
        st_out<uint32_t>(p, d[0]);
    } else if constexpr (ND == 2) {
        st_out<u32x2>(p, u32x2{d[0], d[1]});
    } else {
#pragma unroll
        for (int j = 0; j < ND / 4; ++j) st_out<u32x4>(p + 16 * j, u32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]});
    }
}

// Per-input factors of the product formulas (see dequant_dword).
struct Factors {
    float s;    // the scale
    float mb;   // -2^(bits-1) s
    float s24;  // s * 2^24 (4-bit codes)
    float s20;  // s * 2^20 (4-bit codes)
};

template <int BITS_IN>
__device__ __forceinline__ Factors factors_of(float s) {
    return Factors{s, s * (BITS_IN == 8 ? -128.0f : -8.0f), s * 0x1p24f, s * 0x1p20f};
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// The codes of dword `w` of one input as binary32 products code * s, element
// 0 first. FAST: flipping the top bit of a two's-complement code q gives the
// unsigned q + 2^(bits-1) (q + 8 for a nibble, q + 128 for a byte), and a
// fused multiply-add with mb = -2^(bits-1) s forms (q + 2^(bits-1)) s +
// mb = q s exactly and rounds it once, which is the correctly rounded
// product. 8-bit codes: each byte converts to binary32 in one instruction
// (v_cvt_f32_ubyte0..3); exact whenever mb is finite, |s| <= 2^120. 4-bit
// codes: a 16-bit half holding n < 1024 is the binary16 subnormal n 2^-24,
// which v_fma_mix_f32 widens exactly inside the fused multiply-add; nibbles
// masked into the halves, in place (n = q + 8, factor s 2^24) or four bits
// up (n = 16 (q + 8), factor s 2^20), need no conversion instruction at all.
// Exact whenever s 2^24 is finite: |s| <= 2^103. An exact zero comes out as
// +0 where the product may be -0, which no sum can tell apart: every sum
// starts from +0. (Also measured, and slower on gfx950: FP8 E4M3 decoding
// of byte values below 16, and the sign-extending SDWA conversion followed
// by a multiply.)
template <int BITS_IN, bool FAST>
__device__ __forceinline__ void dequant_dword(uint32_t w, const Factors &f, float (&p)[32 / BITS_IN]) {
    if constexpr (BITS_IN == 8 && FAST) {
        uint32_t u = w ^ 0x80808080u;  // byte i: q_i + 128
        asm("" : "+v"(u));             // opaque: each byte converts straight from the dword
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_fmaf(static_cast<float>((u >> (8 * i)) & 0xFFu), f.s, f.mb);
    } else if constexpr (BITS_IN == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = static_cast<float>(static_cast<int8_t>(w >> (8 * i))) * f.s;
    } else if constexpr (FAST) {
        // Nibble j of w is element j. Halves: d0 = elements 0 | 4, d1 = 1 | 5
        // (four bits up), d2 = 2 | 6, d3 = 3 | 7 (four bits up).
        const uint32_t w8 = w >> 8;
        const h2 d0 = __builtin_bit_cast(h2, (w ^ 0x88888888u) & 0x000F000Fu);
        const h2 d1 = __builtin_bit_cast(h2, (w ^ 0x88888888u) & 0x00F000F0u);
        const h2 d2 = __builtin_bit_cast(h2, (w8 ^ 0x00880088u) & 0x000F000Fu);
        const h2 d3 = __builtin_bit_cast(h2, (w8 ^ 0x00880088u) & 0x00F000F0u);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            p[4 * h + 0] = __builtin_fmaf(static_cast<float>(d0[h]), f.s24, f.mb);
            p[4 * h + 1] = __builtin_fmaf(static_cast<float>(d1[h]), f.s20, f.mb);
            p[4 * h + 2] = __builtin_fmaf(static_cast<float>(d2[h]), f.s24, f.mb);
            p[4 * h + 3] = __builtin_fmaf(static_cast<float>(d3[h]), f.s20, f.mb);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = static_cast<float>(code_at<4>(w, i)) * f.s;
    }
}

// Sum one batch of loaded inputs into acc, in input order.
// Positions from `valid` on (at least 1) are skipped: a wave-uniform branch.
template <typename G, int NB, bool FIRST, bool FAST>
__device__ __forceinline__ void accumulate(const uint32_t (&w)[NB][G::U][G::ND], const float (&s)[NB][G::U],
                                           float (&acc)[G::U][G::E], int valid) {
    constexpr int CPW = 32 / G::BITS_IN;  // codes per dword
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        if (k > 0 && k >= valid) break;
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const Factors f = factors_of<G::BITS_IN>(s[k][u]);
#pragma unroll
            for (int d = 0; d < G::ND; ++d) {
                float p[CPW];
                dequant_dword<G::BITS_IN, FAST>(w[k][u][d], f, p);
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    if (FIRST && k == 0)
                        acc[u][d * CPW + i] = p[i];
                    else
                        acc[u][d * CPW + i] = acc[u][d * CPW + i] + p[i];
                }
            }
        }
    }
}

// The codes and scales of NB consecutive inputs, as one lane loads them.
template <typename G, int NB>
struct Batch {
    uint32_t w[NB][G::U][G::ND];
    float s[NB][G::U];
};

// A lane's byte offsets within one input: of its code vectors and of their
// block scales, the same for every input. An address is then a wave-uniform
// base (input r's) plus a 32-bit lane offset: the LDS-staged layout hands the
// two to its loads as a buffer resource and an offset, the register layouts
// add them. A launch covers at most 2^29 elements, so every offset fits in
// 32 bits.
template <typename G>
struct LaneOffsets {
    uint32_t code[G::U];
    uint32_t scale[G::U];
};

// Inputs r0 .. r0+NB-1. PAD: positions past the last of the n_inputs inputs
// reload it (valid addresses, unused values), so that a last, partial batch
// issues the same loads as a full one.
template <typename G, int NB, bool PAD>
__device__ __forceinline__ void load_batch(const uint8_t *__restrict__ codes_in, int64_t codes_stride,
                                           const float *__restrict__ scales_in, int64_t scales_stride, int r0,
                                           int n_inputs, const LaneOffsets<G> &o, Batch<G, NB> &b) {
    // Scales first: the batch's choice of product formula needs all of them,
    // while each input's codes are needed only when that input is summed.
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const int ri = PAD ? min(r0 + k, n_inputs - 1) : r0 + k;
        const uint8_t *sc = reinterpret_cast<const uint8_t *>(scales_in + static_cast<int64_t>(ri) * scales_stride);
#pragma unroll
        for (int u = 0; u < G::U; ++u) b.s[k][u] = *reinterpret_cast<const float *>(sc + o.scale[u]);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const int ri = PAD ? min(r0 + k, n_inputs - 1) : r0 + k;
        const uint8_t *c = codes_in + static_cast<int64_t>(ri) * codes_stride;
#pragma unroll
        for (int u = 0; u < G::U; ++u) load_dwords<G::ND>(c + o.code[u], b.w[k][u]);
    }
    // Every load of the batch is issued before anything that uses one.
    __builtin_amdgcn_sched_barrier(0);
}

// The largest |s| of a batch of scales: float maxima with absolute-value
// operand modifiers, three values per instruction. An infinite scale makes it
// infinite; a NaN scale may be dropped, which is harmless: every product with
// it is NaN under either formula.
template <typename G, int NB>
__device__ __forceinline__ float batch_abs_max(const float (&s)[NB][G::U]) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
        for (int u = 0; u < G::U; ++u) m = __builtin_fmaxf(m, __builtin_fabsf(s[k][u]));
    return m;
}

// Whether the fused product shortcut of dequant_dword is exact for every
// scale of magnitude at most m (a NaN m takes the plain product).
template <int BITS_IN>
__device__ __forceinline__ bool shortcut_exact(float m) {
    return m <= (BITS_IN == 8 ? 0x1p120f : 0x1p103f);
}

// Add a loaded batch into acc, in input order. FIRST: the batch's first input
// starts the sums, written acc = p instead of acc = +0 + p. The two differ
// only when p is -0 (a negative code times a zero scale, or a zero code times
// a negative one), and then only as long as every later product is -0 as
// well: -0 + x == +0 + x for every other x. The kernel adds +0 to each
// finished sum before writing it (a sum that starts at +0 is never -0), and a
// requantized sum gets the same codes and scale either way.
template <typename G, int NB, bool FIRST>
__device__ __forceinline__ void add_batch(const Batch<G, NB> &b, float (&acc)[G::U][G::E], int valid = NB) {
    const bool fast = shortcut_exact<G::BITS_IN>(batch_abs_max<G, NB>(b.s));
    if (fast)
        accumulate<G, NB, FIRST, true>(b.w, b.s, acc, valid);
    else
        accumulate<G, NB, FIRST, false>(b.w, b.s, acc, valid);
}

// Sum all n_inputs inputs in batches of NB, one batch loaded and then summed
// at a time; the first batch starts the sums. A last, partial batch loads
// like a full one and skips the positions past the last input. With no
// choice of batch size there is one path through the sums, and the compiler
// keeps them in the same registers throughout.
template <typename G, int NB>
__device__ __forceinline__ void consume_padded(const uint8_t *__restrict__ codes_in, int64_t codes_stride,
                                               const float *__restrict__ scales_in, int64_t scales_stride,
                                               int n_inputs, const LaneOffsets<G> &o, float (&acc)[G::U][G::E]) {
    {
        Batch<G, NB> b;
        load_batch<G, NB, true>(codes_in, codes_stride, scales_in, scales_stride, 0, n_inputs, o, b);
        add_batch<G, NB, true>(b, acc, n_inputs);
    }
    for (int r = NB; r < n_inputs; r += NB) {
        Batch<G, NB> b;
        load_batch<G, NB, true>(codes_in, codes_stride, scales_in, scales_stride, r, n_inputs, o, b);
        add_batch<G, NB, false>(b, acc, n_inputs - r);
    }
}

// Sum every remaining full batch of NB inputs from input r on (r advances)
// into sums that already hold +0.
template <typename G, int NB>
__device__ __forceinline__ void consume(const uint8_t *__restrict__ codes_in, int64_t codes_stride,
                                        const float *__restrict__ scales_in, int64_t scales_stride, int n_inputs,
                                        const LaneOffsets<G> &o, int &r, float (&acc)[G::U][G::E]) {
    for (; r + NB <= n_inputs; r += NB) {
        Batch<G, NB> b;
        load_batch<G, NB, false>(codes_in, codes_stride, scales_in, scales_stride, r, n_inputs, o, b);
        add_batch<G, NB, false>(b, acc);
    }
}

// As consume, with each batch's loads issued before the previous batch is
// summed, so that a wave's loads overlap its own arithmetic (two batches of
// registers, used in turn). Every sum of a batch follows the loads of the
// next batch without a branch in between, so the sum waits for its own
// batch's loads only.
template <typename G, int NB>
__device__ __forceinline__ void consume_overlapped(const uint8_t *__restrict__ codes_in, int64_t codes_stride,
                                                   const float *__restrict__ scales_in, int64_t scales_stride,
                                                   int n_inputs, const LaneOffsets<G> &o, int &r,
                                                   float (&acc)[G::U][G::E]) {
    if (r + NB > n_inputs) return;
    Batch<G, NB> a, b;
    load_batch<G, NB, false>(codes_in, codes_stride, scales_in, scales_stride, r, n_inputs, o, a);
    for (;;) {
        if (r + 2 * NB > n_inputs) {
            add_batch<G, NB, false>(a, acc);
            r += NB;
            return;
        }
        load_batch<G, NB, false>(codes_in, codes_stride, scales_in, scales_stride, r + NB, n_inputs, o, b);
        add_batch<G, NB, false>(a, acc);
        r += NB;
        if (r + 2 * NB > n_inputs) {
            add_batch<G, NB, false>(b, acc);
            r += NB;
            return;
        }
        load_batch<G, NB, false>(codes_in, codes_stride, scales_in, scales_stride, r + NB, n_inputs, o, a);
        add_batch<G, NB, false>(b, acc);
        r += NB;
    }
}

// ---- the wide layout with codes staged through LDS -------------------------
//
// With 4-bit inputs a lane's codes of one input are one 16-byte vector. The
// batch's scales are loaded into registers as elsewhere; each code vector
// then goes straight from memory into this wave's own LDS slot (a buffer
// load into LDS: a kilobyte per instruction, no registers held while it is
// in flight), and is read back just before it is summed. The registers
// saved let 5 waves share a SIMD instead of 4 (the kernel is held to that
// register budget), which keeps more loads in flight while other waves sum
// and requantize. Both kinds of load address an input through a buffer
// resource, so the per-input address work is scalar.

// Word 3 of a raw buffer resource (no swizzle, no index stride) on this GPU
// family: the data-format field set to 32 bits, which untyped loads need to
// be served at all.
constexpr int kRawBufferConfig = 0x00020000;

// A buffer resource over one input's bytes of this launch: a wave-uniform
// base and size in scalar registers. Loads through it take a 32-bit lane
// offset, so no lane computes a 64-bit address per input, and a load past
// `bytes` returns zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t input_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), static_cast<int>(bytes),
                                             kRawBufferConfig);
}

// One binary32 at byte offset `off` of a buffer.
__device__ __forceinline__ float buffer_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return as_f(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// 16 bytes per lane at byte offset `off` of a buffer, straight into LDS at
// `dst` (lane i's bytes at dst + 16 i).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t off, void *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding. The compiler does not track loads into LDS, so their readers
// wait here explicitly; the clobber keeps memory accesses on their side.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Sum inputs K .. NB-1 of a batch whose code vectors sit in LDS slots 0 ..
// NB-1, in input order. The loads into the slots were issued in slot order
// after every other outstanding load had completed, and vector-memory
// operations complete in order, so slot K has arrived once at most NB-1-K
// operations are outstanding. Positions from `valid` on are padding.
template <typename G, int NB, int K = 0>
__device__ __forceinline__ void sum_from_lds(const uint32_t (*slot)[kWave][4], const float (&s)[NB][G::U], int lane,
                                             float (&acc)[G::U][G::E], bool first, int valid, bool fast) {
    if constexpr (K < NB) {
        if (K == 0 || K < valid) {
            wait_vmem<NB - 1 - K>();
            uint32_t w[1][G::U][G::ND];
            float sk[1][G::U];
#pragma unroll
            for (int u = 0; u < G::U; ++u) {
                const uint32_t *q = slot[K * G::U + u][lane];
#pragma unroll
                for (int d = 0; d < G::ND; ++d) w[0][u][d] = q[d];
                sk[0][u] = s[K][u];
            }
            if (K == 0 && first) {
                if (fast)
                    accumulate<G, 1, true, true>(w, sk, acc, 1);
                else
                    accumulate<G, 1, true, false>(w, sk, acc, 1);
            } else {
                if (fast)
                    accumulate<G, 1, false, true>(w, sk, acc, 1);
                else
                    accumulate<G, 1, false, false>(w, sk, acc, 1);
            }
        }
        sum_from_lds<G, NB, K + 1>(slot, s, lane, acc, first, valid, fast);
    }
}

// All n_inputs inputs in batches of NB through the wave's NB LDS slots; the
// first batch starts the sums, and a last, partial batch loads its padding
// from the last input and skips it (as consume_padded does).
template <typename G, int NB>
__device__ __forceinline__ void consume_lds(const uint8_t *__restrict__ codes_in, int64_t codes_stride,
                                            const float *__restrict__ scales_in, int64_t scales_stride,
                                            int n_inputs, int numel, const LaneOffsets<G> &o,
                                            float (&acc)[G::U][G::E], uint32_t (*slot)[kWave][4], int lane) {
    static_assert(G::U == 1 && G::ND == 4, "one 16-byte code vector per input and lane");
    // bytes of one input within this launch (numel < 2^30)
    const uint32_t code_bytes = static_cast<uint32_t>(numel) / 2u;
    const uint32_t scale_bytes = (static_cast<uint32_t>(numel) >> G::LOG2B) * 4u;
    for (int r0 = 0; r0 < n_inputs; r0 += NB) {
        // the previous batch's reads of the slots are complete before they are refilled
        if (r0 > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float s[NB][G::U];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int ri = min(r0 + k, n_inputs - 1);
            const __amdgpu_buffer_rsrc_t rs = input_rsrc(scales_in + static_cast<int64_t>(ri) * scales_stride, scale_bytes);
#pragma unroll
            for (int u = 0; u < G::U; ++u) s[k][u] = buffer_f32(rs, o.scale[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int ri = min(r0 + k, n_inputs - 1);
            const __amdgpu_buffer_rsrc_t rc = input_rsrc(codes_in + static_cast<int64_t>(ri) * codes_stride, code_bytes);
#pragma unroll
            for (int u = 0; u < G::U; ++u)
                buffer_to_lds16(rc, o.code[u], &slot[k * G::U + u][0][0]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // The batch's choice of product formula (see add_batch), once the
        // scales are in: the code vectors are already on their way, so a
        // batch costs one memory round trip, not two (7% faster on hops of 4
        // inputs of 4M and 16.8M elements; hop 1's 8 inputs unchanged).
        // Vector-memory operations complete in order, so the scales are in
        // before slot 0, and the waits on the slots below still hold.
        const bool fast = shortcut_exact<4>(batch_abs_max<G, NB>(s));
        sum_from_lds<G, NB>(slot, s, lane, acc, r0 == 0, n_inputs - r0, fast);
    }
    wait_vmem<0>();  // padding loads too: none may land in LDS after this wave moves on
}

// Elements one launch covers at most; a multiple of every block size and
// tile, small enough that every lane offset fits in 32 bits.
constexpr int64_t kDrrChunk = INT64_C(1) << 29;

// Minimum waves per SIMD a hop kernel is compiled for: 5 for the LDS-staged
// wide layout, whose registers fit that budget (and whose 32 KB of LDS per
// workgroup allow 5 workgroups per CU); no minimum for the other layouts.
template <int BITS_IN, int LOG2B, int E>
constexpr int drr_min_waves() {
    return ZPP_DRR_LDS && DrrGeom<BITS_IN, 0, LOG2B, E>::U == 1 && DrrGeom<BITS_IN, 0, LOG2B, E>::ND == 4 &&
                   !DrrGeom<BITS_IN, 0, LOG2B, E>::OVERLAP
               ? 5
               : 1;
}

// Where one launch writes. Sums (or averages) go to sum_out. Requantized
// codes and scales of the elements in the keep window [kb, kb + klen) go to
// codes_keep / scales_keep (element kb first); all others go to codes_out /
// scales_out in element order with the window left out. klen == 0: no
// window. kb and klen are whole blocks.
struct DrrOut {
    uint8_t *codes_out;
    float *scales_out;
    float *sum_out;
    float divisor;
    uint32_t kb, klen;
    uint8_t *codes_keep;
    float *scales_keep;
};

// The end of a tile: the sums (plus +0, see add_batch), or their averages,
// stored; then the sums requantized per block and stored.
//
// With xp (this wave's LDS area of 64 E dwords) the sums go out through it:
// each lane writes its E sums there and reads back 4 consecutive sums from
// every 256, so that each 16-byte store covers one contiguous kilobyte
// across the wave. A lane storing its own E > 4 sums would leave every
// store instruction writing parts of many cache lines, which measured at
// about half the write rate. Without xp (the narrow layout, and launches
// that requantize too) each lane stores its own sums.
template <typename G, int BITS_OUT, bool AVG>
__device__ __forceinline__ void finish_tile(float (&acc)[G::U][G::E], const bool (&ok)[G::U],
                                            const uint32_t (&e)[G::U], uint32_t tb, uint32_t n, int lane,
                                            const DrrOut &out, uint32_t *xp) {
    static_assert(!AVG || BITS_OUT == 0, "the average is a final binary32 output");
    constexpr int U = G::U, E = G::E;
    if (AVG || out.sum_out != nullptr) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < E; ++i) {
                float v = acc[u][i] + 0.0f;          // -0 -> +0 (see add_batch), any other value unchanged
                if constexpr (AVG) v = v / out.divisor;  // IEEE division
                acc[u][i] = v;
            }
    }
    if (out.sum_out != nullptr) {
        if (xp != nullptr) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int v = 0; v < E / 4; ++v)
                    *reinterpret_cast<u32x4 *>(xp + lane * E + 4 * v) =
                        u32x4{as_u(acc[u][4 * v]), as_u(acc[u][4 * v + 1]), as_u(acc[u][4 * v + 2]),
                              as_u(acc[u][4 * v + 3])};
                const uint32_t sb = tb + static_cast<uint32_t>(u * G::SEG);
#pragma unroll
                for (int v = 0; v < E / 4; ++v) {
                    const uint32_t i = static_cast<uint32_t>(v * 4 * kWave + 4 * lane);
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(xp + i);
                    if (sb + i < n) st_out<u32x4>(reinterpret_cast<uint8_t *>(out.sum_out) + (sb + i) * 4u, w);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!ok[u]) continue;
                float *dst = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(out.sum_out) + e[u] * 4u);
#pragma unroll
                for (int v = 0; v < E / 4; ++v)
                    st_out<u32x4>(dst + 4 * v, u32x4{as_u(acc[u][4 * v]), as_u(acc[u][4 * v + 1]),
                                                 as_u(acc[u][4 * v + 2]), as_u(acc[u][4 * v + 3])});
            }
        }
    }
    if constexpr (BITS_OUT != 0) {
        // |acc| maximum as a float maximum with abs operand modifiers (three
        // values per instruction); for non-negative finite values it
        // equals the integer maximum of the bit patterns.
        float fm = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < E; ++i) fm = __builtin_fmaxf(fm, __builtin_fabsf(acc[u][i]));
        uint32_t mx = ok[0] ? as_u(fm) : 0u;
        mx = group_max_u32<G::L>(mx);
        const float sc = block_scale<G::QMAX>(as_f(mx));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float mg[E];
            round_codes<E, BITS_OUT>(acc[u], sc, mg);
            uint32_t cw[E * BITS_OUT / 32];
            pack_codes<E, BITS_OUT>(mg, cw);
            if (!ok[u]) continue;
            // Output position: inside the keep window, or in the rest with the
            // window left out. The window is whole blocks, so a tile lies
            // before it, after it or inside it, decided once for the wave,
            // except for at most two tiles per launch that hold one of its
            // ends, whose lanes decide each for itself.
            const uint32_t k1 = out.kb + out.klen;
            const uint32_t te = tb + G::TILE;
            const bool inside = out.klen != 0 && tb >= out.kb && te <= k1;
            const bool after = out.klen != 0 && tb >= k1;
            if (out.klen == 0 || te <= out.kb || after || inside) {
                const uint32_t idx = e[u] - (inside ? out.kb : (after ? out.klen : 0u));
                uint8_t *cdst = inside ? out.codes_keep : out.codes_out;
                float *sdst = inside ? out.scales_keep : out.scales_out;
                store_dwords<E * BITS_OUT / 32>(cdst + idx * BITS_OUT / 8, cw);
                if (u == 0 && (lane & (G::L - 1)) == 0) sdst[idx >> G::LOG2B] = sc;
            } else {
                const uint32_t rel = e[u] - out.kb;
                const bool keep = rel < out.klen;
                const uint32_t idx = keep ? rel : (e[u] < out.kb ? e[u] : e[u] - out.klen);
                uint8_t *cdst = keep ? out.codes_keep : out.codes_out;
                float *sdst = keep ? out.scales_keep : out.scales_out;
                store_dwords<E * BITS_OUT / 32>(cdst + idx * BITS_OUT / 8, cw);
                if (u == 0 && (lane & (G::L - 1)) == 0) sdst[idx >> G::LOG2B] = sc;
            }
        }
    }
}

template <int BITS_IN, int BITS_OUT, int LOG2B, int E, bool AVG>
__global__ __launch_bounds__(kBlockThreads)
__attribute__((amdgpu_waves_per_eu(drr_min_waves<BITS_IN, LOG2B, E>(), 8))) void drr_kernel(const uint8_t *__restrict__ codes_in,
                                                            int64_t codes_stride,
                                                            const float *__restrict__ scales_in,
                                                            int64_t scales_stride, int n_inputs, int numel,
                                                            DrrOut out) {
    using G = DrrGeom<BITS_IN, BITS_OUT, LOG2B, E>;
    constexpr int U = G::U;

    const int lane = threadIdx.x & (kWave - 1);
    const int wib = wave_in_block();
    const int wave = static_cast<int>(xcd_block(blockIdx.x, gridDim.x)) * (kBlockThreads / kWave) + wib;
    const int n_waves = static_cast<int>(gridDim.x) * (kBlockThreads / kWave);

    // A launch covers at most 2^29 elements: tile offsets, and the grid
    // stride added to them, fit in 32 bits.
    const uint32_t n = static_cast<uint32_t>(numel);
    for (uint32_t t0 = static_cast<uint32_t>(wave) * G::TILE; t0 < n; t0 += static_cast<uint32_t>(n_waves) * G::TILE) {
        uint32_t e[U];
        bool ok[U];
        LaneOffsets<G> o;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e0 = t0 + static_cast<uint32_t>(u * G::SEG + lane * E);
            ok[u] = e0 < n;
            e[u] = ok[u] ? e0 : 0u;
            o.code[u] = e[u] * BITS_IN / 8;
            o.scale[u] = (e[u] >> LOG2B) * 4u;
        }

        float acc[U][E];
        uint32_t *xp = nullptr;  // LDS area for the sums (see finish_tile)
        // Inputs are consumed in batches whose loads are all issued before
        // the batch is summed. The wide layout sums batches of RB (a last,
        // partial one skips its padding), and its first batch starts the
        // sums. The narrow layout,
        // whose waves are few, starts its sums from +0 and overlaps each
        // batch's loads with the previous batch's sums, then takes what is
        // left four inputs at a time and the last 1 to 3 as one batch.
        if constexpr (G::OVERLAP) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < E; ++i) acc[u][i] = 0.0f;
            int r = 0;
            consume_overlapped<G, G::RB>(codes_in, codes_stride, scales_in, scales_stride, n_inputs, o, r, acc);
            if constexpr (G::RB > 4) consume<G, 4>(codes_in, codes_stride, scales_in, scales_stride, n_inputs, o, r, acc);
            // the last 1 to 3 inputs in one batch (one memory round trip):
            // 4-12% faster than one at a time on hops of 2, 3 or 7 inputs
            consume<G, 3>(codes_in, codes_stride, scales_in, scales_stride, n_inputs, o, r, acc);
            consume<G, 2>(codes_in, codes_stride, scales_in, scales_stride, n_inputs, o, r, acc);
            consume<G, 1>(codes_in, codes_stride, scales_in, scales_stride, n_inputs, o, r, acc);
        } else if constexpr (ZPP_DRR_LDS && G::U == 1 && G::ND == 4) {
            __shared__ __attribute__((aligned(16))) uint32_t lds_codes[kBlockThreads / kWave][G::RB][kWave][4];  // 8 KB per wave
            consume_lds<G, G::RB>(codes_in, codes_stride, scales_in, scales_stride, n_inputs, numel, o, acc,
                                  lds_codes[wib], lane);
            // the code slots are free again: every load into them has landed and been read
            if constexpr (BITS_OUT == 0 && ZPP_DRR_SUM_XPOSE && E > 8) {
                static_assert(G::RB * 4 >= E, "the code slots hold the wave's sums");
                xp = &lds_codes[wib][0][0][0];
            }
        } else {
            consume_padded<G, G::RB>(codes_in, codes_stride, scales_in, scales_stride, n_inputs, o, acc);
        }
        if constexpr (BITS_OUT == 0 && ZPP_DRR_SUM_XPOSE && E > 8 && !(ZPP_DRR_LDS && G::U == 1 && G::ND == 4 && !G::OVERLAP)) {
            __shared__ __attribute__((aligned(16))) uint32_t lds_sums[kBlockThreads / kWave][kWave * E];
            xp = lds_sums[wib];
        }
        finish_tile<G, BITS_OUT, AVG>(acc, ok, e, t0, n, lane, out, xp);
    }
}

// The outputs of the launch covering elements [done, done + n): the keep
// window clipped to it, and each output's base for its first element.
template <int BITS_OUT, int LOG2B>
DrrOut chunk_out(const DrrArgs &a, int64_t done, int64_t n) {
    const int64_t k0 = a.keep_begin, k1 = a.keep_begin + a.keep_len;
    const int64_t kb = k0 - done < 0 ? 0 : (k0 - done > n ? n : k0 - done);
    const int64_t ke = k1 - done < 0 ? 0 : (k1 - done > n ? n : k1 - done);
    // elements before `done` that sit in the window
    const int64_t skipped = done - k0 < 0 ? 0 : (done - k0 > a.keep_len ? a.keep_len : done - k0);
    const int64_t send0 = done - skipped;   // output position of the chunk's first element outside the window
    const int64_t keep0 = done + kb - k0;   // keep position of the chunk's first element inside it
    DrrOut o;
    o.codes_out = a.codes_out ? static_cast<uint8_t *>(a.codes_out) + send0 * BITS_OUT / 8 : nullptr;
    o.scales_out = a.scales_out ? a.scales_out + (send0 >> LOG2B) : nullptr;
    o.sum_out = a.sum_out ? a.sum_out + done : nullptr;
    o.divisor = a.divisor;
    o.kb = static_cast<uint32_t>(kb);
    o.klen = static_cast<uint32_t>(ke - kb);
    const bool win = a.keep_len > 0 && ke > kb;
    o.codes_keep = win ? static_cast<uint8_t *>(a.codes_keep) + keep0 * BITS_OUT / 8 : nullptr;
    o.scales_keep = win ? a.scales_keep + (keep0 >> LOG2B) : nullptr;
    return o;
}

// One launch per chunk of at most kDrrChunk elements (blocks are independent).
template <int BITS_IN, int BITS_OUT, int LOG2B, int E, bool AVG>
hipError_t launch_e(const DrrArgs &a) {
    using G = DrrGeom<BITS_IN, BITS_OUT, LOG2B, E>;
    for (int64_t done = 0; done < a.numel; done += kDrrChunk) {
        const int64_t n = a.numel - done < kDrrChunk ? a.numel - done : kDrrChunk;
        const int64_t tiles = (n + G::TILE - 1) / G::TILE;
        const uint8_t *ci = static_cast<const uint8_t *>(a.codes_in) + done * BITS_IN / 8;
        const float *si = a.scales_in + (done >> LOG2B);
        const DrrOut o = chunk_out<BITS_OUT, LOG2B>(a, done, n);
        drr_kernel<BITS_IN, BITS_OUT, LOG2B, E, AVG><<<stream_grid(tiles), kBlockThreads, 0, a.stream>>>(
            ci, a.cstride, si, a.sstride, a.n_inputs, static_cast<int>(n), o);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

template <int BITS_IN, int BITS_OUT, int LOG2B, bool AVG>
hipError_t launch(const DrrArgs &a) {
    using Wide = DrrGeom<BITS_IN, BITS_OUT, LOG2B, ZPP_DRR_WIDE_E>;
    const int64_t wide_waves = (a.numel + Wide::TILE - 1) / Wide::TILE;
    // Blocks of 4096 elements span 8 narrow segments per tile, whose codes
    // and sums do not fit the registers (hundreds of bytes of spills with
    // 8-bit inputs): they always take the wide layout, 2 segments per tile,
    // which measured faster at every size.
    if constexpr (LOG2B >= 12) {
        return launch_e<BITS_IN, BITS_OUT, LOG2B, ZPP_DRR_WIDE_E, AVG>(a);
    } else {
        if (wide_waves >= ZPP_DRR_NARROW_WAVES ||
            (BITS_IN == 4 && a.n_inputs <= ZPP_DRR_FEW_INPUTS && wide_waves >= ZPP_DRR_FEW_INPUTS_WAVES))
            return launch_e<BITS_IN, BITS_OUT, LOG2B, ZPP_DRR_WIDE_E, AVG>(a);
        return launch_e<BITS_IN, BITS_OUT, LOG2B, 8, AVG>(a);
    }
}

template <int BITS_IN, int BITS_OUT, bool AVG>
hipError_t by_block(int log2b, const DrrArgs &a) {
    switch (log2b) {
    case 5: return launch<BITS_IN, BITS_OUT, 5, AVG>(a);
    case 6: return launch<BITS_IN, BITS_OUT, 6, AVG>(a);
    case 7: return launch<BITS_IN, BITS_OUT, 7, AVG>(a);
    case 8: return launch<BITS_IN, BITS_OUT, 8, AVG>(a);
    case 9: return launch<BITS_IN, BITS_OUT, 9, AVG>(a);
    case 10: return launch<BITS_IN, BITS_OUT, 10, AVG>(a);
    case 11: return launch<BITS_IN, BITS_OUT, 11, AVG>(a);
    case 12: return launch<BITS_IN, BITS_OUT, 12, AVG>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace zpp
