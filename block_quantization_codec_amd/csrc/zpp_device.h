// zpp_device.h - device helpers shared by the codec kernels (gfx950 / CDNA4, wave64).
//
// Internal to the library. Every kernel streams HBM with vector accesses
// that are contiguous across the 64 lanes of a wave (inputs read once with
// non-temporal loads, bulk outputs written with streaming stores), reduces
// block maxima across lanes with DPP row operations and the gfx950 permlane
// swaps (no LDS traffic), and keeps all arithmetic in binary32 with fp
// contraction off, so every product and sum is rounded on its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace zpp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;  // 4 waves per workgroup
constexpr float kFltMin = 1.17549435082228750797e-38f;  // smallest normal binary32

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---- global memory -------------------------------------------------------

template <typename T>
__device__ __forceinline__ T ld(const void *p) {
    return *reinterpret_cast<const T *>(p);
}
// Streaming read: non-temporal hint, the data is used once.
template <typename T>
__device__ __forceinline__ T ld_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
}
template <typename T>
__device__ __forceinline__ void st(void *p, T v) {
    *reinterpret_cast<T *>(p) = v;
}
template <typename T>
__device__ __forceinline__ void st_stream(void *p, T v) {
    __builtin_nontemporal_store(v, reinterpret_cast<T *>(p));
}
// Bulk outputs (codes, values, sums) are written with streaming stores: an
// ordinary store leaves dirty lines in L2 and the Infinity Cache that the
// next kernel then pays to write back, while streaming stores go out to HBM
// inside the kernel that produced them.
#ifndef ZPP_STREAM_STORES
#define ZPP_STREAM_STORES 1
#endif
template <typename T>
__device__ __forceinline__ void st_out(void *p, T v) {
    if constexpr (ZPP_STREAM_STORES != 0)
        st_stream<T>(p, v);
    else
        st<T>(p, v);
}

// ---- lane-group maximum of non-negative binary32 bit patterns -------------
//
// Non-negative floats order like their bit patterns, so the block absmax is
// an unsigned-integer maximum. L lanes (a power of two, aligned group) end
// up holding the group's maximum.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lane group must be a power of two <= 64");
    if constexpr (L >= 2) v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (L >= 4) v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (L >= 8) v = max(v, dpp_u32<0x141>(v));  // row_half_mirror: other quad
    if constexpr (L >= 16) v = max(v, dpp_u32<0x140>(v)); // row_mirror: other half-row
    if constexpr (L >= 32) {                              // rows 0<->1, 2<->3
        auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = max(static_cast<uint32_t>(p[0]), static_cast<uint32_t>(p[1]));
    }
    if constexpr (L >= 64) {                              // lanes 0-31 <-> 32-63
        auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = max(static_cast<uint32_t>(p[0]), static_cast<uint32_t>(p[1]));
    }
    return v;
}

// ---- bfloat16 --------------------------------------------------------------

// The two bf16 values packed in a dword, widened exactly to binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// Largest magnitude among the 2*N bf16 values of N dwords, as binary32 bits
// (packed 16-bit maxima of the sign-cleared halves, then the two halves).
template <int N>
__device__ __forceinline__ uint32_t bf16_absmax_bits(const uint32_t *w) {
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < N; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    const uint32_t b = __builtin_bit_cast(uint32_t, m);
    return max(b << 16, b & 0xFFFF0000u);
}

// Two binary32 values rounded to bf16 (nearest, ties to even) and packed,
// `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 ha = static_cast<__bf16>(a);
    __bf16 hb = static_cast<__bf16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// ---- block scale: s = RN(a / Q) ------------------------------------------
//
// For a >= 2^-90, RN(a / Q) == fma(a, H, RN(a * L)) with H = RN(1/Q) and
// L = RN(1/Q - H): the identity holds for every binary32 significand for
// Q = 127 and Q = 7 (checked exhaustively), and carries over to every binade
// from 2^-90 up because all terms stay normal, so a power-of-two change of a
// scales every step exactly. Smaller maxima take a correctly rounded division.
template <int QMAX>
struct InvQ;
template <>
struct InvQ<127> {
    static constexpr float H = 0x1.020408p-7f;
    static constexpr float L = 0x1.020408p-35f;
};
template <>
struct InvQ<7> {
    static constexpr float H = 0x1.24924ap-3f;
    static constexpr float L = -0x1.b6db6ep-28f;
};

template <int QMAX>
__device__ __forceinline__ float block_scale(float a) {
    if (a >= 0x1p-90f) return __builtin_fmaf(a, InvQ<QMAX>::H, a * InvQ<QMAX>::L);
    return a / static_cast<float>(QMAX);
}

// ---- symmetric block quantization of one lane's values --------------------
//
// Each code is rne(fl(x / s)) clamped to [-Q, Q]. For s >= 2^-96 the
// correctly rounded quotient comes from Markstein's division with the
// correctly rounded reciprocal y = RN(1/s) (one IEEE division per block):
//   q0 = RN(x * y),  r = fma(-q0, s, x) (exact: no underflow for |x| >= 2^-103),
//   q1 = fma(r, y, q0) = RN(x / s).
// Checked exhaustively against x / s on every (x, absmax) pair of finite
// bfloat16 values for Q = 127 and 7 (no code differs; quotients differ only
// below 2^-29, where |x| < 2^-103 and the code is 0 either way), and on 3.6e9
// binary32 values within 3 ulps of every half-integer multiple of s. Since
// |x / s| <= Q (1 + 2^-24), no clamp is needed there. Smaller scales (and
// s == 0, which gives code 0) use a correctly rounded division and the clamp.
//
// Rounding and encoding use the binary32 "magic number" 1.5 * 2^23: for
// |q| < 2^22, q + 1.5*2^23 rounds q to an integer (ties to even: the magic
// number is even) and leaves that integer in the low significand bits. With
// the plain magic number the low byte is the two's-complement 8-bit code;
// with 8 added, the low nibble holds code + 8 in [1, 15] (offset binary,
// turned into two's complement by flipping bit 3).
template <int BITS>
struct Codes {
    static constexpr int QMAX = BITS == 8 ? 127 : 7;
    static constexpr float MAGIC = BITS == 8 ? 12582912.0f : 12582920.0f;
};

// Rounded codes of N values, as magic-number floats.
template <int N, int BITS>
__device__ __forceinline__ void round_codes(const float (&x)[N], float s, float (&m)[N]) {
    using C = Codes<BITS>;
    if (s >= 0x1p-96f) {
        const float y = 1.0f / s;  // correctly rounded reciprocal
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float q0 = x[i] * y;
            const float r = __builtin_fmaf(-q0, s, x[i]);
            m[i] = __builtin_fmaf(r, y, q0) + C::MAGIC;
        }
    } else {
        constexpr float Q = static_cast<float>(C::QMAX);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float n = s == 0.0f ? 0.0f : __builtin_amdgcn_fmed3f(__builtin_rintf(x[i] / s), -Q, Q);
            m[i] = n + C::MAGIC;
        }
    }
}

// Pack rounded codes: 8-bit -> one dword per 4 values, 4-bit -> one dword
// per 8 values; element 0 in the lowest byte / nibble.
template <int N, int BITS>
__device__ __forceinline__ void pack_codes(const float (&m)[N], uint32_t (&w)[N * BITS / 32]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const uint32_t lo = __builtin_amdgcn_perm(as_u(m[4 * k + 1]), as_u(m[4 * k]), 0x0C0C0400u);
            const uint32_t hi = __builtin_amdgcn_perm(as_u(m[4 * k + 3]), as_u(m[4 * k + 2]), 0x04000C0Cu);
            w[k] = lo | hi;
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) {
            uint32_t p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)  // low byte: offset nibble 2j | offset nibble 2j+1 << 4
                p[j] = (as_u(m[8 * k + 2 * j + 1]) << 4) | as_u(m[8 * k + 2 * j]);
            const uint32_t lo = __builtin_amdgcn_perm(p[1], p[0], 0x0C0C0400u);
            const uint32_t hi = __builtin_amdgcn_perm(p[3], p[2], 0x04000C0Cu);
            w[k] = (lo | hi) ^ 0x88888888u;
        }
    }
}

// ---- code unpacking ----------------------------------------------------------

// Signed code i of a dword holding 8-bit (4 per dword) or 4-bit (8 per dword) codes.
template <int BITS>
__device__ __forceinline__ int32_t code_at(uint32_t w, int i) {
    if constexpr (BITS == 8)
        return static_cast<int32_t>(static_cast<int8_t>(w >> (8 * i)));
    else
        return __builtin_amdgcn_sbfe(static_cast<int32_t>(w), 4 * i, 4);
}

// ---- launch geometry --------------------------------------------------------

// This wave's index within its workgroup, as a value the compiler knows to be
// the same in every lane: loops and addresses derived from it stay in scalar
// registers and branches on it are uniform.
__device__ __forceinline__ int wave_in_block() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Renumbering them so that each XCD takes one contiguous run of the grid keeps
// neighbouring tiles, which share cache lines of the small scale arrays, in
// the same L2. A bijection on [0, grid) for any grid size.
#ifndef ZPP_XCD_SWIZZLE
#define ZPP_XCD_SWIZZLE 1
#endif
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t xcd_block(int64_t bid, int64_t grid) {
    if (!ZPP_XCD_SWIZZLE) return bid;
    const int64_t xcd = bid % kXcds, k = bid / kXcds;
    const int64_t q = grid / kXcds, r = grid % kXcds;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + k;
}


// Workgroups for a grid-stride loop over `tiles` wave-sized tiles: enough to
// keep every CU of the current device busy, never more than the work needs.
int stream_grid(int64_t tiles);

}  // namespace zpp
