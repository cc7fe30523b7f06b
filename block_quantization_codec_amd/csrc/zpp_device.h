// zpp_device.h - device helpers shared by the codec kernels (gfx950 / CDNA4, wave64).
//
// Internal to the library. Every kernel streams HBM with 16-byte vector
// accesses that are contiguous across the 64 lanes of a wave, reduces block
// maxima across lanes with DPP row operations and the gfx950 permlane swaps
// (no LDS traffic), and keeps all arithmetic in binary32 with fp contraction
// off, so every product and sum is rounded on its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace zpp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;  // 4 waves per workgroup
constexpr float kFltMin = 1.17549435082228750797e-38f;  // smallest normal binary32
// |t - rint(t)| at or above this means t sits within 2^-14 of a half-integer:
// the reciprocal-multiply quotient is then not trusted to round like x / s.
constexpr float kNearTie = 0.49993896484375f;  // 0.5 - 2^-14

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---- global memory -------------------------------------------------------

template <typename T>
__device__ __forceinline__ T ld(const void *p) {
    return *reinterpret_cast<const T *>(p);
}
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

// Two binary32 values rounded to bf16 (nearest, ties to even) and packed,
// `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 ha = static_cast<__bf16>(a);
    __bf16 hb = static_cast<__bf16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// ---- symmetric block quantization of one lane's values --------------------
//
// Given the block scale s (= absmax / Q, correctly rounded), each code is
// rne(fl(x / s)) clamped to [-Q, Q]. The quotient is formed as x * (1/s) with
// hardware reciprocal (error <= 1 ulp). Since |x / s| <= Q (1 + 2^-24) <= 128,
// that product is within 2^-15 of the exact quotient and the correctly
// rounded quotient within 2^-16, so whenever the product lies 2^-14 or more
// away from every half-integer both round to the same integer. Values
// nearer a half-integer, and blocks whose scale is subnormal (where 1/s may
// overflow), are redone with a correctly rounded division.
template <int N, int QMAX>
__device__ __forceinline__ void quantize_values(const float (&x)[N], float s, int32_t (&q)[N]) {
    constexpr float Q = static_cast<float>(QMAX);
    const bool normal_scale = s >= kFltMin;
    const float r = normal_scale ? __builtin_amdgcn_rcpf(s) : 0.0f;
    bool redo = (s != 0.0f) && !normal_scale;
    float n[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float t = x[i] * r;
        n[i] = __builtin_rintf(t);
        redo |= __builtin_fabsf(t - n[i]) >= kNearTie;
    }
    if (redo) {
#pragma unroll
        for (int i = 0; i < N; ++i) n[i] = __builtin_rintf(x[i] / s);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = static_cast<int32_t>(__builtin_amdgcn_fmed3f(n[i], -Q, Q));
}

// ---- code packing ----------------------------------------------------------

// Four int8 codes into a dword, element 0 in the low byte.
__device__ __forceinline__ uint32_t pack_i8x4(int32_t a, int32_t b, int32_t c, int32_t d) {
    return (static_cast<uint32_t>(a) & 0xFFu) | ((static_cast<uint32_t>(b) & 0xFFu) << 8) |
           ((static_cast<uint32_t>(c) & 0xFFu) << 16) | (static_cast<uint32_t>(d) << 24);
}

// Eight int4 codes into a dword, element 0 in the low nibble.
__device__ __forceinline__ uint32_t pack_i4x8(const int32_t *q) {
    uint32_t w = static_cast<uint32_t>(q[0]) & 0xFu;
#pragma unroll
    for (int i = 1; i < 8; ++i) w |= (static_cast<uint32_t>(q[i]) & 0xFu) << (4 * i);
    return w;
}

// Signed code i of a dword holding 8-bit (4 per dword) or 4-bit (8 per dword) codes.
template <int BITS>
__device__ __forceinline__ int32_t code_at(uint32_t w, int i) {
    if constexpr (BITS == 8)
        return static_cast<int32_t>(static_cast<int8_t>(w >> (8 * i)));
    else
        return __builtin_amdgcn_sbfe(static_cast<int32_t>(w), 4 * i, 4);
}

// ---- launch geometry --------------------------------------------------------

// Workgroups for a grid-stride loop over `tiles` wave-sized tiles: enough to
// keep every CU of the current device busy, never more than the work needs.
int stream_grid(int64_t tiles);

}  // namespace zpp
