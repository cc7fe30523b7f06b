// quantize.hip - per-block symmetric absmax quantization (QWZ 8-bit weights,
// QGZ one-shot 4-bit gradients).
//
// Page "Quantized LLM Training at Scale with ZeRO++", section "The Three
// Pillars of ZeRO++": pillar 1 (QWZ) quantizes the weight tensor chunk by
// chunk to 8 bits before the forward all-gather; pillar 3 (QGZ) quantizes
// each GPU's gradient once, to 4 bits (a quarter of the 16-bit volume),
// before its all-to-all.
//
// Layout of the work. A lane owns E contiguous elements per segment: K
// 16-byte vectors (K = 1: 8 bf16 or 4 fp32 elements; every load instruction
// then reads one contiguous kilobyte, which measured faster than wider lanes
// with half the per-block arithmetic), so a block of B elements spans
// L = B / E lanes, or several whole segments when B is larger than a wave
// segment of 64 E elements. Each wave works on tiles of U segments (all
// loads of a tile issued before any use); a tile that lies wholly inside the
// tensor takes a path without range masks. The block maximum is reduced across its lanes with DPP / permlane
// swaps; the lane at the head of each block stores its scale.
#include "zpp_device.h"
#include "zpp_launch.h"

// Segments per wave tile.
#ifndef ZPP_QUANT_SEGS
#define ZPP_QUANT_SEGS 2
#endif
// 16-byte input vectors per lane per segment.
#ifndef ZPP_QUANT_VECS
#define ZPP_QUANT_VECS 1
#endif

namespace zpp {
namespace {

template <int BITS, int LOG2B, bool F32IN>
struct QuantGeom {
    static constexpr int B = 1 << LOG2B;
    static constexpr int IB = F32IN ? 4 : 2;            // input bytes per element
    static constexpr int K = ZPP_QUANT_VECS;            // 16-byte loads per lane per segment
    static constexpr int ND = 4 * K;                    // input dwords per lane per segment
    static constexpr int E = 16 * K / IB;               // elements per lane per segment
    static constexpr int SEG = kWave * E;               // elements per wave segment
    static constexpr int SPB = B > SEG ? B / SEG : 1;   // segments per block
    static constexpr int L = B >= SEG ? kWave : B / E;  // lanes per block within a segment
    static constexpr int U = SPB > ZPP_QUANT_SEGS ? SPB : ZPP_QUANT_SEGS;  // segments per tile
    static constexpr int NB = U / SPB;                  // scale slots per lane per tile
    static constexpr int TILE = U * SEG;
    static constexpr int CB = E * BITS / 8;             // code bytes per lane per segment
    static constexpr int QMAX = BITS == 8 ? 127 : 7;
    static_assert(E <= B, "a lane's elements must lie in one block");
};

// Store a lane's CB code bytes (16-byte aligned runs when CB >= 16).
template <int CB>
__device__ __forceinline__ void store_codes(uint8_t *dst, const uint32_t *cw) {
    if constexpr (CB >= 16) {
#pragma unroll
        for (int j = 0; j < CB / 16; ++j)
            st_out<u32x4>(dst + 16 * j, u32x4{cw[4 * j], cw[4 * j + 1], cw[4 * j + 2], cw[4 * j + 3]});
    } else if constexpr (CB == 8) {
        st_out<u32x2>(dst, u32x2{cw[0], cw[1]});
    } else {
        static_assert(CB == 4, "code bytes per lane");
        st_out<uint32_t>(dst, cw[0]);
    }
}

// One tile: segments t0 + u * SEG (u < U) of the tensor. FULL: the whole
// tile is in range. Otherwise out-of-range lanes (only whole blocks, since
// numel % B == 0) read element 0, contribute nothing and store nothing.
template <int BITS, int LOG2B, bool F32IN, bool FULL>
__device__ __forceinline__ void quantize_tile(const uint8_t *__restrict__ x, int64_t numel,
                                              uint8_t *__restrict__ codes, float *__restrict__ scales, int64_t t0,
                                              int lane) {
    using G = QuantGeom<BITS, LOG2B, F32IN>;
    constexpr int E = G::E, U = G::U, SPB = G::SPB, NB = G::NB, K = G::K, ND = G::ND;

    u32x4 raw[U][K];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e0 = t0 + static_cast<int64_t>(u) * G::SEG + lane * E;
        ok[u] = FULL || e0 < numel;
        const uint8_t *src = x + (ok[u] ? e0 : 0) * G::IB;
#pragma unroll
        for (int k = 0; k < K; ++k) raw[u][k] = ld_stream<u32x4>(src + 16 * k);
    }
    float v[U][E];
    uint32_t m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t w[ND];
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * k + i] = ok[u] ? raw[u][k][i] : 0u;
        if constexpr (F32IN) {
            uint32_t mx = 0;
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                v[u][i] = as_f(w[i]);
                mx = max(mx, w[i] & 0x7FFFFFFFu);
            }
            m[u] = mx;
        } else {
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                v[u][2 * i] = bf16_lo(w[i]);
                v[u][2 * i + 1] = bf16_hi(w[i]);
            }
            m[u] = bf16_absmax_bits<ND>(w);
        }
    }

    // Block absmax -> scale, one per block (per segment when SPB == 1).
    float s[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        uint32_t mx = 0;
#pragma unroll
        for (int k = 0; k < SPB; ++k) mx = max(mx, m[b * SPB + k]);
        mx = group_max_u32<G::L>(mx);
        s[b] = block_scale<G::QMAX>(as_f(mx));
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e0 = t0 + static_cast<int64_t>(u) * G::SEG + lane * E;
        float mg[E];
        round_codes<E, BITS>(v[u], s[u / SPB], mg);
        if constexpr (G::CB >= 4) {
            uint32_t cw[G::CB / 4];
            pack_codes<E, BITS>(mg, cw);
            if (!ok[u]) continue;
            store_codes<G::CB>(codes + e0 * BITS / 8, cw);
        } else {  // fp32 input, one vector per lane, 4-bit codes: 4 nibbles (offset binary)
            static_assert(E == 4 && BITS == 4, "two code bytes per lane");
            const uint32_t p0 = (as_u(mg[1]) << 4) | (as_u(mg[0]) & 0xFu);
            const uint32_t p1 = (as_u(mg[3]) << 4) | (as_u(mg[2]) & 0xFu);
            const uint32_t half = __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u) ^ 0x8888u;
            if (!ok[u]) continue;
            st_out<uint16_t>(codes + e0 * BITS / 8, static_cast<uint16_t>(half));
        }
        if constexpr (SPB == 1) {
            if ((lane & (G::L - 1)) == 0) scales[e0 >> LOG2B] = s[u];
        } else {
            if (lane == 0 && (u % SPB) == 0) scales[e0 >> LOG2B] = s[u / SPB];
        }
    }
}

// Slices: blockIdx.y is an output slice of `numel` elements. With
// n_nodes * gpus_per_node > 1 the input is read in QGZ reordered slice order
// (output slice position p = first_slice + blockIdx.y reads input slice
// (p % n_nodes) * gpus_per_node + p / n_nodes, see reorder.hip); with one
// slice and n_nodes = gpus_per_node = 1 this is a plain quantize of x.
template <int BITS, int LOG2B, bool F32IN>
__global__ __launch_bounds__(kBlockThreads) void quantize_kernel(const uint8_t *__restrict__ x, int64_t numel,
                                                                 uint8_t *__restrict__ codes,
                                                                 float *__restrict__ scales, int n_nodes,
                                                                 int gpus_per_node, int first_slice) {
    using G = QuantGeom<BITS, LOG2B, F32IN>;
    {
        const int p = first_slice + static_cast<int>(blockIdx.y);
        const int local = p / n_nodes;
        const int64_t src = static_cast<int64_t>(p - local * n_nodes) * gpus_per_node + local;
        x += src * numel * G::IB;
        codes += static_cast<int64_t>(blockIdx.y) * numel * BITS / 8;
        scales += static_cast<int64_t>(blockIdx.y) * (numel >> LOG2B);
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_in_group = wave_in_block();
    const int64_t wave = xcd_block(blockIdx.x, gridDim.x) * (kBlockThreads / kWave) + wave_in_group;
    const int64_t n_waves = static_cast<int64_t>(gridDim.x) * (kBlockThreads / kWave);

    for (int64_t t0 = wave * G::TILE; t0 < numel; t0 += n_waves * G::TILE) {
        if (t0 + G::TILE <= numel)
            quantize_tile<BITS, LOG2B, F32IN, true>(x, numel, codes, scales, t0, lane);
        else
            quantize_tile<BITS, LOG2B, F32IN, false>(x, numel, codes, scales, t0, lane);
    }
}

template <int BITS, int LOG2B, bool F32IN>
hipError_t launch(const void *x, int64_t slice_elems, int n_slices, int n_nodes, int g, int first_slice, void *codes,
                  float *scales, hipStream_t stream) {
    using G = QuantGeom<BITS, LOG2B, F32IN>;
    const int64_t tiles = (slice_elems + G::TILE - 1) / G::TILE;
    const dim3 grid(static_cast<unsigned>(stream_grid(tiles)), static_cast<unsigned>(n_slices));
    quantize_kernel<BITS, LOG2B, F32IN><<<grid, kBlockThreads, 0, stream>>>(
        static_cast<const uint8_t *>(x), slice_elems, static_cast<uint8_t *>(codes), scales, n_nodes, g,
        first_slice);
    return hipGetLastError();
}

struct QArgs {
    const void *x;
    int64_t slice_elems;
    int n_slices, n_nodes, g, first_slice;
    void *codes;
    float *scales;
    hipStream_t stream;
};

template <int BITS, bool F32IN>
hipError_t by_block(int log2b, const QArgs &a) {
#define ZPP_Q(L) launch<BITS, L, F32IN>(a.x, a.slice_elems, a.n_slices, a.n_nodes, a.g, a.first_slice, a.codes, \
                                        a.scales, a.stream)
    switch (log2b) {
    case 5: return ZPP_Q(5);
    case 6: return ZPP_Q(6);
    case 7: return ZPP_Q(7);
    case 8: return ZPP_Q(8);
    case 9: return ZPP_Q(9);
    case 10: return ZPP_Q(10);
    case 11: return ZPP_Q(11);
    case 12: return ZPP_Q(12);
    default: return hipErrorInvalidValue;
    }
#undef ZPP_Q
}

hipError_t dispatch(bool f32_in, int bits, int log2b, const QArgs &a) {
    if (bits == 8) return f32_in ? by_block<8, true>(log2b, a) : by_block<8, false>(log2b, a);
    return f32_in ? by_block<4, true>(log2b, a) : by_block<4, false>(log2b, a);
}

}  // namespace

hipError_t launch_quantize(const void *x, bool f32_in, int64_t numel, int log2b, int bits, void *codes,
                           float *scales, hipStream_t stream) {
    return dispatch(f32_in, bits, log2b, QArgs{x, numel, 1, 1, 1, 0, codes, scales, stream});
}

hipError_t launch_quantize_reordered(const void *x, bool f32_in, int64_t slice_elems, int n_nodes, int gpus_per_node,
                                     int first_slice, int n_slices, int log2b, int bits, void *codes, float *scales,
                                     hipStream_t stream) {
    return dispatch(f32_in, bits, log2b,
                    QArgs{x, slice_elems, n_slices, n_nodes, gpus_per_node, first_slice, codes, scales, stream});
}

}  // namespace zpp
