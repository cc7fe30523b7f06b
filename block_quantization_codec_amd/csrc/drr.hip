// drr.hip - fused dequantize -> binary32 reduce -> requantize (the hop step of QGZ).
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
// acc = fl(acc + fl(code_r * s_r)). The first term is formed as
// fma(code_0, s_0, +0), which equals fl(+0 + fl(code_0 * s_0)) exactly (one
// rounding of the exact product; a nonzero integer code times a nonzero
// scale never rounds to zero); every later product and sum is rounded on its
// own, never fused.
//
// Layout of the work: a lane owns 32 consecutive elements of a 2048-element
// wave segment, i.e. one 16-byte vector of 4-bit codes (two of 8-bit codes)
// per input, so each load instruction reads one contiguous kilobyte of an
// input. Inputs are read four at a time, all loads of a batch in flight
// before the batch is summed in input order. The requantized block maximum
// is reduced across the block's lanes with DPP / permlane swaps.
#include "zpp_device.h"
#include "zpp_launch.h"

namespace zpp {
namespace {

constexpr int kE = 32;              // elements per lane per segment
constexpr int kSeg = kWave * kE;    // 2048
constexpr int kRB = 4;              // inputs per load batch

template <int BITS_IN_, int BITS_OUT, int LOG2B_>
struct DrrGeom {
    static constexpr int BITS_IN = BITS_IN_;
    static constexpr int LOG2B = LOG2B_;
    static constexpr int B = 1 << LOG2B;
    static constexpr int SPB = B > kSeg ? B / kSeg : 1;    // segments per block (= per tile)
    static constexpr int L = B >= kSeg ? kWave : B / kE;   // lanes per block within a segment
    static constexpr int U = SPB;
    static constexpr int TILE = U * kSeg;
    static constexpr int NV = kE * BITS_IN / 8 / 16;       // 16-byte vectors per lane per input
    static constexpr int QMAX = BITS_OUT == 8 ? 127 : 7;
};

// Add inputs r0 .. r0+NB-1 (in that order) into acc. FIRST: input r0 starts
// the sums (acc = fma(q, s, +0), equal to +0 + fl(q * s)).
template <typename G, int NB, bool FIRST>
__device__ __forceinline__ void sum_batch(const uint8_t *__restrict__ codes_in, int64_t codes_stride,
                                          const float *__restrict__ scales_in, int64_t scales_stride, int r0,
                                          const int64_t (&e)[G::U], float (&acc)[G::U][kE]) {
    constexpr int U = G::U, NV = G::NV, BITS_IN = G::BITS_IN;
    constexpr int WPV = 4;                 // dwords per vector
    constexpr int CPW = 32 / BITS_IN;      // codes per dword
    u32x4 w[NB][U][NV];
    float s[NB][U];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const uint8_t *c = codes_in + static_cast<int64_t>(r0 + k) * codes_stride;
        const float *sc = scales_in + static_cast<int64_t>(r0 + k) * scales_stride;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int v = 0; v < NV; ++v) w[k][u][v] = ld<u32x4>(c + e[u] * BITS_IN / 8 + 16 * v);
            s[k][u] = sc[e[u] >> G::LOG2B];
        }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int i = 0; i < kE; ++i) {
                const uint32_t word = w[k][u][i / (CPW * WPV)][(i / CPW) % WPV];
                const float q = static_cast<float>(code_at<BITS_IN>(word, i % CPW));
                if (FIRST && k == 0)
                    acc[u][i] = __builtin_fmaf(q, s[k][u], 0.0f);
                else
                    acc[u][i] = acc[u][i] + q * s[k][u];
            }
        }
    }
}

template <int BITS_IN, int BITS_OUT, int LOG2B>
__global__ __launch_bounds__(kBlockThreads) void drr_kernel(const uint8_t *__restrict__ codes_in,
                                                            int64_t codes_stride,
                                                            const float *__restrict__ scales_in,
                                                            int64_t scales_stride, int n_inputs, int64_t numel,
                                                            uint8_t *__restrict__ codes_out,
                                                            float *__restrict__ scales_out,
                                                            float *__restrict__ sum_out) {
    using G = DrrGeom<BITS_IN, BITS_OUT, LOG2B>;
    constexpr int U = G::U;

    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kBlockThreads / kWave) + (threadIdx.x / kWave);
    const int64_t n_waves = static_cast<int64_t>(gridDim.x) * (kBlockThreads / kWave);

    for (int64_t t0 = wave * G::TILE; t0 < numel; t0 += n_waves * G::TILE) {
        int64_t e[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e0 = t0 + static_cast<int64_t>(u) * kSeg + lane * kE;
            ok[u] = e0 < numel;
            e[u] = ok[u] ? e0 : 0;
        }

        float acc[U][kE];
        // Inputs are consumed in batches whose loads are all issued before
        // the batch is summed; the first batch starts the sums.
        int r = 0;
        if (n_inputs >= kRB) {
            sum_batch<G, kRB, true>(codes_in, codes_stride, scales_in, scales_stride, 0, e, acc);
            for (r = kRB; r + kRB <= n_inputs; r += kRB)
                sum_batch<G, kRB, false>(codes_in, codes_stride, scales_in, scales_stride, r, e, acc);
        } else {
            sum_batch<G, 1, true>(codes_in, codes_stride, scales_in, scales_stride, 0, e, acc);
            r = 1;
        }
        for (; r < n_inputs; ++r)
            sum_batch<G, 1, false>(codes_in, codes_stride, scales_in, scales_stride, r, e, acc);

        if (sum_out != nullptr) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!ok[u]) continue;
                float *dst = sum_out + e[u];
#pragma unroll
                for (int v = 0; v < kE / 4; ++v)
                    st<u32x4>(dst + 4 * v, u32x4{as_u(acc[u][4 * v]), as_u(acc[u][4 * v + 1]),
                                                 as_u(acc[u][4 * v + 2]), as_u(acc[u][4 * v + 3])});
            }
        }

        if constexpr (BITS_OUT != 0) {
            uint32_t mx = 0;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < kE; ++i) mx = max(mx, as_u(acc[u][i]) & 0x7FFFFFFFu);
            if (!ok[0]) mx = 0;
            mx = group_max_u32<G::L>(mx);
            const float sc = as_f(mx) / static_cast<float>(G::QMAX);  // correctly rounded division
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int32_t q[kE];
                quantize_values<kE, G::QMAX>(acc[u], sc, q);
                if (!ok[u]) continue;
                uint8_t *dst = codes_out + e[u] * BITS_OUT / 8;
                if constexpr (BITS_OUT == 4) {
                    st<u32x4>(dst, u32x4{pack_i4x8(q), pack_i4x8(q + 8), pack_i4x8(q + 16), pack_i4x8(q + 24)});
                } else {
#pragma unroll
                    for (int v = 0; v < 2; ++v)
                        st<u32x4>(dst + 16 * v,
                                  u32x4{pack_i8x4(q[16 * v], q[16 * v + 1], q[16 * v + 2], q[16 * v + 3]),
                                        pack_i8x4(q[16 * v + 4], q[16 * v + 5], q[16 * v + 6], q[16 * v + 7]),
                                        pack_i8x4(q[16 * v + 8], q[16 * v + 9], q[16 * v + 10], q[16 * v + 11]),
                                        pack_i8x4(q[16 * v + 12], q[16 * v + 13], q[16 * v + 14], q[16 * v + 15])});
                }
                if (u == 0 && (lane & (G::L - 1)) == 0) scales_out[e[u] >> LOG2B] = sc;
            }
        }
    }
}

template <int BITS_IN, int BITS_OUT, int LOG2B>
hipError_t launch(const void *codes_in, int64_t cstride, const float *scales_in, int64_t sstride, int n_inputs,
                  int64_t numel, void *codes_out, float *scales_out, float *sum_out, hipStream_t stream) {
    using G = DrrGeom<BITS_IN, BITS_OUT, LOG2B>;
    const int64_t tiles = (numel + G::TILE - 1) / G::TILE;
    drr_kernel<BITS_IN, BITS_OUT, LOG2B><<<stream_grid(tiles), kBlockThreads, 0, stream>>>(
        static_cast<const uint8_t *>(codes_in), cstride, scales_in, sstride, n_inputs, numel,
        static_cast<uint8_t *>(codes_out), scales_out, sum_out);
    return hipGetLastError();
}

template <int BITS_IN, int BITS_OUT>
hipError_t by_block(int log2b, const void *ci, int64_t cs, const float *si, int64_t ss, int r, int64_t n, void *co,
                    float *so, float *sum, hipStream_t st) {
    switch (log2b) {
    case 5: return launch<BITS_IN, BITS_OUT, 5>(ci, cs, si, ss, r, n, co, so, sum, st);
    case 6: return launch<BITS_IN, BITS_OUT, 6>(ci, cs, si, ss, r, n, co, so, sum, st);
    case 7: return launch<BITS_IN, BITS_OUT, 7>(ci, cs, si, ss, r, n, co, so, sum, st);
    case 8: return launch<BITS_IN, BITS_OUT, 8>(ci, cs, si, ss, r, n, co, so, sum, st);
    case 9: return launch<BITS_IN, BITS_OUT, 9>(ci, cs, si, ss, r, n, co, so, sum, st);
    case 10: return launch<BITS_IN, BITS_OUT, 10>(ci, cs, si, ss, r, n, co, so, sum, st);
    case 11: return launch<BITS_IN, BITS_OUT, 11>(ci, cs, si, ss, r, n, co, so, sum, st);
    case 12: return launch<BITS_IN, BITS_OUT, 12>(ci, cs, si, ss, r, n, co, so, sum, st);
    default: return hipErrorInvalidValue;
    }
}

template <int BITS_IN>
hipError_t by_out(int bits_out, int log2b, const void *ci, int64_t cs, const float *si, int64_t ss, int r,
                  int64_t n, void *co, float *so, float *sum, hipStream_t st) {
    switch (bits_out) {
    case 0: return by_block<BITS_IN, 0>(log2b, ci, cs, si, ss, r, n, co, so, sum, st);
    case 4: return by_block<BITS_IN, 4>(log2b, ci, cs, si, ss, r, n, co, so, sum, st);
    case 8: return by_block<BITS_IN, 8>(log2b, ci, cs, si, ss, r, n, co, so, sum, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_drr(const void *codes_in, int64_t codes_stride, const float *scales_in, int64_t scales_stride,
                      int n_inputs, int bits_in, int64_t numel, int log2b, void *codes_out, float *scales_out,
                      int bits_out, float *sum_out, hipStream_t stream) {
    if (bits_in == 8)
        return by_out<8>(bits_out, log2b, codes_in, codes_stride, scales_in, scales_stride, n_inputs, numel,
                         codes_out, scales_out, sum_out, stream);
    return by_out<4>(bits_out, log2b, codes_in, codes_stride, scales_in, scales_stride, n_inputs, numel, codes_out,
                     scales_out, sum_out, stream);
}

}  // namespace zpp
