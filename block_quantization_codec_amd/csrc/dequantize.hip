// dequantize.hip - codes * scale back to binary32 or bfloat16 (gather side of
// the QWZ all-gather).
//
// Page "Quantized LLM Training at Scale with ZeRO++", section "The Three
// Pillars of ZeRO++", pillar 1 (QWZ): weights travel as 8-bit values; the
// receiver needs the 16-bit layer weights back to compute with. Each value
// is the binary32 product code * s_b; bf16 output rounds it to nearest-even.
//
// Segments of 512 elements. bf16 out: a lane owns 8 consecutive elements
// of a segment, 8 (int8) or 4 (int4) code bytes in and one 16-byte store
// out. binary32 out: a lane owns 4 consecutive elements in each half of a
// segment, so that each of its two 16-byte stores is contiguous across the
// wave (with one lane storing 32 consecutive bytes, each store instruction
// writes parts of many cache lines, and the kernel ran at half the rate).
// The block scale is a per-lane load (lanes of one block hit the same
// address). A wave's tile is 1 segment (int8 to bf16, binary32 out) or 2
// (int4 to bf16: its loads of 4 bytes per lane are too few to keep HBM busy
// with one segment, 15% slower; 4 segments 5% slower than 2).
#include "zpp_device.h"
#include "zpp_launch.h"

namespace zpp {
namespace {

constexpr int kE = 8;              // elements per lane per segment
constexpr int kSeg = kWave * kE;   // 512
#ifndef ZPP_DEQUANT_SEGS8
#define ZPP_DEQUANT_SEGS8 1
#endif
#ifndef ZPP_DEQUANT_SEGS4
#define ZPP_DEQUANT_SEGS4 2
#endif
#ifndef ZPP_DEQUANT_SEGS_F32
#define ZPP_DEQUANT_SEGS_F32 1
#endif
// segments per tile
template <int BITS, bool F32OUT>
constexpr int segs() { return F32OUT ? ZPP_DEQUANT_SEGS_F32 : (BITS == 8 ? ZPP_DEQUANT_SEGS8 : ZPP_DEQUANT_SEGS4); }
template <int BITS, bool F32OUT>
constexpr int tile() { return segs<BITS, F32OUT>() * kSeg; }

template <int BITS, bool F32OUT>
__global__ __launch_bounds__(kBlockThreads) void dequantize_kernel(const uint8_t *__restrict__ codes,
                                                                   const float *__restrict__ scales, int64_t numel,
                                                                   int log2b, uint8_t *__restrict__ y) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = xcd_block(blockIdx.x, gridDim.x) * (kBlockThreads / kWave) + wave_in_block();
    const int64_t n_waves = static_cast<int64_t>(gridDim.x) * (kBlockThreads / kWave);
    constexpr int kU = segs<BITS, F32OUT>();
    constexpr int kTile = tile<BITS, F32OUT>();

    for (int64_t t0 = wave * kTile; t0 < numel; t0 += n_waves * kTile) {
        if constexpr (F32OUT) {
            // binary32 out: the lane takes 4 elements from each half of the segment, so
            // each 16-byte store covers 1 KB that is contiguous across the wave
            constexpr int kH = kSeg / 2;
            uint32_t w[kU][2];
            float s[kU][2];
            bool ok[kU][2];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t e0 = t0 + static_cast<int64_t>(u) * kSeg + h * kH + lane * 4;
                    ok[u][h] = e0 < numel;
                    const int64_t e = ok[u][h] ? e0 : 0;
                    if constexpr (BITS == 8)
                        w[u][h] = ld_stream<uint32_t>(codes + e);
                    else
                        w[u][h] = ld_stream<uint16_t>(codes + e / 2);
                    s[u][h] = scales[e >> log2b];
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (!ok[u][h]) continue;
                    const int64_t e0 = t0 + static_cast<int64_t>(u) * kSeg + h * kH + lane * 4;
                    float f[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) f[i] = static_cast<float>(code_at<BITS>(w[u][h], i)) * s[u][h];
                    st_out<u32x4>(y + e0 * 4, u32x4{as_u(f[0]), as_u(f[1]), as_u(f[2]), as_u(f[3])});
                }
            }
        } else {
            // bf16 out: 8 consecutive elements per lane and segment
            uint32_t w[kU][2];
            float s[kU];
            bool ok[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t e0 = t0 + static_cast<int64_t>(u) * kSeg + lane * kE;
                ok[u] = e0 < numel;
                const int64_t e = ok[u] ? e0 : 0;
                if constexpr (BITS == 8) {
                    const u32x2 c = ld_stream<u32x2>(codes + e);
                    w[u][0] = c[0];
                    w[u][1] = c[1];
                } else {
                    w[u][0] = ld_stream<uint32_t>(codes + e / 2);
                    w[u][1] = 0;
                }
                s[u] = scales[e >> log2b];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (!ok[u]) continue;
                const int64_t e0 = t0 + static_cast<int64_t>(u) * kSeg + lane * kE;
                float f[kE];
#pragma unroll
                for (int i = 0; i < kE; ++i) {
                    const int32_t q = (BITS == 8) ? code_at<8>(w[u][i / 4], i % 4) : code_at<4>(w[u][0], i);
                    f[i] = static_cast<float>(q) * s[u];
                }
                st_out<u32x4>(y + e0 * 2, u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                            pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])});
            }
        }
    }
}

template <int BITS, bool F32OUT>
hipError_t launch(const void *codes, const float *scales, int64_t numel, int log2b, void *y, hipStream_t stream) {
    const int64_t tiles = (numel + tile<BITS, F32OUT>() - 1) / tile<BITS, F32OUT>();
    dequantize_kernel<BITS, F32OUT><<<stream_grid(tiles), kBlockThreads, 0, stream>>>(
        static_cast<const uint8_t *>(codes), scales, numel, log2b, static_cast<uint8_t *>(y));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const void *codes, const float *scales, int bits, int64_t numel, int log2b, void *y,
                             bool f32_out, hipStream_t stream) {
    if (bits == 8)
        return f32_out ? launch<8, true>(codes, scales, numel, log2b, y, stream)
                       : launch<8, false>(codes, scales, numel, log2b, y, stream);
    return f32_out ? launch<4, true>(codes, scales, numel, log2b, y, stream)
                   : launch<4, false>(codes, scales, numel, log2b, y, stream);
}

}  // namespace zpp
