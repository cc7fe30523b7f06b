// reorder.hip - QGZ tensor-slice reordering.
//
// Page "Quantized LLM Training at Scale with ZeRO++", section "The Three
// Pillars of ZeRO++", pillar 3 (QGZ): before any communication the local
// gradient chunks are swapped so that, after the intra-node hop (contiguous
// chunk j to local rank j) and the inter-node hop (sub-chunk k of that chunk
// to node k), each one lands on the GPU that owns it. Ownership follows the
// reduce-scatter of page "ZeRO Stage 2: Gradient Partitioning" (GPU i keeps
// shard i). With node-major ranks, slice position j*n_nodes + k travels to
// rank k*g + j, so it must hold that rank's slice.
//
// A plain copy with a per-slice source: blockIdx.y is the output slice,
// blockIdx.x strides over its tiles; each thread moves U vectors of V bytes
// (V is the widest power of two, up to 16, dividing the slice size and both
// base addresses), all loads issued before the stores.
#include "zpp_device.h"
#include "zpp_launch.h"

namespace zpp {
namespace {

// 16-byte vectors each thread moves per tile.
#ifndef ZPP_REORDER_VECS
#define ZPP_REORDER_VECS 1
#endif
constexpr int kU = ZPP_REORDER_VECS;

template <int V>
struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

template <int V>
__global__ __launch_bounds__(kBlockThreads) void reorder_kernel(const uint8_t *__restrict__ in,
                                                                uint8_t *__restrict__ out, int64_t slice_bytes,
                                                                int n_nodes, int gpus_per_node) {
    using T = typename Vec<V>::T;
    const int p = blockIdx.y;                 // output slice position
    const int local = p / n_nodes;            // hop-1 destination
    const int node = p - local * n_nodes;     // hop-2 destination
    const int64_t src = static_cast<int64_t>(node) * gpus_per_node + local;
    const uint8_t *s = in + src * slice_bytes;
    uint8_t *d = out + static_cast<int64_t>(p) * slice_bytes;
    const int64_t n_vec = slice_bytes / V;
    constexpr int64_t kTileVec = static_cast<int64_t>(kBlockThreads) * kU;

    for (int64_t t0 = xcd_block(blockIdx.x, gridDim.x) * kTileVec; t0 < n_vec;
         t0 += static_cast<int64_t>(gridDim.x) * kTileVec) {
        T v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = t0 + u * kBlockThreads + threadIdx.x;
            v[u] = ld_stream<T>(s + (i < n_vec ? i : 0) * V);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = t0 + u * kBlockThreads + threadIdx.x;
            if (i < n_vec) st_out<T>(d + i * V, v[u]);
        }
    }
}

template <int V>
hipError_t launch(const void *in, void *out, int64_t slice_bytes, int n_nodes, int g, hipStream_t stream) {
    const int64_t n_vec = slice_bytes / V;
    const int64_t tile = static_cast<int64_t>(kBlockThreads) * kU;
    int64_t gx = (n_vec + tile - 1) / tile;
    if (gx > (1 << 20)) gx = 1 << 20;
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(n_nodes * g));
    reorder_kernel<V><<<grid, kBlockThreads, 0, stream>>>(static_cast<const uint8_t *>(in),
                                                            static_cast<uint8_t *>(out), slice_bytes, n_nodes, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reorder(const void *in, void *out, int64_t slice_bytes, int n_nodes, int gpus_per_node,
                          hipStream_t stream) {
    const uint64_t a = static_cast<uint64_t>(slice_bytes) | reinterpret_cast<uintptr_t>(in) |
                       reinterpret_cast<uintptr_t>(out);
    if ((a & 15) == 0) return launch<16>(in, out, slice_bytes, n_nodes, gpus_per_node, stream);
    if ((a & 7) == 0) return launch<8>(in, out, slice_bytes, n_nodes, gpus_per_node, stream);
    if ((a & 3) == 0) return launch<4>(in, out, slice_bytes, n_nodes, gpus_per_node, stream);
    if ((a & 1) == 0) return launch<2>(in, out, slice_bytes, n_nodes, gpus_per_node, stream);
    return launch<1>(in, out, slice_bytes, n_nodes, gpus_per_node, stream);
}

}  // namespace zpp
