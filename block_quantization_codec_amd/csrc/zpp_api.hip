// zpp_api.hip - the C ABI declared in include/zpp.h.
//
// Every entry point validates its arguments on the host before touching the
// GPU: pure argument checks first (null pointers, sizes, block, bit widths,
// alignment, overlapping outputs), then checks with the HIP runtime that
// every pointer is memory the GPU can address and that each buffer's whole
// byte range lies inside its allocation (unless the caller has switched
// those off with zpp_set_pointer_checks). Only then is a kernel launched on
// the caller's stream. Any failure returns a status code with nothing
// launched and every output untouched.
#include <atomic>
#include <cstdint>

#include "../../include/zpp.h"
#include "zpp_device.h"
#include "zpp_launch.h"

namespace zpp {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

}  // namespace

// Workgroups per CU a launch is capped at; 0 launches one wave per tile (no
// grid-stride iterations), which measured fastest for every kernel here on
// MI355X (one short-lived wave per tile keeps more loads in flight than a few
// long-lived waves that alternate between loading and computing).
#ifndef ZPP_GRID_CAP_PER_CU
#define ZPP_GRID_CAP_PER_CU 0
#endif

// A launch's work-items (workgroups x 256) must fit in 32 bits. Past that
// many tiles (2^35 elements for dequantize, 2^36 for the bf16 quantizers)
// the waves take further tiles in their grid-stride loops.
constexpr int64_t kMaxGridBlocks = INT64_C(0xFFFFFFFF) / kBlockThreads;

int stream_grid(int64_t tiles) {
    const int64_t want = (tiles + (kBlockThreads / kWave) - 1) / (kBlockThreads / kWave);
    int64_t cap = static_cast<int64_t>(ZPP_GRID_CAP_PER_CU) * device_cus();
    if (cap <= 0 || cap > kMaxGridBlocks) cap = kMaxGridBlocks;
    const int64_t g = want < cap ? want : cap;
    return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace zpp

namespace {

struct Range {
    const void *p;
    int64_t bytes;
};

bool is_pow2_block(int32_t b) { return b >= ZPP_MIN_BLOCK && b <= ZPP_MAX_BLOCK && (b & (b - 1)) == 0; }

int log2_of(int32_t b) {
    int l = 0;
    while ((1 << l) < b) ++l;
    return l;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(Range a, Range b) {
    if (a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

// Whether calls query the HIP runtime about their pointers (see
// zpp_set_pointer_checks); the pure argument checks always run.
std::atomic<int> g_pointer_checks{1};

// The HIP-runtime checks of one call: every pointer must be memory the
// current GPU can address, and [p, p + bytes) must lie in one allocation.
// The current device is queried once per call, and a buffer inside an
// allocation already validated in this call needs no further queries (its
// memory type and device are the allocation's).
class PointerChecks {
  public:
    template <size_t N>
    zpp_status all(const Range (&rs)[N]) {
        if (g_pointer_checks.load(std::memory_order_relaxed) == 0) return ZPP_OK;
        for (const Range &r : rs) {
            const zpp_status s = one(r);
            if (s != ZPP_OK) return s;
        }
        return ZPP_OK;
    }

  private:
    struct Alloc {
        uintptr_t b0, b1;
    };
    Alloc seen_[8];
    int n_seen_ = 0;
    int dev_ = -1;

    zpp_status one(Range r) {
        if (r.bytes <= 0) return ZPP_OK;
        const uintptr_t p0 = reinterpret_cast<uintptr_t>(r.p);
        const uintptr_t p1 = p0 + static_cast<uintptr_t>(r.bytes);
        for (int i = 0; i < n_seen_; ++i)
            if (seen_[i].b0 <= p0 && p1 <= seen_[i].b1) return ZPP_OK;
        hipPointerAttribute_t attr;
        hipError_t e = hipPointerGetAttributes(&attr, r.p);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return ZPP_ERR_POINTER;
        }
        if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged && attr.type != hipMemoryTypeHost &&
            attr.type != hipMemoryTypeUnified)
            return ZPP_ERR_POINTER;
        if (attr.type == hipMemoryTypeHost && attr.devicePointer == nullptr) return ZPP_ERR_POINTER;
        if (attr.type == hipMemoryTypeDevice) {  // another GPU's memory needs peer access from this one
            if (dev_ < 0 && hipGetDevice(&dev_) != hipSuccess) {
                (void)hipGetLastError();
                dev_ = -1;
                return ZPP_ERR_POINTER;
            }
            if (attr.device != dev_) {
                int can = 0;
                if (hipDeviceCanAccessPeer(&can, dev_, attr.device) != hipSuccess || !can) {
                    (void)hipGetLastError();
                    return ZPP_ERR_POINTER;
                }
            }
        }
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        e = hipMemGetAddressRange(&base, &size, const_cast<void *>(r.p));
        if (e == hipSuccess && base != nullptr && size > 0) {
            const uintptr_t b0 = reinterpret_cast<uintptr_t>(base);
            if (p0 < b0 || p1 > b0 + size) return ZPP_ERR_ARG;
            if (n_seen_ < 8) seen_[n_seen_++] = Alloc{b0, b0 + size};
        } else {
            (void)hipGetLastError();
        }
        return ZPP_OK;
    }
};

template <size_t N>
zpp_status check_all(const Range (&rs)[N]) {
    return PointerChecks().all(rs);
}

// A triple-chevron launch reports failure only through the thread's pending
// HIP error. Clear whatever an earlier, unrelated call left there first, so
// that a good launch is never reported as failed because of it.
template <class Launch>
zpp_status launch_checked(Launch &&launch) {
    (void)hipGetLastError();
    if (launch() != hipSuccess) {
        (void)hipGetLastError();
        return ZPP_ERR_LAUNCH;
    }
    return ZPP_OK;
}

int64_t code_bytes(int64_t numel, int32_t bits) { return numel * bits / 8; }

}  // namespace

extern "C" {

zpp_status zpp_quantize_blocks(const void *x, int32_t x_dtype, int64_t numel, int32_t block, int32_t bits,
                               void *codes, float *scales, void *stream) {
    if (x_dtype != ZPP_BF16 && x_dtype != ZPP_FP32) return ZPP_ERR_ARG;
    if (bits != 8 && bits != 4) return ZPP_ERR_ARG;
    if (!is_pow2_block(block) || numel < 0 || numel > ZPP_MAX_NUMEL || numel % block != 0) return ZPP_ERR_ARG;
    if (numel == 0) return ZPP_OK;
    if (!x || !codes || !scales) return ZPP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return ZPP_ERR_ALIGN;
    const int64_t in_bytes = numel * (x_dtype == ZPP_BF16 ? 2 : 4);
    const Range in{x, in_bytes}, oc{codes, code_bytes(numel, bits)}, os{scales, 4 * (numel / block)};
    if (overlap(oc, in) || overlap(os, in) || overlap(oc, os)) return ZPP_ERR_OVERLAP;
    const Range all[] = {in, oc, os};
    if (zpp_status s = check_all(all); s != ZPP_OK) return s;
    return launch_checked([&] {
        return zpp::launch_quantize(x, x_dtype == ZPP_FP32, numel, log2_of(block), bits, codes, scales,
                   static_cast<hipStream_t>(stream));
    });
}

zpp_status zpp_quantize_reordered(const void *x, int32_t x_dtype, int64_t slice_elems, int32_t n_nodes,
                                  int32_t gpus_per_node, int32_t first_slice, int32_t n_slices, int32_t block,
                                  int32_t bits, void *codes, float *scales, void *stream) {
    if (x_dtype != ZPP_BF16 && x_dtype != ZPP_FP32) return ZPP_ERR_ARG;
    if (bits != 8 && bits != 4) return ZPP_ERR_ARG;
    if (n_nodes < 1 || gpus_per_node < 1) return ZPP_ERR_ARG;
    const int64_t n = static_cast<int64_t>(n_nodes) * gpus_per_node;
    if (n > 65535) return ZPP_ERR_ARG;
    if (!is_pow2_block(block) || slice_elems < 0 || slice_elems % block != 0) return ZPP_ERR_ARG;
    if (first_slice < 0 || n_slices < 0 || first_slice + static_cast<int64_t>(n_slices) > n) return ZPP_ERR_ARG;
    if (slice_elems > ZPP_MAX_NUMEL / n) return ZPP_ERR_ARG;
    if (slice_elems == 0 || n_slices == 0) return ZPP_OK;
    if (!x || !codes || !scales) return ZPP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return ZPP_ERR_ALIGN;
    const int64_t out_elems = slice_elems * n_slices;
    const Range in{x, n * slice_elems * (x_dtype == ZPP_BF16 ? 2 : 4)}, oc{codes, code_bytes(out_elems, bits)},
        os{scales, 4 * (out_elems / block)};
    if (overlap(oc, in) || overlap(os, in) || overlap(oc, os)) return ZPP_ERR_OVERLAP;
    const Range all[] = {in, oc, os};
    if (zpp_status s = check_all(all); s != ZPP_OK) return s;
    return launch_checked([&] {
        return zpp::launch_quantize_reordered(x, x_dtype == ZPP_FP32, slice_elems, n_nodes, gpus_per_node,
                   first_slice, n_slices, log2_of(block), bits, codes, scales, static_cast<hipStream_t>(stream));
    });
}

zpp_status zpp_dequantize_blocks(const void *codes, const float *scales, int32_t bits, int64_t numel, int32_t block,
                                 void *y, int32_t y_dtype, void *stream) {
    if (y_dtype != ZPP_BF16 && y_dtype != ZPP_FP32) return ZPP_ERR_ARG;
    if (bits != 8 && bits != 4) return ZPP_ERR_ARG;
    if (!is_pow2_block(block) || numel < 0 || numel > ZPP_MAX_NUMEL || numel % block != 0) return ZPP_ERR_ARG;
    if (numel == 0) return ZPP_OK;
    if (!codes || !scales || !y) return ZPP_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(y, 16) || !aligned(scales, 4)) return ZPP_ERR_ALIGN;
    const Range ic{codes, code_bytes(numel, bits)}, is{scales, 4 * (numel / block)},
        oy{y, numel * (y_dtype == ZPP_BF16 ? 2 : 4)};
    if (overlap(oy, ic) || overlap(oy, is)) return ZPP_ERR_OVERLAP;
    const Range all[] = {ic, is, oy};
    if (zpp_status s = check_all(all); s != ZPP_OK) return s;
    return launch_checked([&] {
        return zpp::launch_dequantize(codes, scales, bits, numel, log2_of(block), y, y_dtype == ZPP_FP32,
                   static_cast<hipStream_t>(stream));
    });
}

zpp_status zpp_reorder_slices(const void *in, void *out, int64_t slice_bytes, int32_t n_nodes,
                              int32_t gpus_per_node, void *stream) {
    if (n_nodes < 1 || gpus_per_node < 1 || slice_bytes < 0) return ZPP_ERR_ARG;
    if (static_cast<int64_t>(n_nodes) * gpus_per_node > 65535) return ZPP_ERR_ARG;
    const int64_t n = static_cast<int64_t>(n_nodes) * gpus_per_node;
    if (slice_bytes > 4 * ZPP_MAX_NUMEL / n) return ZPP_ERR_ARG;
    if (slice_bytes == 0) return ZPP_OK;
    if (!in || !out) return ZPP_ERR_NULL;
    const Range ri{in, slice_bytes * n}, ro{out, slice_bytes * n};
    if (overlap(ri, ro)) return ZPP_ERR_OVERLAP;
    const Range all[] = {ri, ro};
    if (zpp_status s = check_all(all); s != ZPP_OK) return s;
    return launch_checked([&] {
        return zpp::launch_reorder(in, out, slice_bytes, n_nodes, gpus_per_node, static_cast<hipStream_t>(stream));
    });
}

zpp_status zpp_dequant_reduce_requant(const void *codes_in, int64_t codes_stride_bytes, const float *scales_in,
                                      int64_t scales_stride, int32_t n_inputs, int32_t bits_in, int64_t numel,
                                      int32_t block, void *codes_out, float *scales_out, int32_t bits_out,
                                      float *sum_out, void *stream) {
    if (bits_in != 8 && bits_in != 4) return ZPP_ERR_ARG;
    if (bits_out != 0 && bits_out != 8 && bits_out != 4) return ZPP_ERR_ARG;
    if (!is_pow2_block(block) || numel < 0 || numel > ZPP_MAX_NUMEL || numel % block != 0) return ZPP_ERR_ARG;
    if (n_inputs < 1 || n_inputs > ZPP_MAX_INPUTS) return ZPP_ERR_ARG;
    if (codes_stride_bytes < 0 || codes_stride_bytes > ZPP_MAX_NUMEL) return ZPP_ERR_ARG;
    if (scales_stride < 0 || scales_stride > ZPP_MAX_NUMEL) return ZPP_ERR_ARG;
    if (bits_out == 0 && (codes_out || scales_out)) return ZPP_ERR_ARG;
    if (bits_out == 0 && !sum_out) return ZPP_ERR_ARG;
    if (numel == 0) return ZPP_OK;
    if (!codes_in || !scales_in) return ZPP_ERR_NULL;
    if (bits_out != 0 && (!codes_out || !scales_out)) return ZPP_ERR_NULL;
    if (!aligned(codes_in, 16) || (codes_stride_bytes & 15) != 0 || !aligned(scales_in, 4)) return ZPP_ERR_ALIGN;
    if (codes_out && !aligned(codes_out, 16)) return ZPP_ERR_ALIGN;
    if (scales_out && !aligned(scales_out, 4)) return ZPP_ERR_ALIGN;
    if (sum_out && !aligned(sum_out, 16)) return ZPP_ERR_ALIGN;
    const int64_t nblk = numel / block;
    const Range ic{codes_in, (n_inputs - 1) * codes_stride_bytes + code_bytes(numel, bits_in)},
        is{scales_in, 4 * ((n_inputs - 1) * scales_stride + nblk)},
        oc{codes_out, bits_out ? code_bytes(numel, bits_out) : 0}, os{scales_out, bits_out ? 4 * nblk : 0},
        ou{sum_out, sum_out ? 4 * numel : 0};
    const Range outs[] = {oc, os, ou};
    for (const Range &o : outs) {
        if (overlap(o, ic) || overlap(o, is)) return ZPP_ERR_OVERLAP;
    }
    if (overlap(oc, os) || overlap(oc, ou) || overlap(os, ou)) return ZPP_ERR_OVERLAP;
    const Range all[] = {ic, is, oc, os, ou};
    if (zpp_status s = check_all(all); s != ZPP_OK) return s;
    return launch_checked([&] {
        return zpp::launch_drr(codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs, bits_in, numel,
                   log2_of(block), codes_out, scales_out, bits_out, sum_out, static_cast<hipStream_t>(stream));
    });
}

zpp_status zpp_dequant_reduce_requant_split(const void *codes_in, int64_t codes_stride_bytes, const float *scales_in,
                                            int64_t scales_stride, int32_t n_inputs, int32_t bits_in, int64_t numel,
                                            int32_t block, int64_t keep_begin, int64_t keep_elems, void *codes_send,
                                            float *scales_send, void *codes_keep, float *scales_keep,
                                            int32_t bits_out, void *stream) {
    if (bits_in != 8 && bits_in != 4) return ZPP_ERR_ARG;
    if (bits_out != 8 && bits_out != 4) return ZPP_ERR_ARG;
    if (!is_pow2_block(block) || numel < 0 || numel > ZPP_MAX_NUMEL || numel % block != 0) return ZPP_ERR_ARG;
    if (n_inputs < 1 || n_inputs > ZPP_MAX_INPUTS) return ZPP_ERR_ARG;
    if (codes_stride_bytes < 0 || codes_stride_bytes > ZPP_MAX_NUMEL) return ZPP_ERR_ARG;
    if (scales_stride < 0 || scales_stride > ZPP_MAX_NUMEL) return ZPP_ERR_ARG;
    if (keep_begin < 0 || keep_elems < 0 || keep_begin > numel || keep_elems > numel - keep_begin) return ZPP_ERR_ARG;
    if (keep_begin % block != 0 || keep_elems % block != 0) return ZPP_ERR_ARG;
    if (numel == 0) return ZPP_OK;
    const int64_t send_elems = numel - keep_elems;
    if (!codes_in || !scales_in) return ZPP_ERR_NULL;
    if (send_elems > 0 && (!codes_send || !scales_send)) return ZPP_ERR_NULL;
    if (keep_elems > 0 && (!codes_keep || !scales_keep)) return ZPP_ERR_NULL;
    if (!aligned(codes_in, 16) || (codes_stride_bytes & 15) != 0 || !aligned(scales_in, 4)) return ZPP_ERR_ALIGN;
    if (send_elems > 0 && (!aligned(codes_send, 16) || !aligned(scales_send, 4))) return ZPP_ERR_ALIGN;
    if (keep_elems > 0 && (!aligned(codes_keep, 16) || !aligned(scales_keep, 4))) return ZPP_ERR_ALIGN;
    const int64_t nblk = numel / block;
    const Range ic{codes_in, (n_inputs - 1) * codes_stride_bytes + code_bytes(numel, bits_in)},
        is{scales_in, 4 * ((n_inputs - 1) * scales_stride + nblk)},
        oc{codes_send, code_bytes(send_elems, bits_out)}, os{scales_send, 4 * (send_elems / block)},
        kc{codes_keep, code_bytes(keep_elems, bits_out)}, ks{scales_keep, 4 * (keep_elems / block)};
    const Range outs[] = {oc, os, kc, ks};
    for (const Range &o : outs) {
        if (overlap(o, ic) || overlap(o, is)) return ZPP_ERR_OVERLAP;
    }
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return ZPP_ERR_OVERLAP;
    const Range all[] = {ic, is, oc, os, kc, ks};
    if (zpp_status s = check_all(all); s != ZPP_OK) return s;
    return launch_checked([&] {
        return zpp::launch_drr_split(codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs, bits_in, numel,
                   log2_of(block), keep_begin, keep_elems, send_elems > 0 ? codes_send : nullptr,
                   send_elems > 0 ? scales_send : nullptr, keep_elems > 0 ? codes_keep : nullptr,
                   keep_elems > 0 ? scales_keep : nullptr, bits_out, static_cast<hipStream_t>(stream));
    });
}

zpp_status zpp_dequant_reduce_average(const void *codes_in, int64_t codes_stride_bytes, const float *scales_in,
                                      int64_t scales_stride, int32_t n_inputs, int32_t bits_in, int64_t numel,
                                      int32_t block, int32_t divisor, float *avg_out, void *stream) {
    if (bits_in != 8 && bits_in != 4) return ZPP_ERR_ARG;
    if (!is_pow2_block(block) || numel < 0 || numel > ZPP_MAX_NUMEL || numel % block != 0) return ZPP_ERR_ARG;
    if (n_inputs < 1 || n_inputs > ZPP_MAX_INPUTS) return ZPP_ERR_ARG;
    if (codes_stride_bytes < 0 || codes_stride_bytes > ZPP_MAX_NUMEL) return ZPP_ERR_ARG;
    if (scales_stride < 0 || scales_stride > ZPP_MAX_NUMEL) return ZPP_ERR_ARG;
    if (divisor < 1 || divisor > ZPP_MAX_DIVISOR) return ZPP_ERR_ARG;
    if (numel == 0) return ZPP_OK;
    if (!codes_in || !scales_in || !avg_out) return ZPP_ERR_NULL;
    if (!aligned(codes_in, 16) || (codes_stride_bytes & 15) != 0 || !aligned(scales_in, 4)) return ZPP_ERR_ALIGN;
    if (!aligned(avg_out, 16)) return ZPP_ERR_ALIGN;
    const int64_t nblk = numel / block;
    const Range ic{codes_in, (n_inputs - 1) * codes_stride_bytes + code_bytes(numel, bits_in)},
        is{scales_in, 4 * ((n_inputs - 1) * scales_stride + nblk)}, ou{avg_out, 4 * numel};
    if (overlap(ou, ic) || overlap(ou, is)) return ZPP_ERR_OVERLAP;
    const Range all[] = {ic, is, ou};
    if (zpp_status s = check_all(all); s != ZPP_OK) return s;
    return launch_checked([&] {
        return zpp::launch_drr_average(codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs, bits_in,
                   numel, log2_of(block), divisor, avg_out, static_cast<hipStream_t>(stream));
    });
}

int32_t zpp_set_pointer_checks(int32_t enabled) {
    return g_pointer_checks.exchange(enabled != 0 ? 1 : 0, std::memory_order_relaxed);
}

const char *zpp_status_string(int32_t status) {
    switch (status) {
    case ZPP_OK: return "ZPP_OK";
    case ZPP_ERR_NULL: return "ZPP_ERR_NULL: a required pointer is NULL";
    case ZPP_ERR_ARG: return "ZPP_ERR_ARG: invalid size, block, bit width, count, stride or buffer range";
    case ZPP_ERR_ALIGN: return "ZPP_ERR_ALIGN: pointer or stride misaligned";
    case ZPP_ERR_UNSUPPORTED: return "ZPP_ERR_UNSUPPORTED: combination not implemented";
    case ZPP_ERR_OVERLAP: return "ZPP_ERR_OVERLAP: an output overlaps an input or another output";
    case ZPP_ERR_POINTER: return "ZPP_ERR_POINTER: pointer is not GPU-addressable memory";
    case ZPP_ERR_LAUNCH: return "ZPP_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
    }
    return "unknown zpp_status";
}

int32_t zpp_abi_version(void) { return ZPP_ABI_VERSION; }

}  // extern "C"
