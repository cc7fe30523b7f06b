/*
 * zpp_client.c - a plain C program using the codec through include/zpp.h.
 *
 * It owns its device memory (hipMalloc) and stream, runs every entry point
 * once on the input it is given, copies the results back and writes them to
 * files for the caller to compare. It also checks that a call with ordinary
 * host memory is refused with ZPP_ERR_POINTER.
 *
 * usage: zpp_client <dir>
 *   <dir>/x.bin       n bf16 values (uint16), n = 8 slices of S elements
 *   <dir>/params.txt  "n S block"
 * writes <dir>/codes8.bin scales8.bin y.bin reordered.bin codes4.bin
 *        scales4.bin fused_codes.bin fused_scales.bin sum.bin hop_codes.bin
 *        hop_scales.bin send_codes.bin send_scales.bin keep_codes.bin
 *        keep_scales.bin avg.bin status.txt
 * The split hop keeps blocks [10, 17) of the S-element output.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zpp.h"

static int fail(const char *what, int code) {
    fprintf(stderr, "zpp_client: %s failed (%d)\n", what, code);
    return 1;
}

#define HIP_OK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) return fail(#x, (int)e_); } while (0)
#define ZPP_OK_(x) do { zpp_status s_ = (x); if (s_ != ZPP_OK) { fprintf(stderr, "%s\n", zpp_status_string(s_)); return fail(#x, (int)s_); } } while (0)

static int save(const char *dir, const char *name, const void *dev, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    void *h = malloc(bytes ? bytes : 1);
    if (!h) return fail("malloc", 0);
    if (hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) { free(h); return fail("hipMemcpy", 0); }
    FILE *f = fopen(path, "wb");
    if (!f) { free(h); return fail("fopen", 0); }
    size_t w = fwrite(h, 1, bytes, f);
    fclose(f);
    free(h);
    return w == bytes ? 0 : fail("fwrite", 0);
}

int main(int argc, char **argv) {
    if (argc != 2) { fprintf(stderr, "usage: zpp_client <dir>\n"); return 2; }
    const char *dir = argv[1];
    char path[4096];
    long long n = 0, S = 0, B = 0;
    snprintf(path, sizeof path, "%s/params.txt", dir);
    FILE *pf = fopen(path, "r");
    if (!pf || fscanf(pf, "%lld %lld %lld", &n, &S, &B) != 3) return fail("params.txt", 0);
    fclose(pf);
    if (n != 8 * S || n % B || S % B) return fail("params", 0);

    uint16_t *xh = (uint16_t *)malloc((size_t)n * 2);
    snprintf(path, sizeof path, "%s/x.bin", dir);
    FILE *xf = fopen(path, "rb");
    if (!xh || !xf || fread(xh, 2, (size_t)n, xf) != (size_t)n) return fail("x.bin", 0);
    fclose(xf);

    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    void *x, *codes8, *y, *reord, *codes4, *hop_codes, *fused_codes, *send_codes, *keep_codes;
    float *scales8, *scales4, *sum, *hop_scales, *avg, *fused_scales, *send_scales, *keep_scales;
    const long long K0 = 10 * B, KL = 7 * B; /* kept window of the split hop */
    if (S < K0 + KL) return fail("params", 0);
    HIP_OK(hipMalloc(&x, (size_t)n * 2));
    HIP_OK(hipMalloc(&codes8, (size_t)n));
    HIP_OK(hipMalloc((void **)&scales8, (size_t)(n / B) * 4));
    HIP_OK(hipMalloc(&y, (size_t)n * 2));
    HIP_OK(hipMalloc(&reord, (size_t)n * 2));
    HIP_OK(hipMalloc(&codes4, (size_t)n / 2));
    HIP_OK(hipMalloc((void **)&scales4, (size_t)(n / B) * 4));
    HIP_OK(hipMalloc((void **)&sum, (size_t)S * 4));
    HIP_OK(hipMalloc(&hop_codes, (size_t)S / 2));
    HIP_OK(hipMalloc((void **)&hop_scales, (size_t)(S / B) * 4));
    HIP_OK(hipMalloc((void **)&avg, (size_t)S * 4));
    HIP_OK(hipMalloc(&fused_codes, (size_t)n / 2));
    HIP_OK(hipMalloc((void **)&fused_scales, (size_t)(n / B) * 4));
    HIP_OK(hipMalloc(&send_codes, (size_t)(S - KL) / 2));
    HIP_OK(hipMalloc((void **)&send_scales, (size_t)((S - KL) / B) * 4));
    HIP_OK(hipMalloc(&keep_codes, (size_t)KL / 2));
    HIP_OK(hipMalloc((void **)&keep_scales, (size_t)(KL / B) * 4));
    HIP_OK(hipMemcpy(x, xh, (size_t)n * 2, hipMemcpyHostToDevice));

    /* qwZ: 8-bit quantize and dequantize back to bf16 */
    ZPP_OK_(zpp_quantize_blocks(x, ZPP_BF16, n, (int32_t)B, 8, codes8, scales8, st));
    ZPP_OK_(zpp_dequantize_blocks(codes8, scales8, 8, n, (int32_t)B, y, ZPP_BF16, st));
    /* qgZ on a 2-node x 4-GPU grid: reorder, 4-bit quantize of the reordered buffer */
    ZPP_OK_(zpp_reorder_slices(x, reord, S * 2, 2, 4, st));
    ZPP_OK_(zpp_quantize_blocks(reord, ZPP_BF16, n, (int32_t)B, 4, codes4, scales4, st));
    /* the same, with the reorder fused into the quantize */
    ZPP_OK_(zpp_quantize_reordered(x, ZPP_BF16, S, 2, 4, 0, 8, (int32_t)B, 4, fused_codes, fused_scales, st));
    /* reduce the 8 quantized slices as 8 inputs: sum, requantized sum, average */
    ZPP_OK_(zpp_dequant_reduce_requant(codes4, S / 2, scales4, S / B, 8, 4, S, (int32_t)B, hop_codes, hop_scales, 4,
                                       sum, st));
    ZPP_OK_(zpp_dequant_reduce_requant_split(codes4, S / 2, scales4, S / B, 8, 4, S, (int32_t)B, K0, KL, send_codes,
                                             send_scales, keep_codes, keep_scales, 4, st));
    ZPP_OK_(zpp_dequant_reduce_average(codes4, S / 2, scales4, S / B, 8, 4, S, (int32_t)B, 8, avg, st));
    HIP_OK(hipStreamSynchronize(st));

    /* ordinary host memory is refused, nothing launched */
    zpp_status bad = zpp_quantize_blocks(xh, ZPP_BF16, n, (int32_t)B, 8, codes8, scales8, st);

    int rc = 0;
    rc |= save(dir, "codes8.bin", codes8, (size_t)n);
    rc |= save(dir, "scales8.bin", scales8, (size_t)(n / B) * 4);
    rc |= save(dir, "y.bin", y, (size_t)n * 2);
    rc |= save(dir, "reordered.bin", reord, (size_t)n * 2);
    rc |= save(dir, "codes4.bin", codes4, (size_t)n / 2);
    rc |= save(dir, "scales4.bin", scales4, (size_t)(n / B) * 4);
    rc |= save(dir, "sum.bin", sum, (size_t)S * 4);
    rc |= save(dir, "hop_codes.bin", hop_codes, (size_t)S / 2);
    rc |= save(dir, "hop_scales.bin", hop_scales, (size_t)(S / B) * 4);
    rc |= save(dir, "avg.bin", avg, (size_t)S * 4);
    rc |= save(dir, "fused_codes.bin", fused_codes, (size_t)n / 2);
    rc |= save(dir, "fused_scales.bin", fused_scales, (size_t)(n / B) * 4);
    rc |= save(dir, "send_codes.bin", send_codes, (size_t)(S - KL) / 2);
    rc |= save(dir, "send_scales.bin", send_scales, (size_t)((S - KL) / B) * 4);
    rc |= save(dir, "keep_codes.bin", keep_codes, (size_t)KL / 2);
    rc |= save(dir, "keep_scales.bin", keep_scales, (size_t)(KL / B) * 4);
    snprintf(path, sizeof path, "%s/status.txt", dir);
    FILE *sf = fopen(path, "w");
    if (!sf) return fail("status.txt", 0);
    fprintf(sf, "host_pointer %d\nabi %d\n", (int)bad, (int)zpp_abi_version());
    fclose(sf);

    hipFree(x); hipFree(codes8); hipFree(scales8); hipFree(y); hipFree(reord); hipFree(codes4);
    hipFree(scales4); hipFree(sum); hipFree(hop_codes); hipFree(hop_scales); hipFree(avg);
    hipFree(fused_codes); hipFree(fused_scales); hipFree(send_codes); hipFree(send_scales);
    hipFree(keep_codes); hipFree(keep_scales);
    hipStreamDestroy(st);
    free(xh);
    return rc;
}
