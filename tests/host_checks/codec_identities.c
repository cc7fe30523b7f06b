/*
 * Arithmetic identities the GPU codec kernels rely on, checked on the host
 * with IEEE binary32 (SSE) and the C library's correctly rounded fmaf.
 *
 *   scale      RN(a / Q) == fma(a, H, RN(a * L)),  H = RN(1/Q), L = RN(1/Q - H),
 *              for every significand of the given binades (Q = 127 and 7).
 *   markstein  y = RN(1/s), q0 = RN(x*y), r = fma(-q0, s, x), q1 = fma(r, y, q0):
 *              rne(q1) == rne(x / s) for s = RN(a/Q) >= 2^-96 and every
 *              finite bfloat16 x with |x| <= a, over bfloat16 absmax values a
 *              taken with the given stride (stride 1: all of them).
 *   ties       the same quotient for x within 3 ulps of (k + 1/2) s, every k,
 *              random normal s >= 2^-96: q1 == x / s bit for bit.
 *   nibble     the 4-bit products of the hop kernels: for every code q in
 *              [-8, 7] and scale s with |s| <= 2^103, with n = q + 8 taken
 *              as the binary16 subnormal n 2^-24 (exact in binary32),
 *              fma(n 2^-24, s 2^24, -8 s) and fma(16 n 2^-24, s 2^20, -8 s)
 *              equal RN(q * s) (bit for bit, except that an exact zero may
 *              differ in sign), over every significand (taken with the
 *              given stride) of binades spread over that range, subnormal
 *              ones included, both signs.
 *   byte       the same for 8-bit codes q in [-128, 127] and |s| <= 2^120:
 *              fma(q + 128, s, -128 s) equals RN(q * s).
 *
 * Usage: codec_identities <scale|markstein|ties|nibble|byte> <param>; exits 1 on any
 * mismatch. This is host-side test code; it does not run on the GPU.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u32(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint64_t xr(void) { rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17; return rs; }

/* is s the correctly rounded a / Q (ties to even)? exact in double */
static int is_rn_quotient(float a, float s, int Q) {
    double err = (double)s * Q - (double)a;
    int e;
    frexpf(s, &e);
    double half_ulp_q = ldexp(1.0, e - 25) * Q;
    if (fabs(err) < half_ulp_q) return 1;
    if (fabs(err) == half_ulp_q) return (u32(s) & 1) == 0;
    return 0;
}

static const int QS[2] = {127, 7};

static long check_scale(int binades) {
    static const uint32_t exps[] = {127, 147, 37, 200, 64};
    long bad = 0;
    for (int qi = 0; qi < 2; ++qi) {
        const int Q = QS[qi];
        const float H = 1.0f / (float)Q;
        const float L = (float)((1.0 / Q) - (double)H);
        for (int b = 0; b < binades && b < 5; ++b)
            for (uint32_t m = 0; m < (1u << 23); ++m) {
                const float a = f32((exps[b] << 23) | m);
                if (!is_rn_quotient(a, fmaf(a, H, a * L), Q)) ++bad;
            }
        printf("scale Q=%d: %d binade(s) of significands, mismatches so far %ld\n", Q, binades, bad);
    }
    return bad;
}

static long check_markstein(int stride) {
    long bad = 0;
    for (int qi = 0; qi < 2; ++qi) {
        const float Q = (float)QS[qi];
        long pairs = 0;
        for (uint32_t ab = 1; ab < 0x7F80; ab += (uint32_t)stride) {
            const float a = f32(ab << 16);
            const float s = a / Q;
            if (s < 0x1p-96f) continue;
            const float y = 1.0f / s;
            for (uint32_t xb = 0; xb <= ab; ++xb)
                for (int sg = 0; sg < 2; ++sg) {
                    const float x = f32((xb << 16) | (sg ? 0x80000000u : 0u));
                    const float q0 = x * y;
                    const float r = fmaf(-q0, s, x);
                    const float q1 = fmaf(r, y, q0);
                    ++pairs;
                    if (rintf(q1) != rintf(x / s)) ++bad;
                }
        }
        printf("markstein Q=%g: %ld bf16 pairs (absmax stride %d), code mismatches so far %ld\n", Q, pairs,
               stride, bad);
    }
    return bad;
}

static long check_ties(long iters) {
    long bad = 0;
    for (int qi = 0; qi < 2; ++qi) {
        const int Qi = QS[qi];
        const float Q = (float)Qi;
        long n = 0;
        for (long it = 0; it < iters; ++it) {
            const uint32_t ea = 31 + (uint32_t)(xr() % 223);
            const float a = f32((ea << 23) | (uint32_t)(xr() & 0x7FFFFF));
            const float s = a / Q;
            if (s < 0x1p-96f) continue;
            const float y = 1.0f / s;
            for (int k = -Qi; k < Qi; ++k) {
                const float xc = ((float)k + 0.5f) * s;
                for (int d = -3; d <= 3; ++d) {
                    const float x = f32(u32(xc) + (uint32_t)d);
                    if (!(fabsf(x) <= a)) continue;
                    const float q0 = x * y, r = fmaf(-q0, s, x), q1 = fmaf(r, y, q0);
                    ++n;
                    if (u32(q1) != u32(x / s)) ++bad;
                }
            }
        }
        printf("ties Q=%d: %ld near-tie values, quotient mismatches so far %ld\n", Qi, n, bad);
    }
    return bad;
}

static long nibble_one(float s) {
    long bad = 0;
    const float m8s = s * -8.0f, s24 = s * 0x1p24f, s20 = s * 0x1p20f;
    for (int q = -8; q <= 7; ++q) {
        const float want = (float)q * s;
        const float a = fmaf(ldexpf((float)(q + 8), -24), s24, m8s);
        const float b = fmaf(ldexpf((float)(16 * (q + 8)), -24), s20, m8s);
        if (want == 0.0f) {
            bad += (a != 0.0f) + (b != 0.0f);
        } else {
            bad += (u32(a) != u32(want)) + (u32(b) != u32(want));
        }
    }
    return bad;
}

static long check_nibble(int stride) {
    static const int binades[] = {-145, -135, -127, -126, -122, -100, -64, -1, 0, 1, 63, 102};
    long bad = 0, n = 0;
    for (unsigned i = 0; i < sizeof binades / sizeof binades[0]; ++i) {
        for (uint32_t m = 0; m < (1u << 23); m += (uint32_t)stride) {
            /* binades below 2^-126 are subnormal: significand m scaled by 2^(b + 23 - 126) */
            const float s = binades[i] < -126 ? f32(m >> (-126 - binades[i]))
                                              : f32(((uint32_t)(127 + binades[i]) << 23) | m);
            bad += nibble_one(s) + nibble_one(-s);
            n += 2;
        }
    }
    const float ends[] = {0.0f, -0.0f, 0x1p103f, -0x1p103f, 0x1p-149f, -0x1p-149f};
    for (unsigned i = 0; i < sizeof ends / sizeof ends[0]; ++i, ++n) bad += nibble_one(ends[i]);
    printf("nibble: %ld scales x 16 codes x 2 forms, mismatches %ld\n", n, bad);
    return bad;
}

static long byte_one(float s) {
    long bad = 0;
    const float mb = s * -128.0f;
    for (int q = -128; q <= 127; ++q) {
        const float want = (float)q * s, got = fmaf((float)(q + 128), s, mb);
        bad += want == 0.0f ? got != 0.0f : u32(got) != u32(want);
    }
    return bad;
}

static long check_byte(int stride) {
    static const int binades[] = {-145, -140, -127, -126, -122, -64, -1, 0, 1, 63, 118, 119};
    long bad = 0, n = 0;
    for (unsigned i = 0; i < sizeof binades / sizeof binades[0]; ++i) {
        for (uint32_t m = 0; m < (1u << 23); m += (uint32_t)stride) {
            /* binades below 2^-126 are subnormal: significand m scaled by 2^(b + 23 - 126) */
            const float s = binades[i] < -126 ? f32(m >> (-126 - binades[i])) : f32(((uint32_t)(127 + binades[i]) << 23) | m);
            bad += byte_one(s) + byte_one(-s);
            n += 2;
        }
    }
    const float ends[] = {0.0f, -0.0f, 0x1p120f, -0x1p120f};
    for (unsigned i = 0; i < sizeof ends / sizeof ends[0]; ++i, ++n) bad += byte_one(ends[i]);
    printf("byte: %ld scales x 256 codes, mismatches %ld\n", n, bad);
    return bad;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <scale|markstein|ties|nibble|byte> <param>\n", argv[0]);
        return 2;
    }
    const long p = atol(argv[2]);
    long bad;
    if (!strcmp(argv[1], "scale")) bad = check_scale((int)p);
    else if (!strcmp(argv[1], "markstein")) bad = check_markstein((int)p);
    else if (!strcmp(argv[1], "ties")) bad = check_ties(p);
    else if (!strcmp(argv[1], "nibble")) bad = check_nibble((int)p);
    else if (!strcmp(argv[1], "byte")) bad = check_byte((int)p);
    else return 2;
    return bad ? 1 : 0;
}
