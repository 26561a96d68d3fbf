/*
 * Exhaustive check of the oracle's float -> fp16 / bf16 conversions over all 2^32 float bit
 * patterns (test infrastructure; links the oracle library, shares none of its code).
 *
 * For every non-NaN input the 16-bit code must be the IEEE-754 round-to-nearest, ties-to-even
 * result, which both bit rules on the page "makarna/pkg/kvcache/paged_cache.go"
 * (float32ToFloat16Bits, float32ToBFloat16Bits) produce for non-NaN inputs. Checked two ways:
 *   1. property: the decoded code lies in the rounding interval around the input, a tie lands
 *      on an even code, the sign is kept, and only inputs at or beyond max + half an ulp map to
 *      infinity (decoding done here with the CPU's F16C instruction for fp16, bits << 16 for
 *      bf16);
 *   2. hardware: x86 F16C vcvtps2ph (fp16, all non-NaN inputs) and AVX512-BF16 vcvtneps2bf16
 *      (bf16, normal inputs only: it flushes subnormals), when the CPU has them.
 * NaN inputs: the code must be a NaN of the same sign whose fraction is the input's leading
 * payload bits (10 for fp16, 7 for bf16), or 1 when those bits are all zero.
 *
 * Output: one line per format, "<fmt> checked=<n> bad_property=<n> bad_hw=<n> hw=<0|1>".
 */
#include <immintrin.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t pkvo_f32_to_f16(float x);
uint16_t pkvo_f32_to_bf16(float x);

__attribute__((target("f16c"))) static double dec_f16_hw(uint16_t c)
{
    return (double)_cvtsh_ss(c);
}

__attribute__((target("f16c"))) static uint16_t enc_f16_hw(float x)
{
    return (uint16_t)_cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT);
}

__attribute__((target("avx512bf16,avx512vl"))) static uint16_t enc_bf16_hw(float x)
{
    __m128 v = _mm_set1_ps(x);
    __m128bh r = _mm_cvtneps_pbh(v);
    uint16_t out[8];
    memcpy(out, &r, 8);
    return out[0];
}

static double dec_bf16(uint16_t c)
{
    uint32_t u = (uint32_t)c << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

typedef struct {
    int frac_bits;            /* 10 or 7 */
    uint16_t inf_code;        /* 0x7C00 or 0x7F80 */
    double (*dec)(uint16_t);  /* exact decode of a magnitude code */
} fmt_t;

/* returns 1 when code c is a valid round-to-nearest-even encoding of the non-NaN float x */
static int property_ok(const fmt_t* f, float x, uint16_t c)
{
    const int xneg = signbit(x) != 0;
    const int cneg = (c & 0x8000u) != 0;
    if (xneg != cneg)
        return 0;
    const double a = fabs((double)x);
    const uint16_t m = c & 0x7FFFu;
    const uint16_t maxc = (uint16_t)(f->inf_code - 1u);
    const double vmax = f->dec(maxc);
    const double threshold = vmax + (vmax - f->dec((uint16_t)(maxc - 1u))) / 2.0;
    if (m == f->inf_code)
        return isinf(x) || a >= threshold;
    if (m > f->inf_code)
        return 0; /* a NaN code for a non-NaN input */
    if (isinf(x))
        return 0;
    const double v = f->dec(m);
    const double lo_mid = (m == 0) ? 0.0 : (v + f->dec((uint16_t)(m - 1u))) / 2.0;
    const double hi_mid = (m == maxc) ? threshold : (v + f->dec((uint16_t)(m + 1u))) / 2.0;
    if (a < lo_mid || a > hi_mid)
        return 0;
    if ((a == lo_mid && m != 0) || a == hi_mid)
        return (m & 1u) == 0;
    return 1;
}

static int nan_ok(const fmt_t* f, uint32_t u, uint16_t c)
{
    const uint16_t sign = (u & 0x80000000u) ? 0x8000u : 0u;
    if ((c & 0x8000u) != sign)
        return 0;
    if ((c & f->inf_code) != f->inf_code)
        return 0;
    const uint32_t lead = (u & 0x007FFFFFu) >> (23 - f->frac_bits);
    const uint32_t frac = c & ((1u << f->frac_bits) - 1u);
    return frac == (lead ? lead : 1u);
}

int main(void)
{
    const int have_f16c = __builtin_cpu_supports("f16c");
    const int have_bf16 = __builtin_cpu_supports("avx512bf16") && __builtin_cpu_supports("avx512vl");
    fmt_t f16 = {10, 0x7C00u, NULL};
    fmt_t b16 = {7, 0x7F80u, dec_bf16};
    if (!have_f16c) {
        printf("f16 skipped=no-f16c\n");
    } else {
        f16.dec = dec_f16_hw;
        long long bad_p = 0, bad_h = 0, n = 0;
#pragma omp parallel for reduction(+ : bad_p, bad_h, n) schedule(static)
        for (int64_t i = 0; i < (1ll << 32); ++i) {
            const uint32_t u = (uint32_t)i;
            float x;
            memcpy(&x, &u, 4);
            const uint16_t c = pkvo_f32_to_f16(x);
            ++n;
            if (isnan(x)) {
                bad_p += !nan_ok(&f16, u, c);
                continue;
            }
            bad_p += !property_ok(&f16, x, c);
            bad_h += enc_f16_hw(x) != c;
        }
        printf("f16 checked=%lld bad_property=%lld bad_hw=%lld hw=1\n", n, bad_p, bad_h);
    }
    {
        long long bad_p = 0, bad_h = 0, n = 0;
#pragma omp parallel for reduction(+ : bad_p, bad_h, n) schedule(static)
        for (int64_t i = 0; i < (1ll << 32); ++i) {
            const uint32_t u = (uint32_t)i;
            float x;
            memcpy(&x, &u, 4);
            const uint16_t c = pkvo_f32_to_bf16(x);
            ++n;
            if (isnan(x)) {
                bad_p += !nan_ok(&b16, u, c);
                continue;
            }
            bad_p += !property_ok(&b16, x, c);
            if (have_bf16 && isnormal(x) && fabsf(x) < 3.0e38f)
                bad_h += enc_bf16_hw(x) != c;
        }
        printf("bf16 checked=%lld bad_property=%lld bad_hw=%lld hw=%d\n", n, bad_p, bad_h,
               have_bf16);
    }
    return 0;
}
