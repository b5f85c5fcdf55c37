/*
 * Exhaustive check of the identity the int8 quantiser's fast path relies on.
 *
 * Per-token dynamic quantisation (aclnnMoeDistributeDispatchV4, quantMode 2,
 * read as q = rint(x / scale), scale = amax / 127) needs the correctly rounded
 * fp32 quotient. The kernel replaces the division by one correction step:
 *     inv = RN(1 / scale), q0 = RN(x * inv), r = fma(-q0, scale, x),
 *     q = RN(fma(r, inv, q0))
 * and claims rint(q) == rint(RN(x / scale)) whenever scale >= 2^-100; it also
 * relies on |rint(q)| <= 127 (no clamp) and forms rint(q) as RN(q + 1.5 * 2^23),
 * whose low byte is the two's-complement code. This program checks those claims
 * for every finite 16-bit x (bf16 or fp16) and every positive finite 16-bit amax
 * with |x| <= amax, i.e. for every pair a token row can produce. Prints the
 * counts; exits 1 on any mismatch.
 *
 * With a second argument "e4m3" it checks the per-group FP8 path instead
 * (quantMode 3, read as scale = amax / 448 and code = the E4M3 value nearest
 * to RN(x / scale) clamped to +-448, ties to even, sign of x kept): the same
 * correction step, then an integer rounding of the binary32 bits to 3
 * fraction bits (and a magic add below 2^-6), against the definition (exact
 * division, then rint on the value divided by its E4M3 quantum). The kernel
 * converts with v_cvt_pk_fp8_f32, which was found equal to this integer
 * rounding for every binary32 |v| <= 448 on the GPU.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bf16(uint16_t b) { uint32_t u = (uint32_t)b << 16; float f; memcpy(&f, &u, 4); return f; }

static float from_fp16(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    float v = e == 0 ? ldexpf((float)m, -24) : (e == 31 ? INFINITY : ldexpf((float)(1024 + m), e - 25));
    return s ? -v : v;
}

/* Nearest E4M3 value of |v| <= 448, ties to even, from the definition: the
 * quantum is 2^-9 below 2^-6 and 2^(E-3) in [2^E, 2^(E+1)). */
static uint8_t e4m3_def(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    float a = fabsf(v);
    if (a == 0.0f) return sign;
    if (a < 0x1p-6f) return sign | (uint8_t)rintf(a * 512.0f);
    int e2;
    frexpf(a, &e2);
    int E = e2 - 1;
    float n = rintf(ldexpf(a, 3 - E));
    if (n == 16.0f) { n = 8.0f; E += 1; }
    return sign | (uint8_t)((E + 7) << 3) | (uint8_t)((int)n - 8);
}

/* E4M3 code of 0 <= a <= 448 by integer rounding: round the binary32 fraction to
 * 3 bits at bit 20 (ties to even, carry into the exponent), rebias 127 -> 7;
 * below 2^-6 the subnormal code is RN(a * 512) read from a magic add. */
static uint8_t e4m3_kernel(float a)
{
    uint32_t b;
    memcpy(&b, &a, 4);
    if (b < 0x3c800000u) {
        const float m = a * 512.0f + 0x1.8p23f;
        uint32_t mb;
        memcpy(&mb, &m, 4);
        return (uint8_t)(mb & 0xf);
    }
    const uint32_t r = (b + 0x7ffffu + ((b >> 20) & 1u)) >> 20;
    return (uint8_t)(r - (120u << 3));
}

static int check_e4m3(int bf)
{
    long long pairs = 0, code_bad = 0, quot_bad = 0, slow_scales = 0;
#pragma omp parallel for reduction(+ : pairs, code_bad, quot_bad, slow_scales) schedule(dynamic, 64)
    for (int a = 1; a < 0x8000; ++a) {
        const float amax = bf ? from_bf16((uint16_t)a) : from_fp16((uint16_t)a);
        if (!isfinite(amax) || amax <= 0.0f) continue;
        const float scale = amax / 448.0f;
        if (!(scale >= 0x1p-100f)) { slow_scales++; continue; }
        volatile float one = 1.0f;
        const float inv = one / scale;
        for (int xb = 0; xb < 65536; ++xb) {
            const float x = bf ? from_bf16((uint16_t)xb) : from_fp16((uint16_t)xb);
            if (!isfinite(x) || fabsf(x) > amax) continue;
            const float ax = fabsf(x);
            const float q0 = ax * inv;
            const float r = fmaf(-q0, scale, ax);
            const float q = fmaf(r, inv, q0);
            const uint8_t got = e4m3_kernel(fminf(q, 448.0f)) | (signbit(x) ? 0x80 : 0);
            float d = x / scale;
            d = fminf(fmaxf(d, -448.0f), 448.0f);
            pairs++;
            quot_bad += q != fabsf(x / scale);
            code_bad += got != e4m3_def(d);
        }
    }
    printf("%s-e4m3 pairs=%lld code_mismatches=%lld quotient_mismatches=%lld scales_below_2^-100=%lld\n",
           bf ? "bf16" : "fp16", pairs, code_bad, quot_bad, slow_scales);
    return code_bad != 0;
}

int main(int argc, char **argv)
{
    const int bf = argc > 1 && argv[1][0] == 'b';
    if (argc > 2 && strcmp(argv[2], "e4m3") == 0) return check_e4m3(bf);
    long long pairs = 0, int_bad = 0, quot_bad = 0, slow_scales = 0, range_bad = 0, byte_bad = 0;
#pragma omp parallel for reduction(+ : pairs, int_bad, quot_bad, slow_scales, range_bad, byte_bad) schedule(dynamic, 64)
    for (int a = 1; a < 0x8000; ++a) {
        const float amax = bf ? from_bf16((uint16_t)a) : from_fp16((uint16_t)a);
        if (!isfinite(amax) || amax <= 0.0f) continue;
        const float scale = amax / 127.0f;
        if (!(scale >= 0x1p-100f)) { slow_scales++; continue; }
        volatile float one = 1.0f;
        const float inv = one / scale;
        for (int xb = 0; xb < 65536; ++xb) {
            const float x = bf ? from_bf16((uint16_t)xb) : from_fp16((uint16_t)xb);
            if (!isfinite(x) || fabsf(x) > amax) continue;
            const float q0 = x * inv;
            const float r = fmaf(-q0, scale, x);
            const float q = fmaf(r, inv, q0);
            const float d = x / scale;
            pairs++;
            quot_bad += q != d;
            int_bad += rintf(q) != rintf(d);
            range_bad += fabsf(rintf(d)) > 127.0f;
            const float u = q + 0x1.8p23f;
            uint32_t ub;
            memcpy(&ub, &u, 4);
            byte_bad += (int8_t)(ub & 0xff) != (int8_t)(int)rintf(d);
        }
    }
    printf("%s pairs=%lld integer_mismatches=%lld quotient_mismatches=%lld out_of_range=%lld byte_mismatches=%lld "
           "scales_below_2^-100=%lld\n", bf ? "bf16" : "fp16", pairs, int_bad, quot_bad, range_bad, byte_bad,
           slow_scales);
    return int_bad != 0 || range_bad != 0 || byte_bad != 0;
}
