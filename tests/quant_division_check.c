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

int main(int argc, char **argv)
{
    const int bf = argc > 1 && argv[1][0] == 'b';
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
