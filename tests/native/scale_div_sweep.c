/*
 * Exhaustive check of the scale quotients the quantize kernel forms.
 *
 * The stored scales are binary32 quotients rounded to fp16: INT4-sym
 * s = fp16(a / 7) with a = max |w| ("What is 4-bit quantization and why does
 * it matter?", "How 4-bit quantization works": the scale is the absmax over
 * 7), INT4-asym s = fp16((hi - lo) / 15) with hi = max(0, max w) and
 * lo = min(0, min w) ("INT4", "How it works" / "Components": the range over
 * the 15 steps of the 16 levels).  The divisors are constants, so the kernel
 * forms each quotient with Markstein's correction around the constant
 * reciprocal r = RN(1 / b):
 *     q0 = RN(x * r);  e = fma(-q0, b, x);  q = fma(e, r, q0).
 * This program compares q with the IEEE quotient x / b over every value x
 * can take: a = every non-negative finite fp16 (b = 7), and hi - lo rounded
 * to binary32 for every non-negative finite fp16 hi and every non-positive
 * finite fp16 lo (b = 15).
 *
 * The per-group reciprocal RN(1 / s) (s the stored fp16 scale or the fp16
 * absmax, positive) is formed from the hardware reciprocal r0, accurate to
 * 1 ulp, and one Newton step:
 *     e = fma(-r0, s, 1);  r = fma(e, r0, r0).
 * The program checks r == 1 / s (IEEE) for every positive finite fp16 s and
 * every r0 within 2 ulps of RN(1 / s).
 *
 * It prints the number of cases and of mismatches for each check.  With the
 * argument "uncorrected" it compares q0 (and r0) instead, which must
 * disagree somewhere.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

static float f16_to_f32(uint16_t h)
{
    const int ex = (h >> 10) & 0x1f, man = h & 0x3ff;
    float v = ex == 0 ? ldexpf((float)man, -24) : ldexpf((float)(1024 + man), ex - 25);
    return (h & 0x8000) ? -v : v;
}

static int uncorrected;

static int same(float x, float b, float r)
{
    const float q0 = x * r;
    const float e = fmaf(-q0, b, x);
    const float q = uncorrected ? q0 : fmaf(e, r, q0);
    return q == x / b;
}

int main(int argc, char **argv)
{
    uncorrected = argc > 1 && argv[1][0] == 'u';
    static float mag[31744];
    for (uint32_t h = 0; h < 0x7c00; ++h)
        mag[h] = f16_to_f32((uint16_t)h);
    const float r7 = 1.0f / 7.0f, r15 = 1.0f / 15.0f;
    unsigned long long n7 = 0, bad7 = 0, n15 = 0, bad15 = 0;
    for (int i = 0; i < 31744; ++i) {
        bad7 += !same(mag[i], 7.0f, r7);
        ++n7;
    }
    for (int i = 0; i < 31744; ++i) {
        const float hi = mag[i];
        unsigned long long b = 0;
        for (int j = 0; j < 31744; ++j) {
            const float d = hi - (-mag[j]);
            b += !same(d, 15.0f, r15);
        }
        n15 += 31744;
        bad15 += b;
    }
    unsigned long long nr = 0, badr = 0;
    for (uint32_t h = 1; h < 0x7c00; ++h) {
        const float sv = mag[h];
        const float ref = 1.0f / sv;
        const float lo1 = nextafterf(ref, 0.0f), hi1 = nextafterf(ref, INFINITY);
        const float cand[5] = {nextafterf(lo1, 0.0f), lo1, ref, hi1, nextafterf(hi1, INFINITY)};
        for (int k = 0; k < 5; ++k) {
            const float r0 = cand[k];
            const float e = fmaf(-r0, sv, 1.0f);
            const float r = uncorrected ? r0 : fmaf(e, r0, r0);
            badr += r != ref;
            ++nr;
        }
    }
    printf("div7 operands=%llu mismatches=%llu\n", n7, bad7);
    printf("div15 operands=%llu mismatches=%llu\n", n15, bad15);
    printf("rcp cases=%llu mismatches=%llu\n", nr, badr);
    return (bad7 | bad15 | badr) != 0;
}
