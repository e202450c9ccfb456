/*
 * Exhaustive check of the quotient the quantize kernel forms.
 *
 * The coding rules divide a weight by the stored scale in IEEE binary32
 * ("Loading a model in 4-bit", "Block-wise quantisation, stated exactly":
 * each weight is coded after dividing by the block's absmax).  The kernel
 * forms w / s as one correctly rounded reciprocal r = RN(1 / s) per group and
 * Markstein's correction per weight:
 *     q0 = RN(w * r);  e = fma(-q0, s, w);  q = fma(e, r, q0).
 * Both operands are always fp16 values widened to binary32 (weights, and the
 * absmax or the fp16 scale), so this program compares q with the IEEE
 * quotient w / s for every finite fp16 dividend w and every positive finite
 * fp16 divisor s, and prints the number of pairs and of mismatches.  With
 * the argument "uncorrected" it compares q0 instead (the product by the
 * reciprocal alone), which must disagree somewhere: a check that the sweep
 * can see a wrong quotient.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off (no fast-math; x86 SSE arithmetic
 * is IEEE binary32 with subnormals, as the kernel's).
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

int main(int argc, char **argv)
{
    const int uncorrected = argc > 1 && argv[1][0] == 'u';
    static float dividends[65536];
    int nd = 0;
    for (uint32_t h = 0; h < 65536; ++h)
        if (((h >> 10) & 0x1f) != 0x1f)
            dividends[nd++] = f16_to_f32((uint16_t)h);
    unsigned long long pairs = 0, bad = 0;
    for (uint32_t hs = 1; hs < 0x7c00; ++hs) {
        const float s = f16_to_f32((uint16_t)hs);
        const float r = 1.0f / s;
        unsigned long long bad_s = 0;
        for (int i = 0; i < nd; ++i) {
            const float w = dividends[i];
            const float q0 = w * r;
            const float e = fmaf(-q0, s, w);
            const float q = uncorrected ? q0 : fmaf(e, r, q0);
            const float ref = w / s;
            bad_s += q != ref;
        }
        if (bad_s && bad < 10)
            printf("mismatch for divisor %#06x\n", hs);
        bad += bad_s;
        pairs += (unsigned long long)nd;
    }
    printf("pairs=%llu mismatches=%llu\n", pairs, bad);
    return bad != 0;
}
