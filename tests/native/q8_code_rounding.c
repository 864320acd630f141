/* Exhaustive check of the code rounding in the device int8 activation
 * quantizer (qg_quantize_q8_1 and the fused matvecs).  A block's code is
 * rne(x / d) for a bf16 x and the block's stored fp16 scale d, with
 * |x / d| <= 127.07 (|x| <= amax, d = fp16_rne(amax / 127)).  The device
 * forms it without a division:
 *
 *     r = 4096 * rcp(d)          (rcp within an ulp of 1 / d)
 *     q = rint(rint(x * r) / 4096)
 *
 * This program runs that formula in fp32 for every positive finite fp16 d
 * and every bf16 x (both signs, subnormals included) with |x| <= 128 d, with
 * rcp taken as 1 / d rounded to nearest and as each of its two fp32
 * neighbours, and compares q with rint(x / d) in double (ties to even; a
 * double quotient of these short numbers rounds to a half-integer only when
 * it is one).  Prints the case count and the mismatch count; exit status 1
 * on any mismatch.  Build with -ffp-contract=off so that the fp32 products
 * are rounded one by one, as on the device. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float fp16_to_float(uint16_t h) {
    const int e = (h >> 10) & 31, m = h & 1023;
    return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
}

int main(void) {
    long cases = 0, bad = 0;
#pragma omp parallel for reduction(+ : cases, bad) schedule(dynamic, 64)
    for (int h = 1; h < 0x7c00; ++h) {
        const float d = fp16_to_float((uint16_t)h);
        const float rn = 1.0f / d;
        const float rcps[3] = {rn, nextafterf(rn, 0.0f), nextafterf(rn, INFINITY)};
        for (int b = 0; b < 0x7f80; ++b) {
            const float mag = bf16_to_float((uint16_t)b);
            if ((double)mag > 128.0 * (double)d) break;    /* bf16 bits are ordered by magnitude */
            for (int sign = 0; sign < 2; ++sign) {
                const float x = sign ? -mag : mag;
                const double want = rint((double)x / (double)d);
                for (int i = 0; i < 3; ++i) {
                    const float r = rcps[i] * 4096.0f;
                    const float q = rintf(rintf(x * r) * 0x1p-12f);
                    ++cases;
                    if ((double)q != want) {
                        if (bad < 8) printf("mismatch d=%a x=%a rcp=%a q=%g want=%g\n", d, x, rcps[i], q, want);
                        ++bad;
                    }
                }
            }
        }
    }
    printf("cases %ld mismatches %ld\n", cases, bad);
    return bad != 0;
}
