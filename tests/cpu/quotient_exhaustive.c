/* Exhaustive CPU proof that the quantizer kernels' element quotient equals
 * one IEEE binary32 division, as far as the resulting E4M3 byte goes.
 *
 * The kernels never divide per element. Per group they form the scale
 * s = fl32(amax / 448) and its correctly rounded reciprocal r = fl32(1 / s),
 * then per element
 *     q0 = fl32(x * r);  d = fma(q0, s, -x);  q = fma(-d, r, q0)
 * (Markstein's correction step; Muller et al., Handbook of Floating-Point
 * Arithmetic, section on division by Newton-Raphson iteration; d is the exact
 * residual with its sign flipped so that x = -0 gives q = -0). When amax is
 * below 2^-64 (so s may be subnormal and 1/s may overflow) both x and s are
 * first multiplied by 2^64, which is exact and leaves the real quotient
 * unchanged.
 *
 * The quantizer inputs are bf16, so every (x, amax) pair with |x| <= amax can
 * be enumerated: about 1.07e9 pairs with both signs of x. For each pair the
 * signed E4M3 byte of q must equal the byte of fl32(x / s), and the float32
 * bits must agree whenever |x / s| >= 2^-11 (below that both encode to a
 * signed zero). It also records the largest |q|, which must stay below 449:
 * the kernels hand q to the hardware E4M3 converter without clamping it to
 * +-448, and the converter matches clamp-then-convert for every |v| < 449.
 * Prints counts and exits non-zero on any mismatch or a larger |q|.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off -fopenmp quotient_exhaustive.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E4M3 (OCP, finite-only) byte of a float with |v| <= 464, nearest, ties to even, sign kept. */
static uint8_t enc(float v) {
    uint8_t sign = (bits(v) >> 31) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a < 0.015625f)                          /* below 2^-6: grid k * 2^-9 */
        return sign | (uint8_t)nearbyintf(a * 512.0f);   /* exact scaling; default rounding is RNE */
    uint32_t u = bits(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);           /* round the mantissa to 3 bits, ties to even */
    int e = (int)((u >> 23) & 0xFF) - 127;
    uint32_t m = (u >> 20) & 7u;
    return sign | (uint8_t)(((e + 7) << 3) | m);
}

int main(void) {
    long long pairs = 0, byte_bad = 0, f32_bad = 0;
    float maxq = 0.0f;
    const float two64 = 18446744073709551616.0f;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, byte_bad, f32_bad) reduction(max : maxq)
    for (uint32_t ab = 1; ab < 0x7F80u; ++ab) {
        float amax = bf16(ab);
        float s = amax / 448.0f;
        int tiny = amax < 5.421010862427522e-20f;   /* 2^-64 */
        float sc = tiny ? s * two64 : s;
        float r = 1.0f / sc;
        for (uint32_t mag = 0; mag <= ab; ++mag) {
            for (uint32_t sgn = 0; sgn < 2; ++sgn) {
                float x = bf16(mag | (sgn << 15));
                float xe = tiny ? x * two64 : x;
                float q0 = xe * r;
                float d = fmaf(q0, sc, -xe);
                /* Opaque to the optimizer: gcc -O2 otherwise rewrites
                   fma(-fma(a, b, -c), r, q0) as fma(fma(-a, b, c), r, q0),
                   which differs exactly in the sign of a zero result. */
                __asm__("" : "+x"(d));
                float q = fmaf(-d, r, q0);
                float ref = x / s;
                ++pairs;
                if (fabsf(q) > maxq) maxq = fabsf(q);
                if (enc(q) != enc(ref)) ++byte_bad;
                if (fabsf(ref) >= 0.00048828125f && bits(q) != bits(ref)) ++f32_bad;
            }
        }
    }
    printf("pairs=%lld byte_mismatch=%lld f32_mismatch=%lld max_abs_q=%.9g\n", pairs, byte_bad, f32_bad,
           (double)maxq);
    return (byte_bad || f32_bad || !(maxq < 449.0f)) ? 1 : 0;
}
