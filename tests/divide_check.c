/*
 * Exhaustive check of the quantiser's division shortcut (host C, FMA in
 * hardware or libm, both correctly rounded in binary32).
 *
 * The quantisers compute t = x / s (TeleFuser "Quantization", "Scaled FP8
 * checkpoints: W8A8": q = cast(clamp(x / s)); "Core ideas": q = round(x / s)
 * for INT8) as one Newton (Markstein) correction of the product with the
 * correctly rounded reciprocal:
 *
 *     r = RN(1 / s);  q0 = RN(x r);  e = RN(q0 s - x) (one fused multiply-add);
 *     q = RN(q0 - e r) (one fused multiply-add)
 *
 * (the remainder is negated against the textbook form so that no step loses
 * the sign of a zero x; the kernel applies no separate sign fix-up)
 *
 * and use it only for 2^-90 <= s <= 2^126 (or s == 0); other scales take a
 * true division.  This program walks every positive finite BF16 amax, forms
 * s = RN(amax / qmax) in binary32, and for every BF16 x with |x| <= amax (both
 * signs) compares q with RN(x / s):
 *
 *   - where |RN(x / s)| >= 2^-12 the two must be the same binary32 value;
 *   - below that both must be smaller than 2^-10 in magnitude, so both encode
 *     to a signed zero (E4M3FN's smallest step is 2^-9 and a quotient at or
 *     below half of it rounds to zero; INT8 rounds anything below 1/2 to 0),
 *     and carry the sign of x (zeros included);
 *   - no |q| exceeds that of x = amax: the kernel skips the clamp to +-qmax
 *     for a row whose amax quotient is <= qmax.
 *
 * It also reports, per qmax, how many scales fall outside the fast-path
 * window (those rows divide for real) and checks the window's edges: at the
 * binary32 scales nearest 2^-90 and 2^126 (inside) the shortcut must still
 * agree with the quotient for x over the BF16 grid.
 *
 * Usage: divide_check QMAX [QMAX ...]   (prints one line per qmax, exit 0 if
 * every comparison holds, 1 otherwise)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t u_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* the kernel's formula, scale s >= 2^-90 and <= 2^126, x of either sign */
static float markstein(float x, float s, float r)
{
    const float q0 = x * r;
    /* (the volatile copy keeps the compiler from folding the negation of e
     * into the first fused multiply-add: -RN(a b - c) and RN(c - a b) differ
     * in the sign of an exact zero, which is the point of this form) */
    volatile float ev = fmaf(q0, s, -x);
    const float e = ev;
    return fmaf(-e, r, q0);
}

/* every pair (x, s) with x a BF16 value of magnitude <= amax_bits; returns
 * the number of mismatches and adds to *tested */
static long check_scale(uint32_t amax_bits, float s, long* tested)
{
    const float r = 1.0f / s;
    const float top = fabsf(markstein(f_of(amax_bits << 16), s, r));
    long bad = 0;
    for (uint32_t xb = 0; xb <= amax_bits; ++xb) {
        for (int sg = 0; sg < 2; ++sg) {
            const float x = f_of(((uint32_t)xb << 16) | ((uint32_t)sg << 31));
            const float ref = x / s;
            const float got = markstein(x, s, r);
            if (fabsf(ref) >= 0x1p-12f) {
                if (u_of(got) != u_of(ref)) ++bad;
            } else {
                if (!(fabsf(got) < 0x1p-10f) || signbit(got) != signbit(x)) ++bad;
            }
            if (fabsf(got) > top) ++bad;
        }
    }
    *tested += 2 * (long)(amax_bits + 1);
    return bad;
}

int main(int argc, char** argv)
{
    if (argc < 2) {
        fprintf(stderr, "usage: %s QMAX [QMAX ...]\n", argv[0]);
        return 2;
    }
    int fail = 0;
    for (int a = 1; a < argc; ++a) {
        const float qmax = strtof(argv[a], NULL);
        long tested = 0, bad = 0, slow = 0;
        /* every positive finite BF16 amax: exponent fields 0..254, any mantissa */
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : tested, bad, slow)
        for (int32_t ab = 1; ab < 0x7F80; ++ab) {
            const float amax = f_of((uint32_t)ab << 16);
            const float s = amax / qmax;
            if (!(s >= 0x1p-90f && s <= 0x1p126f)) {
                ++slow; /* the kernel divides for real */
                continue;
            }
            long t = 0;
            bad += check_scale((uint32_t)ab, s, &t);
            tested += t;
        }
        /* the window's edges: the largest binary32 scale below 2^126 and the
         * smallest at or above 2^-90, with every BF16 x up to qmax * s */
        const float edges[2] = {0x1p126f, 0x1p-90f};
        for (int e = 0; e < 2; ++e) {
            const float s = edges[e];
            long t = 0;
            /* x up to the largest BF16 value <= qmax * s (finite) */
            float xmax = qmax * s;
            if (!(xmax <= 0x1.fep127f)) xmax = 0x1.fep127f;
            const uint32_t xb = u_of(xmax) >> 16;
            bad += check_scale(xb, s, &t);
            tested += t;
        }
        printf("qmax %g: %ld pairs tested, %ld mismatches, %ld amax values outside the "
               "fast-path window\n",
               (double)qmax, tested, bad, slow);
        if (bad) fail = 1;
    }
    return fail;
}
