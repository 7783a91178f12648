/* Checks the quotient method the quantising kernels use for scales in
 * [2^-64, 2^64] against the definition, the e4m3 code of the IEEE
 * single-precision quotient x / s:
 *     r = 1/s rounded, c = 440 s rounded, xc = x clamped to [-c, c],
 *     q0 = xc r rounded, t = q0 s - xc (one FMA, exact), q = q0 - t r (one FMA).
 * The clamp keeps the quotient at or below 448, so the conversion that follows
 * needs no clamp of its own: every |x| >= c lies above 432 s, where the code
 * is the one of 448 (0x7E | sign) whatever the exact quotient.
 * Part 1: every bf16 significand of both signs against every fp32 scale
 * significand, the quotient compared bit for bit (the method scales exactly by
 * powers of two while its intermediates stay normal, which the scale range
 * guarantees wherever the code is not 0), plus both zeros.
 * Part 2: every bf16 value with 256 <= |x| < 4096 against every seventh
 * scale significand in [1, 2): the clamp region, compared by code.
 * Part 3: random bf16 values of every exponent and sign (zeros, subnormals
 * and infinities included) against random scales over the whole range,
 * compared by code.  Parts 2 and 3 also require |q| <= 448.
 * Part 4: scales outside [2^-64, 2^64] and negative ones (finite, non-zero,
 * subnormal included) go through the same method after an exact rescaling:
 * |s| = m 2^e with m in [1, 2), x' = ldexp(+-x, -e), quotient x' / m.
 * Random bf16 values against random such scales, compared by code.
 * Prints the number of comparisons and the number of mismatches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

static float method(float x, float s);

/* x / s for any finite non-zero s through the method on [1, 2) */
static float method_scaled(float x, float s)
{
    int e;
    float m = frexpf(fabsf(s), &e) * 2.0f;   /* |s| = m 2^(e-1), m in [1, 2) */
    float xs = ldexpf(s < 0 ? -x : x, 1 - e);
    return method(xs, m);
}

static float method(float x, float s)
{
    volatile float one = 1.0f, k440 = 440.0f;
    float r = one / s, c = k440 * s;
    float xc = fminf(fmaxf(x, -c), c);
    float q0 = xc * r;
    float t = fmaf(q0, s, -xc);
    return fmaf(-t, r, q0);
}

/* e4m3 code of a float: NaN -> 0x7F | sign, |v| >= 448 -> 0x7E | sign,
 * otherwise the nearest code, ties to the even code */
static unsigned enc(float v)
{
    unsigned sign = (bits_of(v) >> 24) & 0x80u;
    double a = fabs((double)v);
    if (isnan(v))
        return 0x7Fu | sign;
    if (a >= 448.0)
        return 0x7Eu | sign;
    if (a < ldexp(1.0, -6))
        return sign | (unsigned)nearbyint(a * 512.0);
    {
        int e;
        double m = frexp(a, &e);          /* a = m 2^e, m in [0.5, 1) */
        double frac = (m * 2.0 - 1.0) * 8.0; /* mantissa in eighths, exact */
        return sign | (unsigned)(((e - 1 + 7) << 3) + (int)nearbyint(frac));
    }
}

static float ieee_div(float x, float s)
{
    volatile float xv = x, sv = s;
    return xv / sv;
}

int main(void)
{
    long long bad = 0, n = 0;
    int64_t sm;
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
    for (sm = 0; sm < (1 << 23); ++sm) {
        float s = f_of(0x3F800000u | (uint32_t)sm);
        int xm, sg;
        for (sg = 0; sg < 2; ++sg)
            for (xm = 0; xm < 128; ++xm) {
                float x = f_of(((uint32_t)sg << 31) | 0x3F800000u | ((uint32_t)xm << 16));
                n++;
                if (bits_of(method(x, s)) != bits_of(ieee_div(x, s)))
                    bad++;
            }
        for (sg = 0; sg < 2; ++sg) {
            float z = f_of((uint32_t)sg << 31);
            n++;
            if (bits_of(method(z, s)) != bits_of(ieee_div(z, s)))
                bad++;
        }
    }
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
    for (sm = 0; sm < (1 << 23); sm += 7) {
        float s = f_of(0x3F800000u | (uint32_t)sm);
        uint32_t xb;
        for (xb = 0x4380u; xb < 0x4580u; ++xb) {   /* |x| in [256, 4096) */
            int sg;
            for (sg = 0; sg < 2; ++sg) {
                float x = f_of(((uint32_t)sg << 31) | (xb << 16)), q = method(x, s);
                n++;
                if (enc(q) != enc(ieee_div(x, s)) || !(fabsf(q) <= 448.0f))
                    bad++;
            }
        }
    }
    {
        uint64_t st = 88172645463325252ull;
        long long it;
        for (it = 0; it < 40000000LL; ++it) {
            uint32_t sb, xb;
            float s, x;
            st ^= st << 13; st ^= st >> 7; st ^= st << 17;
            sb = (uint32_t)((127 - 64 + (st >> 32) % 129) << 23) | (uint32_t)(st & 0x7FFFFF);
            s = f_of(sb);
            if (s > ldexpf(1.0f, 64))
                continue;
            st ^= st << 13; st ^= st >> 7; st ^= st << 17;
            xb = (uint32_t)(st & 0xFFFF) << 16;
            x = f_of(xb);
            if (isnan(x))
                continue;
            n++;
            {
                float q = method(x, s);
                if (enc(q) != enc(ieee_div(x, s)) || !(fabsf(q) <= 448.0f))
                    bad++;
            }
        }
    }
    {
        uint64_t st = 0x9E3779B97F4A7C15ull;
        long long it;
        for (it = 0; it < 40000000LL; ++it) {
            uint32_t sb, xb;
            float s, x, q;
            st ^= st << 13; st ^= st >> 7; st ^= st << 17;
            sb = (uint32_t)(st >> 32);
            s = f_of(sb);
            if (!isfinite(s) || s == 0.0f || (fabsf(s) >= ldexpf(1.0f, -64) && fabsf(s) <= ldexpf(1.0f, 64) && s > 0))
                continue;
            st ^= st << 13; st ^= st >> 7; st ^= st << 17;
            xb = (uint32_t)(st & 0xFFFF) << 16;
            x = f_of(xb);
            if (isnan(x))
                continue;
            n++;
            q = method_scaled(x, s);
            if (enc(q) != enc(ieee_div(x, s)) || !(fabsf(q) <= 448.0f))
                bad++;
        }
    }
    printf("%lld %lld\n", n, bad);
    return 0;
}
