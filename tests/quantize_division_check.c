/* Checks the quotient method the quantising kernels use for scales in
 * [2^-64, 2^64] against IEEE single-precision division (what the encoding
 * is defined on): r = 1/s rounded, a = min(|x|, 1024 s), q0 = a r rounded,
 * e = a - q0 s (one FMA, exact), q = q0 + e r (one FMA), sign of x copied.
 * Part 1: every bf16 significand against every fp32 scale significand (the
 * method scales exactly by powers of two while its intermediates stay
 * normal, which the scale range guarantees wherever the code is not 0).
 * Part 2: random bf16 values of every exponent and sign against random
 * scales over the whole range, compared where it decides the e4m3 code:
 * exactly for |x/s| >= 2^-12, saturation above 1024, magnitude <= 2^-10
 * and the sign below.  Prints the number of mismatches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

static float method(float x, float s)
{
    volatile float one = 1.0f;
    float r = one / s, a = fminf(fabsf(x), 1024.0f * s);
    float q0 = a * r;
    float e = fmaf(-q0, s, a);
    return copysignf(fmaf(e, r, q0), x);
}

int main(void)
{
    long long bad = 0, n = 0;
    int64_t sm;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (sm = 0; sm < (1 << 23); ++sm) {
        float s = f_of(0x3F800000u | (uint32_t)sm);
        int xm;
        for (xm = 0; xm < 128; ++xm) {
            volatile float x = f_of(0x3F800000u | ((uint32_t)xm << 16)), sv = s;
            if (method(x, s) != x / sv)
                bad++;
        }
    }
    {
        uint64_t st = 88172645463325252ull;
        long long it;
        for (it = 0; it < 40000000LL; ++it) {
            uint32_t sb, xb;
            float s, x, q, want, aw;
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
            {
                volatile float xv = x, sv = s;
                want = xv / sv;
            }
            q = method(x, s);
            aw = fabsf(want);
            n++;
            if (aw >= 1024.0f || isinf(want)) {
                if (!(fabsf(q) >= 448.0f) || signbit(q) != signbit(want)) bad++;
            } else if (aw >= ldexpf(1.0f, -12)) {
                if (q != want) bad++;
            } else if (!(fabsf(q) <= ldexpf(1.0f, -10)) || signbit(q) != signbit(want)) {
                bad++;
            }
        }
    }
    printf("%lld %lld\n", (long long)(1 << 23) * 128 + n, bad);
    return 0;
}
