/*
 * fp16.c -- IEEE 754 binary16 <-> binary64, written out from the format's
 * definition (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits,
 * subnormals with quantum 2^-24).  Test infrastructure only.
 *
 * The pages store block scales and the KV cache as F16 (the write-up's
 * "Overview" lists F16 among the formats; its "Roadmap" names the F16 KV
 * cache); they do not spell out the encoding, which is the IEEE one.
 */
#include "oracle.h"

#include <math.h>

double or_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24    */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Common encoder: rnd is rint (ties to even under the default rounding mode)
 * or ceil (round toward +infinity, used only for v >= 0). */
static uint16_t encode(double v, double (*rnd)(double))
{
    uint16_t sign = 0;
    if (isnan(v))
        return 0x7e00;
    if (signbit(v)) {
        sign = 0x8000;
        v = -v;
    }
    if (isinf(v))
        return sign | 0x7c00;
    if (v < ldexp(1.0, -14)) {
        /* Subnormal range: the value is an integer multiple of 2^-24.  The
         * scaling by 2^24 is exact, so one rounding of the scaled value is the
         * one rounding of the encoding.  1024 lands on the smallest normal,
         * whose bit pattern is also 1024. */
        double q = rnd(ldexp(v, 24));
        return sign | (uint16_t)q;
    }
    int e2;
    frexp(v, &e2);                 /* v = f * 2^e2, f in [0.5, 1)            */
    int E = e2 - 1;                /* v = (1 + frac) * 2^E                   */
    double q = rnd(ldexp(v, 10 - E));   /* significand scaled to [1024, 2048] */
    if (q >= 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;      /* overflow to infinity                   */
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)q - 1024);
}

uint16_t or_f64_to_f16_rne(double v) { return encode(v, rint); }

uint16_t or_f64_to_f16_up(double v)
{
    if (v <= 0.0)
        return 0;                  /* callers only ask for v >= 0            */
    return encode(v, ceil);
}
