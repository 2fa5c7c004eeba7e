/*
 * div_by_const.c -- checks, for every non-negative finite binary32 value a
 * (+0 through the largest finite float, subnormals included), that
 *   q0 = a * fl(1/d),  e = fma(-q0, d, a),  q1 = fma(e, fl(1/d), q0)
 * equals the IEEE quotient fl(a / d), for the divisor given on the command
 * line.  The requant kernel of the reduce computes its block scale
 * fl(absmax / 7) this way.  Prints the number of mismatches; exit status 0
 * when there are none.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t to_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

int main(int argc, char **argv)
{
    const float d = argc > 1 ? (float)atof(argv[1]) : 7.0f;
    const float r = 1.0f / d;
    unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (long long i = 0; i < 0x7F800000LL; ++i) {
        const float a = from_bits((uint32_t)i);
        const float q0 = a * r;
        const float e = fmaf(-q0, d, a);
        const float q1 = fmaf(e, r, q0);
        if (to_bits(q1) != to_bits(a / d))
            bad++;
    }
    printf("divisor %g: %llu mismatches\n", d, bad);
    return bad != 0;
}
