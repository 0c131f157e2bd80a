/*
 * Check of the arithmetic identity the device quantizer relies on: with
 * r = RN(1/s), q0 = RN(x r), e = RN(x - q0 s) (one rounding, FMA) and
 * q = RN(q0 + e r) (FMA), q equals the correctly rounded quotient RN(x / s).
 * x runs over every significand of a 16-bit input format (bf16: 8 bits,
 * fp16: 11 bits) at two adjacent exponents, s over a slice of the 2^23 fp32
 * significands (the identity only depends on the significands while nothing
 * overflows or underflows).  Prints the number of mismatches.
 *
 * usage: quotient_check <significand bits of x> <first s significand> <count> <step>
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

int main(int argc, char** argv)
{
    if (argc != 5) return 2;
    const int xbits = atoi(argv[1]);
    const uint32_t first = (uint32_t)strtoul(argv[2], NULL, 0);
    const uint32_t count = (uint32_t)strtoul(argv[3], NULL, 0);
    const uint32_t step = (uint32_t)strtoul(argv[4], NULL, 0);
    unsigned long long bad = 0, total = 0;
    for (uint32_t i = 0; i < count; ++i) {
        const uint32_t sm = (first + i * step) & 0x7fffffu;
        const float s = from_bits((127u << 23) | sm);
        const float r = 1.0f / s;
        for (uint32_t xm = 0; xm < (1u << (xbits - 1)); ++xm) {
            for (int xe = -1; xe <= 0; ++xe) {
                const float x = ldexpf(1.0f + (float)xm / (float)(1u << (xbits - 1)), xe);
                const float q0 = x * r;
                const float e = fmaf(-q0, s, x);
                const float q = fmaf(e, r, q0);
                ++total;
                if (q != x / s) ++bad;
            }
        }
    }
    printf("%llu %llu\n", total, bad);
    return 0;
}
