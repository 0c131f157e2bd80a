/*
 * Checks of the arithmetic the device quantizer relies on to compute
 * fl32(x / s) without a division per element.  With r = RN(1/s),
 * q0 = RN(x r), e = RN(x - q0 s) (one rounding, FMA) and q = RN(q0 + e r)
 * (FMA):
 *
 *   id   q equals the correctly rounded quotient RN(x / s).  x runs over every
 *        significand of a 16-bit input format (bf16: 8 bits, fp16: 11 bits)
 *        at two adjacent exponents, s over a slice of the 2^23 fp32
 *        significands (the identity only depends on the significands while
 *        nothing overflows or underflows).
 *        usage: quotient_check id <significand bits of x> <first s significand> <count> <step>
 *        prints: <cases> <mismatches>
 *
 *   sat  the E4M3 code (OCP E4M3, round to nearest even, saturating at
 *        +-448, infinities included) of the device routine's result equals
 *        the code of the IEEE quotient: every non-NaN bit pattern of a bf16
 *        or fp16 input (infinities included; NaN inputs are outside the
 *        quantizer's contract) against divisors s = 2^E (1 + m 2^-23) for E
 *        in [e_lo, e_hi] and `count` significands m spread by `step`.  The
 *        device routine: q0 = RN(x r) clamped to [-896, 896] (a median of
 *        three), the correction step from the clamped q0, the sign of x put
 *        on the result (which keeps -0), then a clamp to [-448, 448] before
 *        the converter.  (Below 2^-10 every value encodes to a signed zero,
 *        so the routine may differ from the quotient there, where the
 *        residual underflows.)  The same sweep also counts the code
 *        mismatches of the correction step from the unclamped q0, which must
 *        be nonzero wherever the sweep reaches quotients that overflow
 *        binary32 (x r = inf gives x - inf s = -inf, then -inf r + inf).
 *        usage: quotient_check sat <bf16|fp16> <e_lo> <e_hi> <first s significand> <count> <step>
 *        prints: <cases> <mismatches> <mismatches without the guard>
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

/* bf16 / fp16 bit pattern -> binary32 (exact) */
static float bf16_value(uint32_t h) { return from_bits(h << 16); }

static float fp16_value(uint32_t h)
{
    const uint32_t sign = (h >> 15) & 1u, ex = (h >> 10) & 0x1fu, man = h & 0x3ffu;
    float v;
    if (ex == 0) v = ldexpf((float)man, -24);
    else if (ex == 31) v = man ? NAN : INFINITY;
    else v = ldexpf((float)(man | 0x400u), (int)ex - 25);
    return sign ? -v : v;
}

/* OCP E4M3 code of a binary32 value: one rounding to nearest even,
   saturation of |v| >= 448 (infinities included), NaN -> 0x7F | sign,
   subnormals m 2^-9.  Every scaling below is by a power of two (exact), and
   rintf rounds to nearest even in the default rounding mode. */
static unsigned e4m3_code(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    const unsigned sgn = (u >> 31) << 7;
    const float a = fabsf(v);
    if (isnan(v)) return 0x7Fu | sgn;
    if (a >= 448.0f) return 0x7Eu | sgn;
    if (a < 0x1p-6f) return sgn | (unsigned)rintf(a * 512.0f);   /* 8 -> 0x08 = 2^-6 */
    int ex;
    frexpf(a, &ex);                       /* a = f 2^ex, f in [0.5, 1) */
    int e = ex - 1;
    unsigned f = (unsigned)rintf((ldexpf(a, -e) - 1.0f) * 8.0f);
    if (f == 8) {
        ++e;
        f = 0;
    }
    return sgn | (unsigned)((e + 7) << 3) | f;
}

/* v_med3_f32 on non-NaN inputs with lo <= hi */
static float med3(float a, float lo, float hi) { return fminf(fmaxf(a, lo), hi); }

/* the device routine: x / s saturated to [-448, 448], ready for the converter */
static float device_quotient(float x, float s, float r)
{
    const float q0 = med3(x * r, -896.0f, 896.0f);
    const float e = fmaf(-q0, s, x);
    const float q = fmaf(e, r, q0);
    return med3(copysignf(q, x), -448.0f, 448.0f);
}

static int same_code(unsigned a, unsigned b)
{
    if ((a & 0x7fu) == 0x7fu || (b & 0x7fu) == 0x7fu) return (a & 0x7fu) == (b & 0x7fu);
    return a == b;
}

static int run_id(int argc, char** argv)
{
    if (argc != 6) return 2;
    const int xbits = atoi(argv[2]);
    const uint32_t first = (uint32_t)strtoul(argv[3], NULL, 0);
    const uint32_t count = (uint32_t)strtoul(argv[4], NULL, 0);
    const uint32_t step = (uint32_t)strtoul(argv[5], NULL, 0);
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

static int run_sat(int argc, char** argv)
{
    if (argc != 8) return 2;
    const int fp16 = strcmp(argv[2], "fp16") == 0;
    if (!fp16 && strcmp(argv[2], "bf16") != 0) return 2;
    const int e_lo = atoi(argv[3]), e_hi = atoi(argv[4]);
    const uint32_t first = (uint32_t)strtoul(argv[5], NULL, 0);
    const uint32_t count = (uint32_t)strtoul(argv[6], NULL, 0);
    const uint32_t step = (uint32_t)strtoul(argv[7], NULL, 0);
    static float xs[65536];
    for (uint32_t h = 0; h < 65536; ++h) xs[h] = fp16 ? fp16_value(h) : bf16_value(h);
    unsigned long long total = 0, bad = 0, bad_unguarded = 0;
    for (int E = e_lo; E <= e_hi; ++E) {
        for (uint32_t i = 0; i < count; ++i) {
            const uint32_t sm = (first + i * step) & 0x7fffffu;
            const float s = ldexpf(from_bits((127u << 23) | sm), E);
            const float r = 1.0f / s;
            for (uint32_t h = 0; h < 65536; ++h) {
                const float x = xs[h];
                if (isnan(x)) continue;
                const float q0 = x * r;
                const float e = fmaf(-q0, s, x);
                const float unguarded = copysignf(fmaf(e, r, q0), x);
                const float dev = device_quotient(x, s, r);
                const unsigned want = e4m3_code(x / s);
                ++total;
                if (!same_code(e4m3_code(dev), want)) ++bad;
                if (!same_code(e4m3_code(unguarded), want)) ++bad_unguarded;
            }
        }
    }
    printf("%llu %llu %llu\n", total, bad, bad_unguarded);
    return 0;
}

int main(int argc, char** argv)
{
    if (argc < 2) return 2;
    if (strcmp(argv[1], "id") == 0) return run_id(argc, argv);
    if (strcmp(argv[1], "sat") == 0) return run_sat(argc, argv);
    return 2;
}
