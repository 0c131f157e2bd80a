/*
 * fp8q oracle: a plain, slow, obviously-correct CPU model of the FP8 linear
 * layer and of the NestedFP dual-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the package smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or table with the
 * HIP library; the two meet only through the seeded input generator, which
 * holds none of the method's arithmetic.
 *
 * Pages cited (full titles and addresses are listed in the design notes):
 *   [RTX4060]  intelliparadigm.com/article/weixin_29051149/2151670
 *              (7B model on an RTX 4060 with FP8 E4M3)
 *   [C++FP8]   "C++与FP8量化：大模型推理部署的系统级优化实践" (tqpw.cn/news/201730)
 *   [NestedFP] "NestedFP双精度推理框架：LLM部署中的内存与计算优化"
 *              (intelliparadigm.com/article/weixin_42537919/2229392)
 *
 * Every floating-point format below is written from its published bit-level
 * definition: value = (-1)^s * 2^(e-bias) * (1 + m/2^p) for normals and
 * (-1)^s * 2^(1-bias) * (m/2^p) for subnormals.  Rounding to a format is done
 * in double precision by scaling with an exact power of two and calling
 * nearbyint() under the default round-to-nearest-even mode, so the only
 * rounding is the one the definition asks for.
 *
 * Parity status: every function here is pinned by a CPU test against a library
 * routine, a closed form, brute force in exact rational arithmetic or an
 * invariant; none is "parity unpinned".
 */
#include <fenv.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BF16 0
#define ORC_FP16 1

/* ------------------------------------------------------------------------ */
/* Generic helpers                                                           */
/* ------------------------------------------------------------------------ */

static float u32_as_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_as_u32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/*
 * Round a finite, non-negative magnitude `a` to the nearest value of a binary
 * format with `p` stored mantissa bits and minimum normal exponent `emin`
 * (subnormals included, exponent unbounded above), ties to even.
 * The quantum (spacing of representable values) around `a` is
 * 2^(max(exponent(a), emin) - p); a/quantum is exact in double because the
 * division is by a power of two.
 */
static double round_to_format(double a, int p, int emin)
{
    if (a == 0.0) return 0.0;
    int e2;
    (void)frexp(a, &e2);          /* a = f * 2^e2 with f in [0.5,1): exponent(a) = e2-1 */
    int e = e2 - 1;
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - p);
    return nearbyint(a / quantum) * quantum;   /* FE_TONEAREST: ties to even */
}

/* ------------------------------------------------------------------------ */
/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits.                 */
/* The activation dtype of the FP8 GEMM's output and of its input            */
/* ([C++FP8] §3.3, kernel name ..._e4m3bf16_e4m3f32_f32_tn).                 */
/* ------------------------------------------------------------------------ */

float orc_bf16_decode(uint16_t b)
{
    /* bf16 is the upper half of an IEEE binary32. */
    return u32_as_f32((uint32_t)b << 16);
}

uint16_t orc_bf16_encode(float f)
{
    uint32_t u = f32_as_u32(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs((double)f);
    if (isinf(f)) return (uint16_t)(sign | 0x7F80u);
    double r = round_to_format(a, 7, -126);
    if (r > 0x1.FEp127) return (uint16_t)(sign | 0x7F80u);  /* above max finite -> inf */
    if (r == 0.0) return sign;
    /* r is exactly representable in bf16 and therefore in binary32. */
    return (uint16_t)(sign | (f32_as_u32((float)r) >> 16));
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits.            */
/* The dtype of the NestedFP weights and activations ([NestedFP] §2.1).      */
/* ------------------------------------------------------------------------ */

double orc_f16_decode(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) v = (m == 0) ? INFINITY : NAN;
    else if (e == 0) v = ldexp((double)m, -24);                 /* m/2^10 * 2^-14 */
    else v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return s ? -v : v;
}

uint16_t orc_f16_encode(float f)
{
    uint16_t sign = (f32_as_u32(f) >> 31) ? 0x8000u : 0;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    double r = round_to_format(fabs((double)f), 10, -14);
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);       /* overflow -> inf */
    if (r < ldexp(1.0, -14)) {                                  /* subnormal or zero */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    }
    int e2; double fr = frexp(r, &e2);                          /* r = fr*2^e2, fr in [0.5,1) */
    int e = e2 - 1;                                             /* r = (2fr) * 2^e */
    int m = (int)((2.0 * fr - 1.0) * 1024.0);
    return (uint16_t)(sign | ((e + 15) << 10) | m);
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP "FN" variant): 1 sign, 4 exponent (bias 7), 3 mantissa.    */
/* No infinities; S.1111.111 is NaN; largest finite 448 = 1.75*2^8.          */
/* E4M3 is the format named for both operands ([RTX4060] §2.1, [C++FP8]      */
/* §3.1); its bound 448 appears in [RTX4060] §6.1, which only fits the OCP   */
/* variant (the "FNUZ" variant tops out at 240).                             */
/* ------------------------------------------------------------------------ */

double orc_e4m3_decode(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);                  /* m/8 * 2^-6 */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/*
 * Encode one binary32 value to E4M3 with a single round-to-nearest-even step
 * and saturation: magnitudes above 448 (and infinities) become 448, so the
 * exponent field never reaches the NaN pattern ([RTX4060] §6.1 asks that the
 * E4M3 exponent not saturate and that scaled values stay within 448).
 * Values below the smallest normal 2^-6 round into the subnormals, without
 * flushing to zero ([NestedFP] §4.1 asks that the E4M3 converter handle
 * underflow).  NaN maps to the NaN code with its sign.
 */
uint8_t orc_e4m3_encode(float f)
{
    uint8_t sign = (f32_as_u32(f) >> 31) ? 0x80u : 0;
    if (isnan(f)) return (uint8_t)(sign | 0x7Fu);
    double a = fabs((double)f);                                  /* inf stays inf */
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
    double r = round_to_format(a, 3, -6);
    if (r > 448.0) r = 448.0;                                    /* (unreachable: a < 448) */
    uint8_t code;
    if (r < ldexp(1.0, -6)) {
        code = (uint8_t)ldexp(r, 9);                             /* subnormal: r = m * 2^-9 */
    } else {
        int e2; double fr = frexp(r, &e2);
        int e = e2 - 1;                                          /* r = (2fr) * 2^e, e in [-6, 8] */
        int m = (int)((2.0 * fr - 1.0) * 8.0);
        code = (uint8_t)(((e + 7) << 3) | m);
    }
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* FP8 E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa, IEEE-style inf/NaN.   */
/* Named next to E4M3 in [C++FP8] §3.1.  In the NestedFP byte split the      */
/* upper byte of an fp16 word is, bit for bit, an E5M2 code ([NestedFP]      */
/* §2.1: upper 8 bits carry sign, the exponent and the top mantissa bits).   */
/* ------------------------------------------------------------------------ */

double orc_e5m2_decode(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31) v = (m == 0) ? INFINITY : NAN;
    else if (e == 0) v = ldexp((double)m, -16);                 /* m/4 * 2^-14 */
    else v = ldexp(1.0 + (double)m / 4.0, e - 15);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Dynamic per-tensor quantization ([RTX4060] §2.2: activations quantized at */
/* run time from each layer's amax; weights quantized statically offline).   */
/* Steps, in order:                                                          */
/*   1. amax = max |x_i|                                                     */
/*   2. s = fl32(amax / 448), or 1 when amax == 0                            */
/*   3. q_i = E4M3(fl32(x_i / s))                                            */
/* ------------------------------------------------------------------------ */

static float load_elem(const uint16_t* x, int dtype, int64_t i)
{
    return dtype == ORC_BF16 ? orc_bf16_decode(x[i]) : (float)orc_f16_decode(x[i]);
}

/* Step 1.  NaN elements are skipped (non-finite inputs are outside the
   parity contract; this is the documented behaviour). */
float orc_amax(const uint16_t* x, int dtype, int64_t n)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(load_elem(x, dtype, i));
        if (a > amax) amax = a;
    }
    return amax;
}

/* Step 2. */
float orc_scale_from_amax(float amax)
{
    if (amax > 0.0f) return amax / 448.0f;      /* one IEEE binary32 division */
    return 1.0f;
}

/* Step 3, for elements [0, n) with a given scale. */
void orc_quantize_with_scale(const uint16_t* x, int dtype, int64_t n, float s, uint8_t* q)
{
    for (int64_t i = 0; i < n; ++i) {
        float v = load_elem(x, dtype, i);
        float t = v / s;                        /* one IEEE binary32 division */
        q[i] = orc_e4m3_encode(t);
    }
}

/* All three steps. */
void orc_quantize(const uint16_t* x, int dtype, int64_t n, uint8_t* q, float* scale, float* amax)
{
    float a = orc_amax(x, dtype, n);
    float s = orc_scale_from_amax(a);
    orc_quantize_with_scale(x, dtype, n, s, q);
    *scale = s;
    *amax = a;
}

/* One scale per row of a [rows, cols] matrix: per-token activation scales   */
/* and per-channel weight scales (the per-token / per-channel options of the */
/* TensorRT-LLM build in [C++FP8] §4.2).  Each row is quantized on its own   */
/* with the three steps above.                                               */
void orc_quantize_rows(const uint16_t* x, int dtype, int64_t rows, int64_t cols, uint8_t* q,
                       float* scale, float* amax)
{
    for (int64_t r = 0; r < rows; ++r)
        orc_quantize(x + r * cols, dtype, cols, q + r * cols, scale + r, amax + r);
}

/* FP8 KV cache ([RTX4060] §1 stores the KV cache in FP8; [C++FP8] §4.2 builds */
/* with an FP8 KV-cache type): a K or V block x[T, H, D] (token-major, then   */
/* heads, then head dimension) with one scale per head h over all tokens and */
/* all D elements of that head.  Head h is gathered into a plain vector and   */
/* quantized by the three steps above; the codes go back to their places.  */
void orc_quantize_kv(const uint16_t* x, int dtype, int64_t T, int64_t H, int64_t D, uint8_t* q,
                     float* scale, float* amax)
{
    uint16_t* g = (uint16_t*)malloc((size_t)(T * D) * sizeof(uint16_t));
    uint8_t* c = (uint8_t*)malloc((size_t)(T * D));
    if (!g || !c) { free(g); free(c); return; }
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t t = 0; t < T; ++t)
            for (int64_t d = 0; d < D; ++d) g[t * D + d] = x[(t * H + h) * D + d];
        orc_quantize(g, dtype, T * D, c, scale + h, amax + h);
        for (int64_t t = 0; t < T; ++t)
            for (int64_t d = 0; d < D; ++d) q[(t * H + h) * D + d] = c[t * D + d];
    }
    free(g);
    free(c);
}

/* Delayed scaling with an amax history ([RTX4060] §6.1 asks that the amax   */
/* history be at least 1024 long).  Reading: history[L] holds the amax of    */
/* the last L calls on this tensor (zeros before any call), state[0] is the  */
/* scale the next call uses (0 = no history yet, meaning 1) and state[2] the */
/* ring position (as an integer).  One call:                                 */
/*   1. s = state[0] > 0 ? state[0] : 1                                      */
/*   2. q_i = E4M3_rne_sat(fl32(x_i / s))   (values beyond 448 s saturate)    */
/*   3. a = max |x_i|                                                        */
/*   4. history[pos] = a; pos = (pos + 1) mod L                              */
/*   5. state[0] = scale_from_amax(max over history)                         */
/* and the call reports s and a.  state[1] and state[3] are the device's     */
/* accumulators; the oracle leaves them at 0, as the device does between    */
/* calls.                                                                    */
void orc_quantize_delayed(const uint16_t* x, int dtype, int64_t n, uint8_t* q, float* scale,
                          float* amax, float* history, int64_t L, uint32_t* state)
{
    float next;
    memcpy(&next, &state[0], 4);
    float s = next > 0.0f ? next : 1.0f;
    orc_quantize_with_scale(x, dtype, n, s, q);
    float a = orc_amax(x, dtype, n);
    uint32_t pos = state[2];
    history[pos] = a;
    state[2] = (uint32_t)((pos + 1) % (uint64_t)L);
    float hmax = 0.0f;
    for (int64_t i = 0; i < L; ++i)
        if (history[i] > hmax) hmax = history[i];
    next = orc_scale_from_amax(hmax);
    memcpy(&state[0], &next, 4);
    *scale = s;
    *amax = a;
}

/* ------------------------------------------------------------------------ */
/* NestedFP byte split and rebuild ([NestedFP] §2.1): an fp16 word is kept   */
/* as its upper byte and its lower byte; FP16 mode rebuilds (upper<<8)|lower */
/* and FP8 mode uses the upper byte alone as an 8-bit float.                 */
/* ------------------------------------------------------------------------ */

void orc_nested_split(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        hi[i] = (uint8_t)(w[i] >> 8);
        lo[i] = (uint8_t)(w[i] & 0xFF);
    }
}

void orc_nested_rebuild(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) w[i] = (uint16_t)(((uint16_t)hi[i] << 8) | lo[i]);
}

/* The E4M3 upper-byte split ([NestedFP] §2.1 also names E4M3 as the upper  */
/* byte's format).  Reading: an fp16 word s|e4..e0|m9..m0 with e4 = 0 (|w| < 2) keeps  */
/* s|e3..e0|m9..m7 in the upper byte, which is then the E4M3 code of w * 2^8    */
/* truncated to 3 mantissa bits (fp16 subnormals land on E4M3 subnormals), and */
/* e4|m6..m0 in the lower byte, so the rebuild is exact for every fp16 word.   */
/* The FP8 mode (upper byte as E4M3, scale 2^-8) holds for finite |w| < 1.875; */
/* beyond that e4 = 1 or the code would read as NaN.  Returns how many words   */
/* break that range.                                                           */
int64_t orc_nested_split_e4m3(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n)
{
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint16_t v = w[i];
        uint16_t s = (uint16_t)(v >> 15);
        uint16_t e4 = (uint16_t)((v >> 14) & 1);
        uint16_t rest = (uint16_t)((v >> 7) & 0x7F);       /* e3..e0 m9 m8 m7 */
        hi[i] = (uint8_t)((s << 7) | rest);
        lo[i] = (uint8_t)((e4 << 7) | (v & 0x7F));
        double a = fabs(orc_f16_decode(v));
        if (e4 || !(a < 1.875)) ++bad;
    }
    return bad;
}

void orc_nested_rebuild_e4m3(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        w[i] = (uint16_t)(((hi[i] & 0x80) << 8) | ((lo[i] & 0x80) << 7) | ((hi[i] & 0x7F) << 7) |
                          (lo[i] & 0x7F));
}

/* ------------------------------------------------------------------------ */
/* GEMM checkers (fp64).  All matrices are row-major: activations [M,K],     */
/* weights [N,K] (K contiguous: the "tn" layout of the FP8 GEMM named in     */
/* [C++FP8] §3.3), outputs [M,N].  Each checker returns, for a list of       */
/* (m, n) pairs, ref = sum_k a[m,k]*w[n,k] times the dequantization scale,   */
/* and absref = sum_k |a[m,k]*w[n,k]| times the same scale, both in double.  */
/* ------------------------------------------------------------------------ */

/* The checkers evaluate each requested (m, n) pair independently; threads
   only split the list of pairs (no change to any sum). */
typedef struct {
    int kind;                       /* 0: FP8, 1: NestedFP FP16, 2: NestedFP FP8 */
    const void* a; const uint8_t* w; const uint8_t* w2;
    float sa, sw;
    int64_t K;
    const int64_t* ms; const int64_t* ns;
    int64_t t0, t1;
    double* ref; double* absref;
    const float* sav; const float* swv;   /* FP8 with a scale per row of a and of w */
} ref_job;

static void ref_pair(const ref_job* j, int64_t t)
{
    const int64_t K = j->K, m = j->ms[t], n = j->ns[t];
    double sum = 0.0, sabs = 0.0, scale = 1.0;
    if (j->kind == 0) {
        /* FP8 GEMM: E4M3 x E4M3, scale = s_a * s_w */
        const uint8_t* a = (const uint8_t*)j->a + m * K;
        const uint8_t* w = j->w + n * K;
        for (int64_t k = 0; k < K; ++k) {
            double p = orc_e4m3_decode(a[k]) * orc_e4m3_decode(w[k]);
            sum += p;
            sabs += fabs(p);
        }
        scale = (double)(j->sav ? j->sav[m] : j->sa) * (double)(j->swv ? j->swv[n] : j->sw);
    } else if (j->kind == 1) {
        /* NestedFP FP16 mode: fp16 activation x fp16 word (hi<<8)|lo, no scale */
        const uint16_t* a = (const uint16_t*)j->a + m * K;
        const uint8_t* h = j->w + n * K;
        const uint8_t* l = j->w2 + n * K;
        for (int64_t k = 0; k < K; ++k) {
            uint16_t wbits = (uint16_t)(((uint16_t)h[k] << 8) | l[k]);
            double p = orc_f16_decode(a[k]) * orc_f16_decode(wbits);
            sum += p;
            sabs += fabs(p);
        }
    } else {
        /* NestedFP FP8 mode: E4M3 activation x E5M2(hi), scale = s_a */
        const uint8_t* a = (const uint8_t*)j->a + m * K;
        const uint8_t* h = j->w + n * K;
        for (int64_t k = 0; k < K; ++k) {
            double p = orc_e4m3_decode(a[k]) * orc_e5m2_decode(h[k]);
            sum += p;
            sabs += fabs(p);
        }
        scale = (double)j->sa;
    }
    j->ref[t] = sum * scale;
    j->absref[t] = sabs * scale;
}

static void* ref_worker(void* arg)
{
    const ref_job* j = (const ref_job*)arg;
    for (int64_t t = j->t0; t < j->t1; ++t) ref_pair(j, t);
    return NULL;
}

static int g_ref_threads = 1;

/* Number of host threads the checkers below may use (default 1). */
void orc_set_ref_threads(int n) { g_ref_threads = n < 1 ? 1 : (n > 256 ? 256 : n); }

static void run_ref(ref_job proto, int64_t count)
{
    int nt = g_ref_threads;
    if (nt > count) nt = count > 0 ? (int)count : 1;
    pthread_t th[256];
    ref_job jobs[256];
    int64_t chunk = (count + nt - 1) / nt;
    int started = 0;
    for (int t = 0; t < nt; ++t) {
        jobs[t] = proto;
        jobs[t].t0 = t * chunk;
        jobs[t].t1 = jobs[t].t0 + chunk < count ? jobs[t].t0 + chunk : count;
        if (jobs[t].t0 >= jobs[t].t1) break;
        if (pthread_create(&th[t], NULL, ref_worker, &jobs[t]) != 0) {
            ref_worker(&jobs[t]);
            th[t] = 0;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t)
        if (th[t]) pthread_join(th[t], NULL);
}

/* FP8 GEMM: operands are E4M3 codes; scale = s_a * s_w. */
void orc_gemm_fp8_ref(const uint8_t* qa, float sa, const uint8_t* qw, float sw,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* ms, const int64_t* ns, int64_t count,
                      double* ref, double* absref)
{
    (void)M; (void)N;
    ref_job j = {0, qa, qw, NULL, sa, sw, K, ms, ns, 0, 0, ref, absref, NULL, NULL};
    run_ref(j, count);
}

/* FP8 GEMM with a scale per activation row (sa[M]) and per weight row (sw[N]):
   the pair (m, n) is scaled by sa[m] * sw[n]. */
void orc_gemm_fp8_rowwise_ref(const uint8_t* qa, const float* sa, const uint8_t* qw,
                              const float* sw, int64_t M, int64_t N, int64_t K,
                              const int64_t* ms, const int64_t* ns, int64_t count,
                              double* ref, double* absref)
{
    (void)M; (void)N;
    ref_job j = {0, qa, qw, NULL, 0.0f, 0.0f, K, ms, ns, 0, 0, ref, absref, sa, sw};
    run_ref(j, count);
}

/* NestedFP FP16 mode: a is fp16 [M,K]; weight = fp16 word (hi<<8)|lo. */
void orc_nested_fp16_ref(const uint16_t* a16, const uint8_t* hi, const uint8_t* lo,
                         int64_t M, int64_t N, int64_t K,
                         const int64_t* ms, const int64_t* ns, int64_t count,
                         double* ref, double* absref)
{
    (void)M; (void)N;
    ref_job j = {1, a16, hi, lo, 1.0f, 1.0f, K, ms, ns, 0, 0, ref, absref, NULL, NULL};
    run_ref(j, count);
}

/* NestedFP FP8 mode: a is E4M3 codes with scale s_a; weight = E5M2(hi). */
void orc_nested_fp8_ref(const uint8_t* qa, float sa, const uint8_t* hi,
                        int64_t M, int64_t N, int64_t K,
                        const int64_t* ms, const int64_t* ns, int64_t count,
                        double* ref, double* absref)
{
    (void)M; (void)N;
    ref_job j = {2, qa, hi, NULL, sa, 1.0f, K, ms, ns, 0, 0, ref, absref, NULL, NULL};
    run_ref(j, count);
}

/* ------------------------------------------------------------------------ */
/* Plain fp32-accumulating GEMMs: the same triple loop the method states     */
/* (fp32 accumulate in k order, then dequantize and round the output once).  */
/* These are what the CPU baseline times.  Threads only split the N range.   */
/* ------------------------------------------------------------------------ */

enum { KIND_FP8 = 0, KIND_NESTED_FP16 = 1, KIND_NESTED_FP8 = 2, KIND_FP8_FP16OUT = 3 };

typedef struct {
    int kind;
    const void* a; const uint8_t* w; const uint8_t* w2;
    float sa, sw;
    int64_t M, N, K, n0, n1;
    uint16_t* y;
    const float* sav; const float* swv;   /* KIND_FP8 with per-row scales, else NULL */
} gemm_job;

static void* gemm_worker(void* arg)
{
    gemm_job* j = (gemm_job*)arg;
    for (int64_t m = 0; m < j->M; ++m) {
        for (int64_t n = j->n0; n < j->n1; ++n) {
            float acc = 0.0f;
            if (j->kind == KIND_FP8) {
                const uint8_t* a = (const uint8_t*)j->a + m * j->K;
                const uint8_t* w = j->w + n * j->K;
                for (int64_t k = 0; k < j->K; ++k)
                    acc += (float)orc_e4m3_decode(a[k]) * (float)orc_e4m3_decode(w[k]);
                float s = (j->sav ? j->sav[m] : j->sa) *
                          (j->swv ? j->swv[n] : j->sw);     /* fl32(s_a * s_w) */
                j->y[m * j->N + n] = orc_bf16_encode(acc * s);
            } else if (j->kind == KIND_NESTED_FP16) {
                const uint16_t* a = (const uint16_t*)j->a + m * j->K;
                const uint8_t* h = j->w + n * j->K;
                const uint8_t* l = j->w2 + n * j->K;
                for (int64_t k = 0; k < j->K; ++k) {
                    uint16_t wbits = (uint16_t)(((uint16_t)h[k] << 8) | l[k]);
                    acc += (float)orc_f16_decode(a[k]) * (float)orc_f16_decode(wbits);
                }
                j->y[m * j->N + n] = orc_f16_encode(acc);
            } else if (j->kind == KIND_NESTED_FP8) {
                const uint8_t* a = (const uint8_t*)j->a + m * j->K;
                const uint8_t* h = j->w + n * j->K;
                for (int64_t k = 0; k < j->K; ++k)
                    acc += (float)orc_e4m3_decode(a[k]) * (float)orc_e5m2_decode(h[k]);
                j->y[m * j->N + n] = orc_f16_encode(acc * j->sa);
            } else {
                /* E4M3 x E4M3, fp16 output: the NestedFP FP8 mode of the E4M3 split */
                const uint8_t* a = (const uint8_t*)j->a + m * j->K;
                const uint8_t* h = j->w + n * j->K;
                for (int64_t k = 0; k < j->K; ++k)
                    acc += (float)orc_e4m3_decode(a[k]) * (float)orc_e4m3_decode(h[k]);
                float s = j->sa * j->sw;                    /* fl32(s_a * s_w) */
                j->y[m * j->N + n] = orc_f16_encode(acc * s);
            }
        }
    }
    return NULL;
}

static void run_gemm_scaled(int kind, const void* a, const uint8_t* w, const uint8_t* w2,
                            float sa, float sw, const float* sav, const float* swv,
                            int64_t M, int64_t N, int64_t K, uint16_t* y, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > N) nthreads = (int)N;
    pthread_t th[256];
    gemm_job jobs[256];
    int64_t chunk = (N + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t n0 = t * chunk, n1 = n0 + chunk < N ? n0 + chunk : N;
        if (n0 >= n1) break;
        jobs[t] = (gemm_job){kind, a, w, w2, sa, sw, M, N, K, n0, n1, y, sav, swv};
        if (pthread_create(&th[t], NULL, gemm_worker, &jobs[t]) != 0) {
            gemm_worker(&jobs[t]);                           /* run inline if no thread */
            th[t] = 0;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t)
        if (th[t]) pthread_join(th[t], NULL);
}

static void run_gemm(int kind, const void* a, const uint8_t* w, const uint8_t* w2,
                     float sa, float sw, int64_t M, int64_t N, int64_t K,
                     uint16_t* y, int nthreads)
{
    run_gemm_scaled(kind, a, w, w2, sa, sw, NULL, NULL, M, N, K, y, nthreads);
}

/* y[M,N] bf16 = bf16(fl32(acc) * fl32(s_a[m]*s_w[n])), acc = fp32 sum over k. */
void orc_gemm_fp8_rowwise_f32(const uint8_t* qa, const float* sa, const uint8_t* qw,
                              const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                              int nthreads)
{
    run_gemm_scaled(KIND_FP8, qa, qw, NULL, 0.0f, 0.0f, sa, sw, M, N, K, y, nthreads);
}

/* y[M,N] bf16 = bf16(fl32(acc) * fl32(s_a*s_w)), acc = fp32 sum over k. */
void orc_gemm_fp8_f32(const uint8_t* qa, float sa, const uint8_t* qw, float sw,
                      int64_t M, int64_t N, int64_t K, uint16_t* y, int nthreads)
{
    run_gemm(KIND_FP8, qa, qw, NULL, sa, sw, M, N, K, y, nthreads);
}

/* y[M,N] fp16 = fp16(acc), acc = fp32 sum of a16 * fp16((hi<<8)|lo). */
void orc_nested_fp16_f32(const uint16_t* a16, const uint8_t* hi, const uint8_t* lo,
                         int64_t M, int64_t N, int64_t K, uint16_t* y, int nthreads)
{
    run_gemm(KIND_NESTED_FP16, a16, hi, lo, 1.0f, 1.0f, M, N, K, y, nthreads);
}

/* y[M,N] fp16 = fp16(acc * s_a), acc = fp32 sum of E4M3(qa) * E5M2(hi). */
void orc_nested_fp8_f32(const uint8_t* qa, float sa, const uint8_t* hi,
                        int64_t M, int64_t N, int64_t K, uint16_t* y, int nthreads)
{
    run_gemm(KIND_NESTED_FP8, qa, hi, NULL, sa, 1.0f, M, N, K, y, nthreads);
}

/* y[M,N] fp16 = fp16(acc * fl32(s_a*s_w)), acc = fp32 sum of E4M3(qa) * E4M3(hi). */
void orc_gemm_fp8_f32_fp16out(const uint8_t* qa, float sa, const uint8_t* hi, float sw,
                              int64_t M, int64_t N, int64_t K, uint16_t* y, int nthreads)
{
    run_gemm(KIND_FP8_FP16OUT, qa, hi, NULL, sa, sw, M, N, K, y, nthreads);
}

/* Reports the rounding mode the oracle runs under (must be FE_TONEAREST). */
int orc_rounding_is_nearest(void) { return fegetround() == FE_TONEAREST; }

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar codecs above (plain loops, for the tests).      */
/* ------------------------------------------------------------------------ */

void orc_e4m3_encode_array(const float* v, uint8_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]); }

void orc_e4m3_decode_array(const uint8_t* c, double* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]); }

void orc_e5m2_decode_array(const uint8_t* c, double* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_decode(c[i]); }

void orc_f16_decode_array(const uint16_t* h, double* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_decode(h[i]); }

void orc_f16_encode_array(const float* v, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_encode(v[i]); }

void orc_bf16_decode_array(const uint16_t* b, float* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_decode(b[i]); }

void orc_bf16_encode_array(const float* v, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_encode(v[i]); }
