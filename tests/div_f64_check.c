/*
 * CPU check of the binary64 route the GPU kernels take for every division
 * with binary32 operands: the INT4/INT8 scale of fp32 blocks (including the
 * hop-1 requantization of fp32 sums), their codes, and the hop-2 average.
 * By definition these are IEEE binary32 quotients (then rounded to integers
 * for codes).  The kernels compute
 *
 *   scale:  s = (float)((double)a * RN64(1/qmax))     for a >= 2^-118,
 *           the binary32 quotient a / qmax otherwise;
 *   code:   rd = RN64(1/s) (0 when s == 0),
 *           q = rint_even((float)((double)x * rd)), clamped to [-qmax, qmax]
 *           when s is subnormal;
 *   mean:   y = (float)((double)acc * RN64(1/d)) when |acc| >= thr or acc == 0,
 *           thr = the binary32 number 2^-126 * d rounded up; else acc / d.
 *
 * Modes (argument 1):
 *   scale Q T   every positive finite binary32 absmax a, qmax Q, T threads:
 *               the kernel's scale equals a / Q (all 2^31 - 2^23 values).
 *   codes Q T   quantizer-produced scales s = a / Q for 2048 absmax values a
 *               in every binade (subnormal ones included, all significands of
 *               a at the binades' ends), and every x within 16 ulp of each
 *               rounding boundary (k + 1/2) * s, k = 0..Q, both signs, plus x
 *               = a and 64 random |x| <= a: the kernel's code equals
 *               clamp(rint_even(x / s)).
 *   fastcodes Q T   the same scales and values for the hop-1 requantization's
 *               faster code route: with a normal scale, r either of the two
 *               floats next to 1/s (the kernel refines the hardware
 *               reciprocal to one of them), the code is y = rint_even(x * r)
 *               of the exact product (one fused multiply-add with 1.5 * 2^23)
 *               unless the residual fl32(x * r - y) (a second fused
 *               multiply-add) exceeds 0.5 - 2^-19 in magnitude (then, and
 *               for scales below 2^-126, the binary64 route above): every
 *               value that takes the fast route, with either r, gets the
 *               definition's code.  Each (value, r) pair is a case.  Output
 *               adds "near K", the pairs sent to the binary64 route.
 *   mean T      divisors d = 1..65536, all powers of two 2^-40..2^40 and
 *               200000 random floats in [2^-20, 2^40]; for each, sums next to
 *               binary32 rounding boundaries of the quotient (16 ulp either
 *               side) across the normal range, and the threshold itself:
 *               the kernel's mean equals acc / d.
 * Output: "mismatches N cases M".
 *
 * Written from the definitions only; shares nothing with the oracle or the
 * kernels.  Uses IEEE binary32/binary64 arithmetic of the host (SSE2 on
 * x86-64), round to nearest even, no contraction (-ffp-contract=off).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int g_q, g_threads;

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* the kernels' formulas.  PLANT_FP32_PRODUCT replaces each binary64 product
 * by a binary32 one (a plausible mistake) so that the test can show the
 * checker catching it. */
#ifdef PLANT_FP32_PRODUCT
#define PRODUCT(x, r) ((x) * (float)(r))
#else
#define PRODUCT(x, r) ((float)((double)(x) * (r)))
#endif
static float k_scale(float a, int q) {
    const double inv = 1.0 / (double)q;
    return a >= 0x1p-118f ? PRODUCT(a, inv) : a / (float)q;
}
static float k_code(float x, float s, int q) {
    const double rd = s > 0.0f ? 1.0 / (double)s : 0.0;
    float t = PRODUCT(x, rd);
    if (!(s >= 0x1p-126f)) t = fminf(fmaxf(t, -(float)q), (float)q);
    return rintf(t);
}
/* the hop-1 requantization's faster route: the exact product x * r, r next
 * to 1/s, is within 7.0000009 * 2^-23 of x / s when s is normal and |x| <=
 * 7.0000009 s (the absmax element included), and fl32(x / s) within 2^-22 of
 * x / s, so rint_even of the product is the code unless the product lies
 * within 2^-19 of a half-integer.  PLANT_NARROW_MARGIN shrinks the margin to
 * 2^-30 (a plausible mistake) so that the test can show the checker catching
 * it. */
#ifdef PLANT_NARROW_MARGIN
#define FAST_MARGIN (0.5f - 0x1p-30f)
#else
#define FAST_MARGIN (0.5f - 0x1p-19f)
#endif
static float k_code_fast(float x, float s, float r, int q, int* exact_route) {
    if (!(s >= 0x1p-126f)) { *exact_route = 1; return k_code(x, s, q); }
    const float y = fmaf(x, r, 12582912.0f) - 12582912.0f;   /* rint_even(x * r), |x * r| < 2^22 */
    const float d = fmaf(x, r, -y);                           /* x * r - y, rounded once */
    if (fabsf(d) > FAST_MARGIN) { *exact_route = 1; return k_code(x, s, q); }
    *exact_route = 0;
    return y;
}
/* the definition */
static float d_code(float x, float s, int q) {
    if (s == 0.0f) return 0.0f;
    float t = rintf(x / s);
    if (t > (float)q) t = (float)q;
    if (t < -(float)q) t = -(float)q;
    return t;
}

/* splitmix64, for the random samples */
static uint64_t sm_next(uint64_t* st) {
    uint64_t z = (*st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

typedef struct { int t; long long bad, cases, near; } job_t;
static int g_fast;     /* fastcodes mode: check k_code_fast instead of k_code */

static void* scale_job(void* arg) {
    job_t* j = (job_t*)arg;
    const uint32_t top = 0x7F7FFFFFu;          /* FLT_MAX */
    const uint32_t per = top / (uint32_t)g_threads + 1;
    uint32_t lo = 1 + per * (uint32_t)j->t;
    uint64_t hi64 = (uint64_t)lo + per;
    uint32_t hi = hi64 > top + 1ull ? top + 1 : (uint32_t)hi64;
    for (uint32_t u = lo; u < hi && u <= top; ++u) {
        const float a = from_bits(u);
        j->cases++;
        if (bits_of(k_scale(a, g_q)) != bits_of(a / (float)g_q)) j->bad++;
    }
    return NULL;
}

static void check_code(job_t* j, float x, float s) {
    j->cases++;
    if (g_fast) {
        /* the two floats around 1/s (one float if 1/s is one) */
        const double rd = 1.0 / (double)s;
        float r[2];
        r[0] = (float)rd;
        r[1] = (double)r[0] == rd ? r[0]
               : (double)r[0] < rd ? nextafterf(r[0], INFINITY) : nextafterf(r[0], 0.0f);
        const float want = d_code(x, s, g_q);
        for (int i = 0; i < 2; ++i) {
            int exact_route = 0;
            if (i) j->cases++;
            const float c = k_code_fast(x, s, r[i], g_q, &exact_route);
            j->near += exact_route;
            if (c != want) j->bad++;
        }
    } else if (k_code(x, s, g_q) != d_code(x, s, g_q)) {
        j->bad++;
    }
}

static void* codes_job(void* arg) {
    job_t* j = (job_t*)arg;
    uint64_t rng = 0x1234567ull + (uint64_t)j->t;
    /* binades of a: exponent field 0 (subnormal) .. 254 */
    for (int e = j->t; e <= 254; e += g_threads) {
        for (int m = 0; m < 2048; ++m) {
            uint32_t mant;
            if (m < 512) mant = (uint32_t)m;                         /* low end */
            else if (m < 1024) mant = 0x7FFFFFu - (uint32_t)(m - 512); /* high end */
            else mant = (uint32_t)(sm_next(&rng) & 0x7FFFFFu);
            const uint32_t ua = ((uint32_t)e << 23) | mant;
            if (ua == 0) continue;
            const float a = from_bits(ua);
            const float s = a / (float)g_q;            /* the quantizer's scale */
            for (int k = 0; k <= g_q; ++k) {
                const double mid = ((double)k + 0.5) * (double)s;  /* exact in binary64 */
                const float x0 = (float)mid;
                float lo = x0, hi = x0;
                for (int step = 0; step <= 16; ++step) {
                    if (fabsf(lo) <= a) { check_code(j, lo, s); check_code(j, -lo, s); }
                    if (step && fabsf(hi) <= a) { check_code(j, hi, s); check_code(j, -hi, s); }
                    lo = nextafterf(lo, 0.0f);
                    hi = nextafterf(hi, INFINITY);
                }
            }
            check_code(j, a, s);
            check_code(j, -a, s);
            for (int r = 0; r < 64; ++r) {
                const float x = (float)((double)(sm_next(&rng) >> 11) * 0x1p-53 * (double)a);
                check_code(j, (r & 1) ? -x : x, s);
            }
        }
    }
    return NULL;
}

static float k_thr(float d) {
    const double t64 = ldexp((double)d, -126);
    float thr = (float)t64;
    if ((double)thr < t64) thr = nextafterf(thr, INFINITY);
    return thr;
}

static void check_mean(job_t* j, float acc, float d, double rd, float thr) {
    if (!(fabsf(acc) >= thr || acc == 0.0f)) return;   /* IEEE path on the GPU */
    j->cases++;
    if (bits_of(PRODUCT(acc, rd)) != bits_of(acc / d)) j->bad++;
}

static void mean_one(job_t* j, float d, uint64_t* rng) {
    const double rd = 1.0 / (double)d;
    const float thr = k_thr(d);
    /* the threshold: thr / d >= 2^-126 and the float below it is below */
    j->cases++;
    if (!((double)thr / (double)d >= 0x1p-126) ||
        !((double)nextafterf(thr, 0.0f) / (double)d < 0x1p-126))
        j->bad++;
    for (int r = 0; r < 24; ++r) {
        /* a binary32 quotient q, normal, such that q * d stays finite */
        const int lim = (int)floor(127.0 - log2((double)d));
        int emax = lim < 127 ? lim : 127;
        int ex = -126 + (int)(sm_next(rng) % (uint64_t)(emax + 127));
        const float qv = ldexpf(1.0f + (float)(sm_next(rng) & 0x7FFFFF) * 0x1p-23f, ex);
        const double mid = (double)qv + ldexp(1.0, ex - 24);      /* boundary above q */
        const double p = mid * (double)d;                          /* exact: 25 x 24 bits */
        if (!(fabs(p) < 3.4e38)) continue;
        float a0 = (float)p, lo = a0, hi = a0;
        for (int step = 0; step <= 16; ++step) {
            check_mean(j, lo, d, rd, thr);
            check_mean(j, -lo, d, rd, thr);
            if (step) { check_mean(j, hi, d, rd, thr); check_mean(j, -hi, d, rd, thr); }
            lo = nextafterf(lo, 0.0f);
            hi = nextafterf(hi, INFINITY);
        }
    }
    check_mean(j, thr, d, rd, thr);
    check_mean(j, 0.0f, d, rd, thr);
}

static void* mean_job(void* arg) {
    job_t* j = (job_t*)arg;
    uint64_t rng = 0xABCDEFull + (uint64_t)j->t;
    for (int d = 1 + j->t; d <= 65536; d += g_threads) mean_one(j, (float)d, &rng);
    for (int e = -40 + j->t; e <= 40; e += g_threads) mean_one(j, ldexpf(1.0f, e), &rng);
    for (int r = j->t; r < 200000; r += g_threads) {
        const float d = ldexpf(1.0f + (float)(sm_next(&rng) & 0x7FFFFF) * 0x1p-23f,
                               -20 + (int)(sm_next(&rng) % 60));
        mean_one(j, d, &rng);
    }
    return NULL;
}

int main(int argc, char** argv) {
    if (argc < 3) return 2;
    const char* mode = argv[1];
    void* (*fn)(void*) = NULL;
    if (!strcmp(mode, "scale") || !strcmp(mode, "codes") || !strcmp(mode, "fastcodes")) {
        if (argc < 4) return 2;
        g_q = atoi(argv[2]);
        g_threads = atoi(argv[3]);
        g_fast = !strcmp(mode, "fastcodes");
        fn = !strcmp(mode, "scale") ? scale_job : codes_job;
    } else if (!strcmp(mode, "mean")) {
        g_threads = atoi(argv[2]);
        fn = mean_job;
    } else {
        return 2;
    }
    if (g_threads < 1 || g_threads > 64) g_threads = 1;
    pthread_t th[64];
    job_t jobs[64];
    for (int t = 0; t < g_threads; ++t) {
        memset(&jobs[t], 0, sizeof jobs[t]);
        jobs[t].t = t;
        pthread_create(&th[t], NULL, fn, &jobs[t]);
    }
    long long bad = 0, cases = 0, near = 0;
    for (int t = 0; t < g_threads; ++t) {
        pthread_join(th[t], NULL);
        bad += jobs[t].bad;
        cases += jobs[t].cases;
        near += jobs[t].near;
    }
    if (g_fast) printf("mismatches %lld cases %lld near %lld\n", bad, cases, near);
    else printf("mismatches %lld cases %lld\n", bad, cases);
    return 0;
}
