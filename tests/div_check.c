/*
 * Exhaustive check, on the CPU, of the arithmetic shortcuts the GPU quantizer
 * takes for 16-bit (fp16 / bf16) inputs.  By definition a block with absmax a
 * has scale s = fl32(a / qmax) and codes rint_even(fl32(x / s)), with IEEE
 * divisions.  The kernels instead compute
 *
 *   scale:       s0 = fl32(a * k) with k = fl32(1/qmax), then ONE residual
 *                correction s = fma(fma(-s0, qmax, a), k, s0)   (a >= 2^-90);
 *   reciprocal:  r = a float within one ulp of 1/s (either neighbour of the
 *                exact 1/s: the hardware reciprocal refined by one Newton
 *                step lands on one of them, whichever the hardware gives);
 *   code:        q0 = fl32(x * r), q1 = fma(fma(-q0, s, x), r, q0),
 *                rint_even(q1).
 *
 * This program enumerates every positive finite absmax a of the type and
 * checks
 *   (1) for a >= 2^-90: the corrected scale equals fl32(a / qmax);
 *   (2) for every a with fl32(a / qmax) >= 2^-100, every value 0 <= x <= a
 *       of the type (codes are odd in x) and BOTH floats r adjacent to the
 *       exact 1/s (a single one when 1/s is a float): rint_even(q1) equals
 *       rint_even(fl32(x / s)).
 * Written independently of both the oracle and the kernel source; uses only
 * IEEE float operations and the correctly rounded fmaf of the C library.
 *
 * usage: div_check f16|bf16 qmax nthreads
 *   -> prints "mismatches N cases M scale_mismatches K scales L"
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int g_bf16, g_qmax, g_threads;
static float g_vals[1 << 16];   /* all non-negative finite values, ascending */
static int g_nvals;

static float from_bits16(uint16_t h) {
    if (g_bf16) {
        uint32_t u = (uint32_t)h << 16;
        float f;
        memcpy(&f, &u, 4);
        return f;
    }
    int e = (h >> 10) & 0x1F, m = h & 0x3FF;
    if (e == 0) return ldexpf((float)m, -24);
    return ldexpf((float)(1024 + m), e - 25);
}

typedef struct { int t; long long bad, cases, sbad, scases; } job_t;

static void* work(void* arg) {
    job_t* j = (job_t*)arg;
    const float fq = (float)g_qmax;
    const float k = 1.0f / fq;
    for (int ia = 1 + j->t; ia < g_nvals; ia += g_threads) {
        const float a = g_vals[ia];
        const float s = a / fq;
        if (a >= 0x1p-90f) {
            const float s0 = a * k;
            const float sc = fmaf(fmaf(-s0, fq, a), k, s0);
            j->scases++;
            if (sc != s) j->sbad++;
        }
        if (!(s >= 0x1p-100f)) continue;          /* exact slow path on the GPU */
        /* the floats on either side of the exact 1/s */
        const float rn = 1.0f / s;
        const float res = fmaf(-s, rn, 1.0f);     /* exact: sign of 1/s - rn */
        float rr[2];
        int nr = 1;
        rr[0] = rn;
        if (res > 0.0f) { rr[1] = nextafterf(rn, INFINITY); nr = 2; }
        else if (res < 0.0f) { rr[1] = nextafterf(rn, 0.0f); nr = 2; }
        for (int ix = 0; ix <= ia; ++ix) {
            const float x = g_vals[ix];
            const float ref = rintf(x / s);
            for (int t = 0; t < nr; ++t) {
                const float r = rr[t];
                const float q0 = x * r;
                const float q1 = fmaf(fmaf(-q0, s, x), r, q0);
                j->cases++;
                if (rintf(q1) != ref) j->bad++;
            }
        }
    }
    return NULL;
}

int main(int argc, char** argv) {
    if (argc < 4) return 2;
    g_bf16 = strcmp(argv[1], "bf16") == 0;
    g_qmax = atoi(argv[2]);
    g_threads = atoi(argv[3]);
    if (g_threads < 1 || g_threads > 64) g_threads = 1;
    for (uint32_t h = 0; h < 0x8000; ++h) {
        float f = from_bits16((uint16_t)h);
        if (isfinite(f)) g_vals[g_nvals++] = f;   /* bit order is value order */
    }
    pthread_t th[64];
    job_t jobs[64];
    for (int t = 0; t < g_threads; ++t) {
        memset(&jobs[t], 0, sizeof jobs[t]);
        jobs[t].t = t;
        pthread_create(&th[t], NULL, work, &jobs[t]);
    }
    long long bad = 0, cases = 0, sbad = 0, scases = 0;
    for (int t = 0; t < g_threads; ++t) {
        pthread_join(th[t], NULL);
        bad += jobs[t].bad;
        cases += jobs[t].cases;
        sbad += jobs[t].sbad;
        scases += jobs[t].scases;
    }
    printf("mismatches %lld cases %lld scale_mismatches %lld scales %lld\n", bad, cases, sbad,
           scases);
    return 0;
}
