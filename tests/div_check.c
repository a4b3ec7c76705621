/*
 * Exhaustive check, on the CPU, of the division shortcut the GPU quantizer
 * uses for 16-bit inputs.
 *
 * The code of x in a block with absmax a is rint_even(fl32(x / s)) with
 * s = fl32(a / qmax) (IEEE division).  The kernel computes r = fl32(1 / s),
 * q0 = fl32(x * r) and ONE residual correction
 *     q1 = fma(fma(-q0, s, x), r, q0),
 * and rounds q1 to an integer.  This program checks, for every positive
 * finite fp16 (or bf16) absmax a whose scale is at least 2^-100 and every
 * value x of the same type with 0 <= x <= a (codes are odd in x), that
 * rint_even(q1) == rint_even(fl32(x / s)).  Written independently of both
 * the oracle and the kernel source; uses only IEEE float operations and the
 * correctly rounded fmaf of the C library.
 *
 * usage: div_check f16|bf16 qmax nthreads   -> prints "mismatches N cases M"
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

typedef struct { int t; long long bad, cases; } job_t;

static void* work(void* arg) {
    job_t* j = (job_t*)arg;
    const float fq = (float)g_qmax;
    for (int ia = 1 + j->t; ia < g_nvals; ia += g_threads) {
        float a = g_vals[ia];
        float s = a / fq;
        if (!(s >= 0x1p-100f)) continue;        /* slow path on the GPU */
        float r = 1.0f / s;
        for (int ix = 0; ix <= ia; ++ix) {
            float x = g_vals[ix];
            float q0 = x * r;
            float q1 = fmaf(fmaf(-q0, s, x), r, q0);
            float ref = x / s;
            j->cases++;
            if (rintf(q1) != rintf(ref)) j->bad++;
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
        jobs[t].t = t; jobs[t].bad = 0; jobs[t].cases = 0;
        pthread_create(&th[t], NULL, work, &jobs[t]);
    }
    long long bad = 0, cases = 0;
    for (int t = 0; t < g_threads; ++t) {
        pthread_join(th[t], NULL);
        bad += jobs[t].bad;
        cases += jobs[t].cases;
    }
    printf("mismatches %lld cases %lld\n", bad, cases);
    return 0;
}
