/*
 * synth.c -- seeded synthetic inputs for tests and benchmarks.
 *
 * Holds no quantization arithmetic: only a counter-based random generator and
 * the distributions the workloads are drawn from.  Every value is a pure
 * function of (seed, stream, index), so any slice of a tensor can be
 * regenerated on its own and the result does not depend on the thread count.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; the finalizer as published by Vigna).
 * Counter c of stream (seed, stream) is the 64-bit output of the finalizer
 * applied to  key + (c + 1) * 0x9E3779B97F4A7C15,
 * key = seed * 0xD1B54A32D192ED03 + stream * 0x8CB92BA72F3D8DD7.
 * Uniforms use the top 53 bits.  Normals use Box-Muller in double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t key_of(uint64_t seed, uint64_t stream) {
    return seed * 0xD1B54A32D192ED03ULL + stream * 0x8CB92BA72F3D8DD7ULL;
}

static inline uint64_t draw(uint64_t key, uint64_t c) {
    return mix64(key + (c + 1) * GOLDEN);
}

/* uniform in (0, 1]: never 0, so log() is finite */
static inline double unif_open0(uint64_t key, uint64_t c) {
    return (double)((draw(key, c) >> 11) + 1) * 0x1.0p-53;
}

/* uniform in [0, 1) */
static inline double unif(uint64_t key, uint64_t c) {
    return (double)(draw(key, c) >> 11) * 0x1.0p-53;
}

/* Box-Muller pair from counters 2i, 2i+1 */
static inline void normal_pair(uint64_t key, uint64_t i, double* z0, double* z1) {
    double u1 = unif_open0(key, 2 * i);
    double u2 = unif(key, 2 * i + 1);
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925 * u2;
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

enum { K_NORMAL = 0, K_T3 = 1, K_BLOCKVAR = 2, K_U64 = 3, K_UNIF = 4 };

typedef struct {
    int kind;
    uint64_t key, key2;
    int64_t offset, begin, end;
    double a, b, c;     /* kind-specific parameters */
    int64_t block;
    void* out;
} job_t;

static void run_range(const job_t* j) {
    for (int64_t k = j->begin; k < j->end; ++k) {
        uint64_t i = (uint64_t)(j->offset + k);
        switch (j->kind) {
        case K_NORMAL: {               /* mean a, standard deviation b */
            double z0, z1;
            normal_pair(j->key, i, &z0, &z1);
            ((float*)j->out)[k] = (float)(j->a + j->b * z0);
            break;
        }
        case K_T3: {                   /* b * t_3; t_3 = z / sqrt(chi2_3 / 3) */
            /* chi2_3 = chi2_2 + chi2_1, chi2_2 = -2 ln U (an exponential of
             * mean 2), chi2_1 = z1^2 with z1 independent of z0 */
            double z0, z1;
            normal_pair(j->key, i, &z0, &z1);
            double chi2 = -2.0 * log(unif_open0(j->key2, i)) + z1 * z1;
            ((float*)j->out)[k] = (float)(j->b * z0 / sqrt(chi2 / 3.0));
            break;
        }
        case K_BLOCKVAR: {             /* b * sqrt(v) * z, v = 10^U(a_lo, c_hi) per block */
            double z0, z1;
            normal_pair(j->key, i, &z0, &z1);
            uint64_t blk = i / (uint64_t)j->block;
            double e = j->a + (j->c - j->a) * unif(j->key2, blk);
            double v = pow(10.0, e);
            ((float*)j->out)[k] = (float)(j->b * sqrt(v) * z0);
            break;
        }
        case K_U64:
            ((uint64_t*)j->out)[k] = draw(j->key, i);
            break;
        case K_UNIF:
            ((double*)j->out)[k] = unif(j->key, i);
            break;
        }
    }
}

static void* thread_main(void* arg) {
    run_range((const job_t*)arg);
    return NULL;
}

static void run_parallel(job_t proto, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < 65536) nthreads = 1;
    pthread_t th[256];
    job_t jobs[256];
    int64_t per = (n + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].begin = (int64_t)t * per;
        jobs[t].end = jobs[t].begin + per < n ? jobs[t].begin + per : n;
        if (jobs[t].begin >= jobs[t].end) break;
        if (nthreads == 1 || pthread_create(&th[t], NULL, thread_main, &jobs[t]) != 0) {
            run_range(&jobs[t]);
            th[t] = 0;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t)
        if (nthreads > 1 && th[t]) pthread_join(th[t], NULL);
}

/* out[k] = mean + std * z for element index offset + k */
void synth_normal(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                  double mean, double std, float* out, int nthreads) {
    job_t j = {K_NORMAL, key_of(seed, stream), 0, offset, 0, 0, mean, std, 0, 0, out};
    run_parallel(j, n, nthreads);
}

/* out[k] = scale * t_3 (Student t with 3 degrees of freedom) */
void synth_student_t3(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                      double scale, float* out, int nthreads) {
    job_t j = {K_T3, key_of(seed, stream), key_of(seed, stream + 0x10000), offset, 0, 0,
               0, scale, 0, 0, out};
    run_parallel(j, n, nthreads);
}

/* out[k] = base * sqrt(v_b) * z, v_b = 10^(lo + (hi-lo)*U_b) drawn once per
 * `block` consecutive elements (a log-uniform variance multiplier) */
void synth_blockvar_normal(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                           int64_t block, double base, double log10_lo, double log10_hi,
                           float* out, int nthreads) {
    job_t j = {K_BLOCKVAR, key_of(seed, stream), key_of(seed, stream + 0x10000), offset,
               0, 0, log10_lo, base, log10_hi, block, out};
    run_parallel(j, n, nthreads);
}

/* raw 64-bit draws (keys for seeded selection of positions or blocks) */
void synth_u64(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
               uint64_t* out, int nthreads) {
    job_t j = {K_U64, key_of(seed, stream), 0, offset, 0, 0, 0, 0, 0, 0, out};
    run_parallel(j, n, nthreads);
}

/* uniforms in [0, 1) */
void synth_uniform(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                   double* out, int nthreads) {
    job_t j = {K_UNIF, key_of(seed, stream), 0, offset, 0, 0, 0, 0, 0, 0, out};
    run_parallel(j, n, nthreads);
}
