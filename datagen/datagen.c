/*
 * datagen.c -- seeded, counter-based synthetic inputs for the codec.
 *
 * Holds no codec arithmetic: it only draws random numbers.  Every value is a
 * pure function of (seed, element index, draw number), so any slice of a
 * stream can be regenerated on its own and the result does not depend on the
 * thread count.
 *
 * Generator: SplitMix64 finalizer (Steele, Lea, Flood 2014, "Fast splittable
 * pseudorandom number generators") applied to a counter built from
 * (seed, index, draw).  Uniforms on (0,1) take the top 53 bits plus 2^-54.
 * Normals: Box-Muller, cosine branch, in binary64.  Student-t with nu = 4:
 * z / sqrt(chi2_4 / 4), chi2_4 = -2 ln(u1 u2).  Values are returned as
 * binary32 (one rounding from binary64); narrowing to bf16 / fp16 is left to
 * the caller.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

static inline uint64_t mix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t draw64(uint64_t seed, uint64_t idx, unsigned draw)
{
    return mix64(mix64(seed * 0xD1B54A32D192ED03ull) ^ (idx * 8u + draw));
}

static inline double uniform01(uint64_t seed, uint64_t idx, unsigned draw)
{
    return (double)(draw64(seed, idx, draw) >> 11) * 0x1p-53 + 0x1p-54;
}

static inline double normal01(uint64_t seed, uint64_t idx, unsigned d0)
{
    double u1 = uniform01(seed, idx, d0), u2 = uniform01(seed, idx, d0 + 1);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

enum { DG_NORMAL = 0, DG_STUDENT4 = 1, DG_NORMAL_OUTLIER = 2, DG_ROWDRIFT = 3,
       DG_UNIFORM = 4 };

typedef struct {
    int kind;
    uint64_t seed, seed2, start;
    double p0, p1, p2;          /* kind-specific parameters */
    uint64_t cols;
    float *out;
    size_t lo, hi;
} job_t;

static float one_value(const job_t *j, uint64_t idx)
{
    switch (j->kind) {
    case DG_NORMAL:              /* mean p0, standard deviation p1 */
        return (float)(j->p0 + j->p1 * normal01(j->seed, idx, 0));
    case DG_STUDENT4: {          /* scale p1 */
        double z = normal01(j->seed, idx, 0);
        double chi2 = -2.0 * log(uniform01(j->seed, idx, 2) * uniform01(j->seed, idx, 3));
        return (float)(j->p1 * z / sqrt(chi2 / 4.0));
    }
    case DG_NORMAL_OUTLIER: {    /* N(0, p1); with prob p2 times p0 (separate draw) */
        double z = j->p1 * normal01(j->seed, idx, 0);
        if (uniform01(j->seed, idx, 4) < j->p2) z *= j->p0;
        return (float)z;
    }
    case DG_ROWDRIFT: {          /* p1 * N(0,1) * d_row, d_row ~ U[p0, p2] from seed2 */
        uint64_t row = idx / j->cols;
        double d = j->p0 + (j->p2 - j->p0) * uniform01(j->seed2, row, 0);
        return (float)(j->p1 * normal01(j->seed, idx, 0) * d);
    }
    default:                     /* U[p0, p1) */
        return (float)(j->p0 + (j->p1 - j->p0) * uniform01(j->seed, idx, 0));
    }
}

static void *run_job(void *arg)
{
    job_t *j = (job_t *)arg;
    for (size_t i = j->lo; i < j->hi; ++i) j->out[i] = one_value(j, j->start + i);
    return NULL;
}

/* Fill out[0..n) with values of elements start..start+n-1 of the stream.
 * threads <= 1 runs inline.  Returns 0 on success. */
int rcg_fill(int kind, uint64_t seed, uint64_t seed2, double p0, double p1, double p2,
             uint64_t cols, uint64_t start, size_t n, float *out, int threads)
{
    job_t base = {kind, seed, seed2, start, p0, p1, p2, cols ? cols : 1, out, 0, n};
    if (threads <= 1 || n < (1u << 16)) { run_job(&base); return 0; }
    if (threads > 64) threads = 64;
    pthread_t th[64];
    job_t jobs[64];
    int created[64] = {0};
    size_t chunk = (n + (size_t)threads - 1) / (size_t)threads;
    for (int t = 0; t < threads; ++t) {
        jobs[t] = base;
        jobs[t].lo = (size_t)t * chunk;
        jobs[t].hi = jobs[t].lo + chunk > n ? n : jobs[t].lo + chunk;
        if (jobs[t].lo >= jobs[t].hi) continue;
        if (pthread_create(&th[t], NULL, run_job, &jobs[t]) == 0) created[t] = 1;
        else run_job(&jobs[t]);
    }
    for (int t = 0; t < threads; ++t)
        if (created[t]) pthread_join(th[t], NULL);
    return 0;
}

/* Raw 64-bit draws, exposed so the tests can pin the generator itself. */
uint64_t rcg_draw64(uint64_t seed, uint64_t idx, unsigned draw) { return draw64(seed, idx, draw); }
uint64_t rcg_mix64(uint64_t z) { return mix64(z); }
