/*
 * device_arith.c -- CPU emulation of the binary32 instruction sequences the
 * gfx950 kernels use in place of IEEE division, each checked against the
 * exact rule it stands for.  Test infrastructure (run by
 * tests/test_device_arith.py); it restates the kernels' sequences with C's
 * fmaf and binary32 arithmetic and shares no code with the kernels or with
 * the oracle.
 *
 *   div      q = a * RN(1/B); result = fma(fma(-q, B, a), RN(1/B), q) for
 *            B = 3, 7 (INT scales: absmax / qmax) and 448, 57344 (FP8
 *            scales): equal to the IEEE quotient a / B for every finite
 *            a >= 0 (448, 57344: wherever that quotient is normal, and below
 *            2^-126 exactly when it is).
 *   recip    r = fma(fma(-s, y0, 1), y0, y0) for every positive finite fp16
 *            s and every y0 the hardware reciprocal may return (the two
 *            binary32 values around 1/s, or 1/s itself): r = RN(1/s).
 *   int      INT3 / INT4 codes from y = fma(x, r c, x (r_lo c)) with r =
 *            1/s rounded down (RN(1/s), stepped down one ulp when above 1/s),
 *            r_lo = fma(-s, r, 1) r >= 0 and c = 1/2 (E2M1 conversion) or 2^-9
 *            (E4M3 subnormals), converted with round-to-nearest-even and
 *            clamped only for abnormal scales: equal to round-half-even of
 *            the exact quotient x / s clamped to qmax.  Exhaustive over every
 *            fp16 scale and every bf16 x of the domain a block can produce,
 *            plus binary32 x within 16 ulp of every half step of every
 *            scale, plus random binary32 x.  For every scale r_lo >= 0, and
 *            y of -0 is -0 (the sign plane keeps the sign of a -0 element).
 *   fp8      the round-to-odd quotient sequence (y0 = |x| rs, y1 = y0 +
 *            fma(-y0, s, |x|) rs, side from fma(-y1, s, |x|), then
 *            round-to-odd, clamp with FP16 scales) followed by the RNE
 *            conversion to E4M3 / E5M2: equal to the RNE code of the exact
 *            quotient, for binary32 x within 16 ulp of every rounding
 *            midpoint (and of the saturation point) of the format, over
 *            random FP32 scales, scales below 2^-64 (x and s times 2^64),
 *            and every fp16 scale, with rs either binary32 neighbour of 1/s.
 *
 * Usage: device_arith <check> [threads]; prints one line per check and exits
 * 0 when no case differs.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float half_value(uint16_t h)            /* exact fp16 -> binary32 */
{
    int e = (h >> 10) & 31, m = h & 1023;
    double v = e ? ldexp(1024 + m, e - 25) : ldexp(m, -24);
    return (float)((h >> 15) ? -v : v);
}

/* ---------------------------------------------------------------- threads */

typedef struct { uint64_t lo, hi, bad, cases; int arg, tid, nthr; uint64_t seed, total; } job;
typedef void *(*worker)(void *);

static uint64_t run_parallel(worker fn, uint64_t total, int threads, int arg, uint64_t *cases)
{
    pthread_t t[64];
    job j[64];
    if (threads > 64) threads = 64;
    for (int i = 0; i < threads; ++i) {
        j[i].lo = total * (uint64_t)i / threads;
        j[i].hi = total * (uint64_t)(i + 1) / threads;
        j[i].bad = j[i].cases = 0;
        j[i].arg = arg;
        j[i].tid = i;
        j[i].nthr = threads;
        j[i].total = total;
        j[i].seed = 0x9E3779B97F4A7C15ull * (uint64_t)(i + 1) + (uint64_t)arg;
        pthread_create(&t[i], NULL, fn, &j[i]);
    }
    uint64_t bad = 0;
    *cases = 0;
    for (int i = 0; i < threads; ++i) { pthread_join(t[i], NULL); bad += j[i].bad; *cases += j[i].cases; }
    return bad;
}

static uint64_t splitmix(uint64_t *s)
{
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* ------------------------------------------------------------------- div */

static const float kDivB[4] = {3.0f, 7.0f, 448.0f, 57344.0f};

static void *div_worker(void *p)
{
    job *j = p;
    const float B = kDivB[j->arg];
    volatile float Bv = B;
    const float y = 1.0f / Bv;                     /* RN(1/B) */
    /* chunks of 2^16 values dealt round-robin: the tiny values (subnormal
     * residuals run in microcode on the CPU) spread over every thread */
    for (uint64_t u = (uint64_t)j->tid << 16; u < j->total;
         u = ((u & 0xFFFFu) == 0xFFFFu) ? u + 1 + ((uint64_t)(j->nthr - 1) << 16) : u + 1) {
        const float a = u2f((uint32_t)u);
        const float q = a * y;
        const float got = fmaf(fmaf(-q, B, a), y, q);
        const float want = a / B;
        j->cases++;
        if (j->arg < 2) { if (f2u(got) != f2u(want)) j->bad++; }
        else if (want >= 0x1p-126f) { if (f2u(got) != f2u(want)) j->bad++; }
        else if (got >= 0x1p-126f) j->bad++;       /* flush decision must agree */
    }
    return NULL;
}

/* ----------------------------------------------------------------- recip */

static float recip_seq(float s, float y0) { return fmaf(fmaf(-s, y0, 1.0f), y0, y0); }

/* the binary32 values the hardware reciprocal of s may return: 1/s itself
 * when exact, else the two neighbours around it */
static int rcp_candidates(float s, float out[2])
{
    const float r = 1.0f / s;
    const long double p = (long double)r * (long double)s;    /* exact: 24 + 24 bits */
    if (p == 1.0L) { out[0] = r; return 1; }
    out[0] = r;
    out[1] = nextafterf(r, p < 1.0L ? INFINITY : 0.0f);         /* the other side of 1/s */
    return 2;
}

static uint64_t check_recip(uint64_t *cases)
{
    uint64_t bad = 0;
    *cases = 0;
    for (uint32_t h = 1; h < 0x7C00; ++h) {
        const float s = half_value((uint16_t)h);
        float c[2];
        const int nc = rcp_candidates(s, c);
        for (int i = 0; i < nc; ++i) {
            ++*cases;
            if (f2u(recip_seq(s, c[i])) != f2u(1.0f / s)) ++bad;
        }
    }
    return bad;
}

/* ------------------------------------------------------------------- int */

/* round-half-even of the exact quotient x / s, clamped to qmax (x >= 0) */
static int int_exact(float xf, float sf, int qmax)
{
    const double x = xf, s = sf;
    if (!(x < (qmax + 0.5) * s)) return qmax;
    int m = (int)nearbyint(x / s);
    while (m > 0 && x < (m - 0.5) * s) --m;        /* products are exact */
    while (x > (m + 0.5) * s) ++m;
    if (x == (m - 0.5) * s && (m & 1)) --m;        /* tie: even neighbour */
    if (x == (m + 0.5) * s && (m & 1)) ++m;
    return m > qmax ? qmax : m;
}

typedef struct { float s, r, r_lo; int abnormal; } iscale;

static iscale int_scale_of(uint16_t h)
{
    iscale k;
    k.s = half_value(h);
    float c[2];
    rcp_candidates(k.s, c);
    k.r = recip_seq(k.s, c[0]);                     /* RN(1/s) */
    float e = fmaf(-k.s, k.r, 1.0f);
    if (e < 0.0f) k.r = u2f(f2u(k.r) - 1u);          /* rounded down: r <= 1/s */
    e = fmaf(-k.s, k.r, 1.0f);
    k.r_lo = e * k.r;
    k.abnormal = (h < 0x0400) || (h == 0x7BFF);
    return k;
}

/* nearest entry of an increasing table (exact comparisons), ties to the
 * even index, saturating */
static int nearest_tab(const double *tab, int cnt, double num, double den)
{
    int lo = 0, hi = cnt - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (tab[mid] * den <= num) lo = mid; else hi = mid - 1;
    }
    if (lo == cnt - 1) return lo;
    const double mid = 0.5 * (tab[lo] + tab[lo + 1]) * den;
    if (num > mid) return lo + 1;
    if (num < mid) return lo;
    return (lo & 1) ? lo + 1 : lo;
}

static double e2m1_tab[8] = {0, 0.5, 1, 1.5, 2, 3, 4, 6};
static double e4m3_tab[127], e5m2_tab[124];

static void init_tables(void)
{
    for (int c = 0; c < 127; ++c) {
        int e = c >> 3, m = c & 7;
        e4m3_tab[c] = e ? ldexp(8 + m, e - 10) : ldexp(m, -9);
    }
    for (int c = 0; c < 124; ++c) {
        int e = c >> 2, m = c & 3;
        e5m2_tab[c] = e ? ldexp(4 + m, e - 17) : ldexp(m, -16);
    }
}

/* the kernel's INT code of x >= 0 (qmax 3: E2M1 route; 7: E4M3 route);
 * returns -1 when the unclamped code of a normal scale exceeds qmax.  With
 * single_product the low part is dropped (y = x r c alone): the control
 * that must differ, showing the cases reach the rounding decisions. */
static int single_product = 0;

static int int_device(float x, const iscale *k, int qmax)
{
    int code;
    if (single_product) {
        const float y = x * ((qmax == 3 ? 0.5f : 0x1p-9f) * k->r);
        code = nearest_tab(qmax == 3 ? e2m1_tab : e4m3_tab, qmax == 3 ? 8 : 127, (double)y, 1.0);
        return code > qmax ? qmax : code;
    }
    if (qmax == 3) {
        const float y = fmaf(x, 0.5f * k->r, x * (0.5f * k->r_lo));
        code = nearest_tab(e2m1_tab, 8, (double)y, 1.0);
        if (code > 3) { if (!k->abnormal) return -1; code = 3; }
    } else {
        const float y = fmaf(x, 0x1p-9f * k->r, x * (0x1p-9f * k->r_lo));
        code = nearest_tab(e4m3_tab, 127, (double)y, 1.0);
        if (code > 7) { if (!k->abnormal) return -1; code = 7; }
    }
    return code;
}

/* one fp16 scale per index: every bf16 x >= 0 of the block domain */
static void *int_bf16_worker(void *p)
{
    job *j = p;
    const int qmax = j->arg;
    for (uint64_t h = j->lo + 1; h < j->hi + 1; ++h) {
        const iscale k = int_scale_of((uint16_t)h);
        /* a block with this scale holds |x| <= absmax < (qmax + 1/2) s for a
         * normal scale; below 2^-11 for a subnormal one; anything for 65504 */
        const double bound = (h == 0x7BFF) ? INFINITY : (h < 0x0400 ? 0x1p-11 : (qmax + 0.5) * (double)k.s);
        for (uint32_t b = 0; b < 0x7F80; ++b) {
            const float x = u2f(b << 16);
            if (!((double)x < bound)) break;
            j->cases++;
            if (int_device(x, &k, qmax) != int_exact(x, k.s, qmax)) j->bad++;
        }
    }
    return NULL;
}

/* binary32 x within 16 ulp of every half step (k + 1/2) s, every fp16 scale */
static void *int_ties_worker(void *p)
{
    job *j = p;
    const int qmax = j->arg;
    for (uint64_t h = j->lo + 1; h < j->hi + 1; ++h) {
        const iscale k = int_scale_of((uint16_t)h);
        for (int m = 0; m < qmax; ++m) {
            const float t = (float)((m + 0.5) * (double)k.s);        /* exact */
            float x = t;
            for (int i = 0; i < 16; ++i) x = nextafterf(x, 0.0f);
            for (int i = 0; i <= 32; ++i, x = nextafterf(x, INFINITY)) {
                j->cases++;
                if (int_device(x, &k, qmax) != int_exact(x, k.s, qmax)) j->bad++;
            }
        }
    }
    return NULL;
}

/* random binary32 x with x / s uniform below qmax + 1/2, random fp16 scale */
static void *int_random_worker(void *p)
{
    job *j = p;
    const int qmax = j->arg;
    for (uint64_t i = j->lo; i < j->hi; ++i) {
        const uint16_t h = (uint16_t)(1 + splitmix(&j->seed) % 0x7BFE);
        const iscale k = int_scale_of(h);
        const double u = (double)(splitmix(&j->seed) >> 11) * 0x1p-53;
        float x = (float)(u * (qmax + 0.5) * (double)k.s);
        if (!((double)x < (qmax + 0.5) * (double)k.s)) x = nextafterf(x, 0.0f);
        j->cases++;
        if (int_device(x, &k, qmax) != int_exact(x, k.s, qmax)) j->bad++;
    }
    return NULL;
}

/* ------------------------------------------------------------------- fp8 */

/* the kernel's round-to-odd quotient of |x| / s (sign dropped: x >= 0) */
static float ro_quotient(float ax, float s, float rs, float fmax, int clamp)
{
    const float y0 = ax * rs;
    const float y1 = fmaf(fmaf(-y0, s, ax), rs, y0);
    const float r = fmaf(-y1, s, ax);
    uint32_t t = f2u(y1);
    t = (t - (r < 0.0f ? 1u : 0u)) | (r != 0.0f ? 1u : 0u);
    const float yo = u2f(t);
    return clamp ? fminf(yo, fmax) : yo;
}

/* hardware RNE conversion of a binary32 value >= 0 to the format; -1 where
 * the instruction would leave the finite range (the kernel must never feed
 * such a value) */
static int fp8_convert(float y, int e5)
{
    const double *tab = e5 ? e5m2_tab : e4m3_tab;
    const int cnt = e5 ? 124 : 127;
    const double top = tab[cnt - 1], next = e5 ? 65536.0 : 512.0;
    if ((double)y > 0.5 * (top + next)) return -1;
    if ((double)y == 0.5 * (top + next)) return -1;
    return nearest_tab(tab, cnt, (double)y, 1.0);
}

/* kernel: x and s below 2^-64 are multiplied by 2^64 first */
static int fp8_device(float x, float s, int which_rcp, int e5, int clamp)
{
    const float fmax = e5 ? 57344.0f : 448.0f;
    float kx = x, ks = s;
    if (s < 0x1p-64f) { kx = x * 0x1p64f; ks = s * 0x1p64f; }
    float c[2];
    const int nc = rcp_candidates(ks, c);
    const float rs = c[which_rcp < nc ? which_rcp : 0];
    return fp8_convert(ro_quotient(kx, ks, rs, fmax, clamp), e5);
}

static int fp8_exact(float x, float s, int e5)
{
    return e5 ? nearest_tab(e5m2_tab, 124, (double)x, (double)s) : nearest_tab(e4m3_tab, 127, (double)x, (double)s);
}

/* the FP8 scale of a random block: s = RN32(absmax / fmax), or an fp16 scale */
static void fp8_one_scale(job *j, float s, int e5, int clamp)
{
    const double *tab = e5 ? e5m2_tab : e4m3_tab;
    const int cnt = e5 ? 124 : 127;
    /* every midpoint between neighbouring magnitudes, and the point halfway
     * to the next binade above the largest (where saturation takes over) */
    for (int c = 0; c < cnt; ++c) {
        const double mid = (c + 1 < cnt) ? 0.5 * (tab[c] + tab[c + 1]) : tab[c] * 1.0625;
        const double target = mid * (double)s;
        if (target > 3.0e38) continue;
        float x = (float)target;
        for (int i = 0; i < 16; ++i) x = nextafterf(x, 0.0f);
        for (int i = 0; i <= 32; ++i, x = nextafterf(x, INFINITY)) {
            /* the block's absmax bounds x: with an FP32 scale x <= fmax s
             * (RN32 of absmax / fmax), nothing above needs to encode */
            if (!clamp && (double)x > tab[cnt - 1] * (double)s * (1.0 + 0x1p-23)) break;
            const int want = fp8_exact(x, s, e5);
            for (int w = 0; w < 2; ++w) {
                j->cases++;
                if (fp8_device(x, s, w, e5, clamp) != want) j->bad++;
            }
        }
    }
}

static void *fp8_worker(void *p)
{
    job *j = p;
    const int e5 = j->arg & 1, mode = j->arg >> 1;
    for (uint64_t i = j->lo; i < j->hi; ++i) {
        if (mode == 2) {                               /* every fp16 scale */
            fp8_one_scale(j, half_value((uint16_t)(i + 1)), e5, 1);
            continue;
        }
        /* random normal FP32 scale (mode 0) or one below 2^-64 (mode 1) */
        const uint64_t r = splitmix(&j->seed);
        const int ex = mode == 0 ? (int)(r % 200) - 100 : -126 + (int)(r % 62);
        const float s = ldexpf(1.0f + (float)((r >> 8) & 0x7FFFFF) * 0x1p-23f, ex);
        fp8_one_scale(j, s, e5, 0);
    }
    return NULL;
}

/* ------------------------------------------------------------------- main */

static int report(const char *name, uint64_t bad, uint64_t cases)
{
    printf("%-28s cases %12llu  differ %llu\n", name, (unsigned long long)cases, (unsigned long long)bad);
    return bad != 0 || cases == 0;
}

int main(int argc, char **argv)
{
    if (argc < 2) { fprintf(stderr, "usage: %s div|recip|int|fp8 [threads]\n", argv[0]); return 2; }
    const int T = argc > 2 ? atoi(argv[2]) : 8;
    init_tables();
    int fail = 0;
    uint64_t cases, bad;
    if (!strcmp(argv[1], "div")) {
        static const char *names[4] = {"div 3 (all binary32)", "div 7 (all binary32)",
                                       "div 448 (all binary32)", "div 57344 (all binary32)"};
        for (int b = 0; b < 4; ++b) {
            bad = run_parallel(div_worker, 0x7F800000ull, T, b, &cases);
            fail |= report(names[b], bad, cases);
        }
    } else if (!strcmp(argv[1], "recip")) {
        bad = check_recip(&cases);
        fail |= report("recip (every fp16, 1 ulp)", bad, cases);
    } else if (!strcmp(argv[1], "int")) {
        uint64_t sb = 0, sc = 0;
        for (uint32_t h = 1; h < 0x7C00; ++h) {
            const iscale k = int_scale_of((uint16_t)h);
            const float z = -0.0f;
            const float y3 = fmaf(z, 0.5f * k.r, z * (0.5f * k.r_lo));
            const float y4 = fmaf(z, 0x1p-9f * k.r, z * (0x1p-9f * k.r_lo));
            sc += 3;
            sb += !(k.r_lo >= 0.0f) + !signbit(y3) + !signbit(y4);
        }
        fail |= report("int low part >= 0, -0 kept", sb, sc);
        for (int q = 3; q <= 7; q += 4) {
            char nm[64];
            snprintf(nm, sizeof nm, "int qmax %d bf16 exhaustive", q);
            bad = run_parallel(int_bf16_worker, 0x7BFF, T, q, &cases);
            fail |= report(nm, bad, cases);
            snprintf(nm, sizeof nm, "int qmax %d half steps", q);
            bad = run_parallel(int_ties_worker, 0x7BFF, T, q, &cases);
            fail |= report(nm, bad, cases);
            snprintf(nm, sizeof nm, "int qmax %d random fp32", q);
            bad = run_parallel(int_random_worker, 20000000, T, q, &cases);
            fail |= report(nm, bad, cases);
            single_product = 1;
            bad = run_parallel(int_ties_worker, 0x7BFF, T, q, &cases);
            single_product = 0;
            snprintf(nm, sizeof nm, "control qmax %d one product", q);
            printf("%-28s cases %12llu  differ %llu (must differ)\n", nm, (unsigned long long)cases,
                   (unsigned long long)bad);
            fail |= bad == 0;
        }
    } else if (!strcmp(argv[1], "fp8")) {
        static const char *names[6] = {"e4m3 fp32 scales", "e5m2 fp32 scales", "e4m3 scales < 2^-64",
                                       "e5m2 scales < 2^-64", "e4m3 every fp16 scale", "e5m2 every fp16 scale"};
        for (int m = 0; m < 6; ++m) {
            const uint64_t n = (m >> 1) == 2 ? 0x7BFF : ((m >> 1) == 1 ? 3000 : 20000);
            bad = run_parallel(fp8_worker, n, T, m, &cases);
            fail |= report(names[m], bad, cases);
        }
    } else {
        return 2;
    }
    return fail;
}
