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
 *   fp8narrow  inputs of at most 11 significant bits (bf16, fp16): every
 *            pair x <= a (a the block maximum), FP32 and FP16 scales, both
 *            formats, both reciprocal neighbours.  Where the bracket is
 *            undecided the code follows the block rule (FP32 scale: upper
 *            code when a - s fmax > 0, lower when < 0, even when 0; FP16
 *            scale: even) and equals the exact code.
 *   fp8      two stages.  The bracket: x times the hardware reciprocal
 *            rounded down and up by 2^-21 (clamped with FP16 scales), both
 *            products converted; where the codes agree that is the code.
 *            Else (and for scales below 2^-64) the round-to-odd quotient
 *            sequence (y1 = fma(|x|, rs, |x| rl) with rl = fma(-s, rs, 1) rs,
 *            side from the sign bit of fma(-y1, s, |x|), then round-to-odd,
 *            clamp with FP16 scales) followed by the RNE conversion to E4M3
 *            / E5M2.  Together equal to the RNE code of the exact quotient,
 *            for binary32 x within 16 ulp of every rounding midpoint (and of
 *            the saturation point), random x up to the block maximum and in
 *            the subnormal range, x far into saturation (FP16 scales), over
 *            random FP32 scales up to 2^119, scales below 2^-64 (x and s
 *            times 2^64), and every fp16 scale, with rs either binary32
 *            neighbour of 1/s.  No product converted by the bracket may lie
 *            beyond the format's finite range.
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

/* the kernel's round-to-odd quotient of |x| / s (sign dropped: x >= 0): the
 * quotient from the hardware reciprocal rs and its low part rl =
 * fma(-s, rs, 1) rs, the exact residual's sign bit steps it down one binary32
 * value, and an inexact result gets its last bit set */
static float ro_quotient(float ax, float s, float rs, float fmax, int clamp)
{
    const float rl = fmaf(-s, rs, 1.0f) * rs;
    const float y1 = fmaf(ax, rs, ax * rl);
    const float r = fmaf(-y1, s, ax);
    const uint32_t rb = f2u(r);
    uint32_t t = f2u(y1) - (rb >> 31);
    t |= rb < 1u ? rb : 1u;
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

/* how often the bracket gave one code or fell back (per thread, summed at
 * the end of each worker) */
static _Thread_local unsigned long long fp8_fast_hits, fp8_fallbacks;
static _Atomic unsigned long long fp8_fast_total, fp8_fallback_total;

/* kernel: first the bracket, x times the reciprocal rounded down and up by
 * 2^-21 (clamped to the largest magnitude with FP16 scales); when both
 * products convert to one code that is the code.  Otherwise, and for scales
 * below 2^-64, the round-to-odd quotient (x and s below 2^-64 multiplied by
 * 2^64 first).  A product whose conversion leaves the finite range is a
 * failure: the kernel must never convert it. */
static int fp8_device(float x, float s, int which_rcp, int e5, int clamp)
{
    const float fmax = e5 ? 57344.0f : 448.0f;
    float c[2];
    if (s >= 0x1p-64f) {
        const int nc = rcp_candidates(s, c);
        const float rs = c[which_rcp < nc ? which_rcp : 0];
        const float rlo = rs * 0x1.fffffp-1f, rhi = rs * 0x1.000008p0f;
        float a = x * rlo, b = x * rhi;
        if (clamp) { a = fminf(a, fmax); b = fminf(b, fmax); }
        const int ca = fp8_convert(a, e5), cb = fp8_convert(b, e5);
        if (ca < 0 || cb < 0) return -2;
        if (ca == cb) { fp8_fast_hits++; return ca; }
        fp8_fallbacks++;
    }
    float kx = x, ks = s;
    if (s < 0x1p-64f) { kx = x * 0x1p64f; ks = s * 0x1p64f; }
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
    /* random magnitudes up to the block maximum (mostly decided by the
     * bracket), and tiny ones in the format's subnormal range */
    for (int i = 0; i < 64; ++i) {
        const uint64_t r = splitmix(&j->seed);
        const double u = (double)(r >> 11) * 0x1p-53;
        const double target = (i & 1 ? tab[cnt - 1] * u : tab[3] * u * 4.0) * (double)s;
        if (target > 3.0e38) continue;
        const float x = (float)target;
        const int want = fp8_exact(x, s, e5);
        for (int w = 0; w < 2; ++w) {
            j->cases++;
            if (fp8_device(x, s, w, e5, clamp) != want) j->bad++;
        }
    }
    /* FP16 scales (subnormal, or clamped at 65504) leave quotients far above
     * the largest magnitude: they saturate, up to the largest binary32 x */
    if (!clamp) return;
    for (int k = 1; k < 300; ++k) {
        const double target = tab[cnt - 1] * (double)s * ldexp(1.0, k);
        if (target > 3.0e38) break;
        float x = (float)target;
        for (int i = 0; i < 4; ++i) x = nextafterf(x, 0.0f);
        for (int i = 0; i <= 8; ++i, x = nextafterf(x, INFINITY)) {
            for (int w = 0; w < 2; ++w) {
                j->cases++;
                if (fp8_device(x, s, w, e5, clamp) != cnt - 1) j->bad++;
            }
        }
    }
    for (int w = 0; w < 2; ++w) {
        j->cases++;
        if (fp8_device(3.4028234663852886e38f, s, w, e5, clamp) != cnt - 1) j->bad++;
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
        /* normal scales up to RN32(FLT_MAX / 448) < 2^120 */
        const int ex = mode == 0 ? (int)(r % 184) - 64 : -126 + (int)(r % 62);
        const float s = ldexpf(1.0f + (float)((r >> 8) & 0x7FFFFF) * 0x1p-23f, ex);
        fp8_one_scale(j, s, e5, 0);
    }
    fp8_fast_total += fp8_fast_hits;
    fp8_fallback_total += fp8_fallbacks;
    fp8_fast_hits = fp8_fallbacks = 0;
    return NULL;
}

/* ------------------------------------------------------------ fp8narrow */

/* RNE E4M3 / E5M2 code of a binary32 y >= 0 by bit arithmetic (normal
 * range: carry into the kept mantissa bits, ties to the even one; subnormal
 * range: y times 2^9 (2^16) rounded to an integer by the 2^23 addition);
 * -1 at or above the midpoint past the largest magnitude.  Checked against
 * the table search fp8_convert before use. */
static int fp8_fast_code(float y, int e5)
{
    if (y >= (e5 ? 61440.0f : 464.0f)) return -1;
    const uint32_t u = f2u(y);
    if (y >= (e5 ? 0x1p-14f : 0x1p-6f)) {
        const int sh = e5 ? 21 : 20;
        const uint32_t t = u + ((1u << (sh - 1)) - 1u) + ((u >> sh) & 1u);
        return (int)(t >> sh) - (e5 ? 448 : 960);
    }
    volatile float k = y * (e5 ? 0x1p16f : 0x1p9f);
    volatile float r = (k + 0x1p23f) - 0x1p23f;
    return (int)r;
}

static float narrow_value(uint16_t b, int fp16)
{
    return fp16 ? half_value(b) : u2f((uint32_t)b << 16);
}

/* RN of a binary32 value in [0, 65504] to fp16, as a binary32 value */
static float round_to_half(float v)
{
    double q = (v >= 0x1p-14f) ? ldexp(1.0, (int)floor(log2((double)v)) - 10) : 0x1p-24;
    if (v >= 0x1p-14f && ldexp(1.0, (int)floor(log2((double)v))) > v) q *= 0.5;   /* log2 rounding guard */
    return (float)(nearbyint((double)v / q) * q);
}

/* Inputs of at most 11 significant bits (bf16, fp16): every (x, block
 * maximum a) pair, x <= a.  The bracket's undecided pairs must be exact ties
 * (fmax x = m a with an FP32 scale, x = m s with an FP16 one), resolved per
 * block: FP32 scale by the sign of a - s fmax (s rounded down: the quotient
 * lies above the midpoint), FP16 scale to the even code.  Job arg bits:
 * 0 = fp16 inputs, 1 = E5M2, 2 = FP16 scale. */
static _Atomic unsigned long long narrow_undecided;

static void *fp8narrow_worker(void *p)
{
    job *j = p;
    const int fp16 = j->arg & 1, e5 = (j->arg >> 1) & 1, s16 = (j->arg >> 2) & 1;
    const float fmax = e5 ? 57344.0f : 448.0f;
    unsigned long long und = 0;
    for (uint64_t ai = j->lo; ai < j->hi; ++ai) {
        const uint16_t ab = (uint16_t)(ai + 1);
        const float a = narrow_value(ab, fp16);
        float sc, dir;
        if (!s16) {
            sc = a / fmax;
            if (!(sc >= 0x1p-64f)) continue;     /* zero block, or the 2^64 path */
            dir = fmaf(-sc, fmax, a);
        } else {
            sc = round_to_half(fminf(a / fmax, 65504.0f));
            if (sc == 0.0f) continue;
            dir = 0.0f;
        }
        float c[2];
        const int nc = rcp_candidates(sc, c);
        for (int w = 0; w < nc; ++w) {
            const float rlo = c[w] * 0x1.fffffp-1f, rhi = c[w] * 0x1.000008p0f;
            for (uint32_t xb = 0; xb <= ab; ++xb) {
                const float x = narrow_value((uint16_t)xb, fp16);
                float lo = x * rlo, hi = x * rhi;
                if (s16) { lo = fminf(lo, fmax); hi = fminf(hi, fmax); }
                const int cl = fp8_fast_code(lo, e5), ch = fp8_fast_code(hi, e5);
                j->cases++;
                if (cl < 0 || ch < 0) { j->bad++; continue; }
                int code = cl;
                if (cl != ch) {
                    und++;
                    if (ch != cl + 1) { j->bad++; continue; }
                    code = dir > 0.0f ? ch : (dir < 0.0f ? cl : ((cl & 1) ? ch : cl));
                } else if ((xb & 63u) != 7u) {
                    continue;                     /* decided: the enclosure check covers it; sample 1/64 */
                }
                if (code != fp8_exact(x, sc, e5)) j->bad++;
            }
        }
    }
    narrow_undecided += und;
    return NULL;
}

/* the table search, out of range (-1) from the midpoint past the largest
 * magnitude on: 464 for E4M3, whose next code point is NaN */
static int fast_code_want(float y, int e5)
{
    return y >= (e5 ? 61440.0f : 464.0f) ? -1 : fp8_convert(y, e5);
}

/* the bit-arithmetic conversion against the table search */
static uint64_t check_fast_code(uint64_t *cases)
{
    uint64_t bad = 0, seed = 12345;
    *cases = 0;
    for (int e5 = 0; e5 < 2; ++e5) {
        const double *tab = e5 ? e5m2_tab : e4m3_tab;
        const int cnt = e5 ? 124 : 127;
        for (int cc = 0; cc < cnt; ++cc) {                 /* around every code and midpoint */
            const double pts[2] = {tab[cc], cc + 1 < cnt ? 0.5 * (tab[cc] + tab[cc + 1]) : tab[cc] * 1.0625};
            for (int p = 0; p < 2; ++p) {
                float y = (float)pts[p];
                for (int i = 0; i < 8; ++i) y = nextafterf(y, 0.0f);
                for (int i = 0; i <= 16; ++i, y = nextafterf(y, INFINITY)) {
                    ++*cases;
                    if (fp8_fast_code(y, e5) != fast_code_want(y, e5)) ++bad;
                }
            }
        }
        for (int i = 0; i < 4000000; ++i) {                /* random binary32 below the top */
            const uint64_t r = splitmix(&seed);
            const float y = u2f((uint32_t)(r % (f2u(e5 ? 65536.0f : 512.0f))));
            ++*cases;
            if (fp8_fast_code(y, e5) != fast_code_want(y, e5)) ++bad;
        }
    }
    return bad;
}

/* ------------------------------------------------------------------- main */

static int report(const char *name, uint64_t bad, uint64_t cases)
{
    printf("%-28s cases %12llu  differ %llu\n", name, (unsigned long long)cases, (unsigned long long)bad);
    return bad != 0 || cases == 0;
}

int main(int argc, char **argv)
{
    if (argc < 2) { fprintf(stderr, "usage: %s div|recip|int|fp8|fp8narrow [threads]\n", argv[0]); return 2; }
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
        printf("bracket decided %llu, fell back %llu\n", (unsigned long long)fp8_fast_total,
               (unsigned long long)fp8_fallback_total);
    } else if (!strcmp(argv[1], "fp8narrow")) {
        init_tables();
        bad = check_fast_code(&cases);
        fail |= report("fp8 bit-arith conversion", bad, cases);
        static const char *names[8] = {"bf16 e4m3 fp32 scale", "fp16 e4m3 fp32 scale", "bf16 e5m2 fp32 scale",
                                       "fp16 e5m2 fp32 scale", "bf16 e4m3 fp16 scale", "fp16 e4m3 fp16 scale",
                                       "bf16 e5m2 fp16 scale", "fp16 e5m2 fp16 scale"};
        for (int m = 0; m < 8; ++m) {
            const uint64_t n = (m & 1) ? 0x7BFF : 0x7F7F;     /* positive finite maxima */
            bad = run_parallel(fp8narrow_worker, n, T, m, &cases);
            fail |= report(names[m], bad, cases);
        }
        printf("undecided pairs resolved per block %llu\n", (unsigned long long)narrow_undecided);
        fail |= narrow_undecided == 0;
    } else {
        return 2;
    }
    return fail;
}
