/*
 * rcodec_oracle.c -- plain, slow CPU oracle of the inline-compression codec.
 *
 * TEST INFRASTRUCTURE ONLY (see rcodec_oracle.h).  Build with
 *   gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * so that every float operation below is one correctly rounded IEEE binary32
 * (or binary64) operation, with nothing fused.
 *
 * Style: every rounding decision is taken by an exact comparison written out
 * in double precision, with a comment saying why the double arithmetic is
 * exact.  Nothing here is blocked, fused or reordered for speed.
 *
 * Layout of one 2048-element tile (32-element blocks b = 0..63; element i of
 * the tile lies in block i/32 at position e = i%32):
 *
 * INT codes: magnitude = the integer nearest to the exact quotient |v| / s,
 * ties to even, clamped to qmax.
 *
 *   INT4 (1152 B):  nibble i of bytes [0,1024) (low nibble first) holds
 *                   (sign << 3) | magnitude, magnitude 0..7;
 *                   fp16 scale of block b at 1024 + 2b.
 *   INT3 (896 B):   q2w plane = bytes [0,512): magnitude (2 bits) of element
 *                   e of block b at bit 64b + 32*((e/2)%2) + 4*((e/2)/2) +
 *                   2*(e%2); q1w plane = bytes [512,768): sign of tile element
 *                   i at bit i; fp16 scale of block b at 768 + 2b.
 *   FP8 (2304 B):   E4M3 / E5M2 codes in two planes: element e < 16 of the
 *                   32-element group g at byte 16g + e, element e >= 16 at
 *                   1024 + 16g + (e - 16); fp32 scale of block b at 2048 + 4b.
 *   MXFP4 (1088 B): nibble i of bytes [0,1024) = E2M1 code;
 *                   E8M0 scale byte of block b at 1024 + b.
 * All planes are little-endian bit streams (bit j of a plane is bit j%8 of
 * its byte j/8).  Positions of the tail tile beyond n hold +0.
 */
#include "rcodec_oracle.h"

#include <float.h>
#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* sizes                                                               */
/* ------------------------------------------------------------------ */

static int is_fp8(int f) { return f == RCO_FMT_FP8_E4M3 || f == RCO_FMT_FP8_E5M2; }
static int is_int(int f) { return f == RCO_FMT_INT4 || f == RCO_FMT_INT3; }

static int codec_ok(rco_codec c)
{
    if (c.block != 16 && c.block != 32 && c.block != 64) return 0;
    if (is_int(c.format)) return c.scale == RCO_SCALE_FP16 || c.scale == RCO_SCALE_E8M0;
    if (is_fp8(c.format))
        return c.scale == RCO_SCALE_FP32 || c.scale == RCO_SCALE_FP16 || c.scale == RCO_SCALE_E8M0;
    if (c.format == RCO_FMT_MXFP4) return c.scale == RCO_SCALE_E8M0;
    return 0;
}

/* Bytes of the code region of a 2048-element tile: 4 bits per element for
 * INT4 and E2M1, 2 + 1 bits for INT3 (q2w and q1w planes), 8 bits for FP8. */
static size_t code_bytes(int format)
{
    switch (format) {
    case RCO_FMT_INT4: case RCO_FMT_MXFP4: return 1024;
    case RCO_FMT_INT3:                     return 768;
    default:                               return 2048;
    }
}

static size_t scale_size(int scale)
{
    return scale == RCO_SCALE_FP16 ? 2 : (scale == RCO_SCALE_FP32 ? 4 : 1);
}

/* Tile = code region + 2048/block scales.  The defaults give 1024 code bytes
 * + 64 fp16 scales = 1152 B for INT4 and 512 + 256 code bytes + 128 = 896 B
 * for INT3, the two sizes printed on "QuickReduce INT3 Quantization and
 * Benchmarking on MI355" (Summary); FP8: 2048 + 64 fp32 scales; MXFP4:
 * 1024 + 64 E8M0 bytes. */
size_t rco_tile_bytes(rco_codec c)
{
    if (!codec_ok(c)) return 0;
    return code_bytes(c.format) + (size_t)(RCO_TILE_ELEMS / c.block) * scale_size(c.scale);
}

size_t rco_packed_bytes(rco_codec c, size_t n)
{
    return ((n + RCO_TILE_ELEMS - 1) / RCO_TILE_ELEMS) * rco_tile_bytes(c);
}

/* ------------------------------------------------------------------ */
/* binary16 / bfloat16 conversions, written from the IEEE definitions  */
/* ------------------------------------------------------------------ */

float rco_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

float rco_f16_to_f32(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)       v = ldexp((double)m, -24);              /* subnormal */
    else if (e == 31) v = m ? NAN : INFINITY;
    else              v = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -v : v);                               /* exact */
}

/* Round |x| to a significand of p bits (p-1 stored) with exponent range
 * [emin, emax], ties to even; returns the biased pattern without sign,
 * or the infinity pattern on overflow.  a*2^(p-1-E) is an exact power-of-two
 * scaling of a double, and nearbyint() rounds it to an integer with ties to
 * even (default rounding mode), which is the definition of RNE. */
static uint32_t round_to_format(double a, int p, int emin, int emax, int bias,
                                uint32_t inf_pattern)
{
    int ex;
    if (a == 0.0) return 0;
    frexp(a, &ex);                 /* a = f*2^ex, f in [0.5,1) */
    int E = ex - 1;                /* 2^E <= a < 2^(E+1)      */
    if (E < emin) E = emin;        /* subnormal quantum 2^(emin-p+1) */
    double q = nearbyint(ldexp(a, p - 1 - E));
    double one = ldexp(1.0, p - 1);
    if (q >= 2.0 * one) { q *= 0.5; E += 1; }   /* carried into next binade */
    if (E > emax) return inf_pattern;
    if (q < one) return (uint32_t)q;            /* subnormal (E == emin)   */
    return ((uint32_t)(E + bias) << (p - 1)) | (uint32_t)(q - one);
}

uint16_t rco_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return sign | 0x7E00;
    if (isinf(x)) return sign | 0x7C00;
    return sign | (uint16_t)round_to_format(fabs((double)x), 11, -14, 15, 15, 0x7C00);
}

uint16_t rco_f32_to_bf16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return sign | 0x7FC0;
    if (isinf(x)) return sign | 0x7F80;
    return sign | (uint16_t)round_to_format(fabs((double)x), 8, -126, 127, 127, 0x7F80);
}

/* ------------------------------------------------------------------ */
/* narrow element formats                                              */
/* ------------------------------------------------------------------ */

/* OCP E4M3: bias 7, no infinities, the one NaN mantissa pattern is S.1111.111
 * ("FP8 Formats for Deep Learning", abstract).  Largest finite = 448. */
float rco_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else        v = ldexp((double)(8 + m), e - 10);
    return (float)(s ? -v : v);
}

/* E2M1 (the MXFP4 element): 1 sign, 2 exponent (bias 1), 1 mantissa bit;
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN. */
float rco_e2m1_decode(uint8_t n)
{
    int s = (n >> 3) & 1, e = (n >> 1) & 3, m = n & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(s ? -v : v);
}

/* E5M2: bias 15, IEEE conventions for special values (exponent 31: infinity
 * with a zero mantissa, NaN otherwise) ("FP8 Formats for Deep Learning",
 * abstract).  Largest finite = 1.75 * 2^15 = 57344 (code 0x7B). */
float rco_e5m2_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -16);
    else v = ldexp((double)(4 + m), e - 17);
    return (float)(s ? -v : v);
}

/* E8M0 shared scale (MX): value 2^(byte-127); 0xFF is NaN. */
float rco_e8m0_decode(uint8_t b)
{
    if (b == 0xFF) return NAN;
    return (float)ldexp(1.0, (int)b - 127);
}

/* Nearest entry of an increasing table of magnitudes val[0..cnt) to num/den
 * (num >= 0, den > 0), ties to the even index, values beyond the last entry
 * saturating to it.  Comparisons are exact: num and den are doubles holding
 * binary32 values, every val[] and every midpoint of neighbours has at most
 * 6 significant bits, so mid*den has at most 30 significant bits and is exact
 * in binary64. */
static int nearest_of_quotient(const double *val, int cnt, double num, double den)
{
    int lo = 0, hi = cnt - 1;                 /* largest c with val[c]*den <= num */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (val[mid] * den <= num) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    if (c == cnt - 1) return c;               /* saturate */
    double mid = 0.5 * (val[c] + val[c + 1]) * den;
    if (num > mid) return c + 1;
    if (num < mid) return c;
    return (c % 2 == 0) ? c : c + 1;          /* tie: even code */
}

static double e4m3_mag[127];
static double e2m1_mag[8];
static double e5m2_mag[124];

/* Filled once when the library is loaded, before any caller thread runs. */
__attribute__((constructor)) static void init_tables(void)
{
    for (int c = 0; c < 127; ++c) e4m3_mag[c] = rco_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 8; ++c)   e2m1_mag[c] = rco_e2m1_decode((uint8_t)c);
    for (int c = 0; c < 124; ++c) e5m2_mag[c] = rco_e5m2_decode((uint8_t)c);
}

/* E4M3 magnitude code of the exact quotient num/den, round to nearest even,
 * saturating at 448 (code 0x7E). */
int rco_e4m3_mag_of_quotient(double num, double den)
{
    return nearest_of_quotient(e4m3_mag, 127, num, den);
}

/* E5M2 magnitude code of the exact quotient num/den, round to nearest even,
 * saturating at 57344 (code 0x7B): finite data never encodes to infinity. */
int rco_e5m2_mag_of_quotient(double num, double den)
{
    return nearest_of_quotient(e5m2_mag, 124, num, den);
}

/* E2M1 magnitude code of an exact value, round to nearest even, saturating
 * at 6 (code 7). */
int rco_e2m1_mag_of(double y_abs)
{
    return nearest_of_quotient(e2m1_mag, 8, y_abs, 1.0);
}

/* Symmetric integer magnitude ("symmetric quantization" with a block-level
 * FP16 scale, QuickReduce INT3 Quantization and Benchmarking on MI355 --
 * Method): the integer nearest to the exact quotient v_abs / s, ties to the
 * even integer, clamped to qmax.  Written with products instead of the
 * quotient: m * s and (m + 1/2) * s have at most 4 + 11 significant bits (s
 * is an fp16 value, m <= 8), so every product below is exact in binary64 and
 * every comparison with v_abs (a binary32 value) is exact. */
int rco_int_mag(float v_abs, float s, int qmax)
{
    const double x = v_abs, sd = s;
    if (!(x < (qmax + 0.5) * sd)) return qmax;          /* clamp (NaN: qmax) */
    int m = 0;                                          /* m = floor(x / s)  */
    while ((m + 1) * sd <= x) ++m;
    const double mid = (m + 0.5) * sd;
    if (x > mid) return m + 1;
    if (x < mid) return m;
    return (m % 2 == 0) ? m : m + 1;                    /* tie: even integer */
}

/* ------------------------------------------------------------------ */
/* block scale rules                                                   */
/* ------------------------------------------------------------------ */

/* FP16 block scale: the block absmax over qmax, one IEEE binary32 division,
 * clamped to the largest half and rounded to fp16 (RNE; subnormal halves
 * kept).  QuickReduce INT3 ... -- Method ("block-level FP16 scale"). */
uint16_t rco_int_scale_bits(float amax, int qmax)
{
    float s32 = amax / (float)qmax;
    if (s32 > 65504.0f) s32 = 65504.0f;
    return rco_f32_to_f16(s32);
}

/* FP32 block scale for FP8: absmax/448 in binary32, so the block maximum maps
 * to the largest E4M3 magnitude; scales below FLT_MIN are flushed to 0 and the
 * block is then stored as zeros.  RCCLX ... -- Low-Precision Collectives
 * (FP8 with computation in FP32). */
float rco_fp8_scale(float amax)
{
    float s = amax / 448.0f;
    return (s < FLT_MIN) ? 0.0f : s;
}

/* Largest exponent of an element format, the offset of the MX shared
 * exponent: E2M1 2 (6 = 1.5 * 2^2), E4M3 8 (448 = 1.75 * 2^8), E5M2 15
 * (57344 = 1.75 * 2^15); for the integer formats floor(log2 qmax): INT4 2
 * (7), INT3 1 (3).  "Microscaling Data Formats for Deep Learning" (abstract:
 * a per-block scaling factor over narrow floating-point and integer types). */
int rco_elem_emax(int format)
{
    switch (format) {
    case RCO_FMT_INT4:     return 2;
    case RCO_FMT_INT3:     return 1;
    case RCO_FMT_FP8_E4M3: return 8;
    case RCO_FMT_FP8_E5M2: return 15;
    default:               return 2;
    }
}

/* MX shared exponent: floor(log2(absmax)) minus the element format's largest
 * exponent, clamped to the E8M0 range; a zero block uses the smallest
 * scale. */
int rco_e8m0_exponent(float amax, int emax)
{
    int ex;
    if (amax == 0.0f) return -127;
    frexp((double)amax, &ex);            /* exact for binary32 subnormals too */
    int e = (ex - 1) - emax;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

int rco_mx_exponent(float amax)
{
    return rco_e8m0_exponent(amax, 2);
}

static float fp8_max(int format)
{
    return format == RCO_FMT_FP8_E5M2 ? 57344.0f : 448.0f;
}

/* FP32 block scale of either FP8 encoding: the RCCLX rule of rco_fp8_scale
 * with the encoding's largest magnitude. */
float rco_fp8_scale_f32(float amax, int format)
{
    float s = amax / fp8_max(format);
    return (s < FLT_MIN) ? 0.0f : s;
}

/* FP16 block scale of an FP8 encoding: amax over the largest magnitude in
 * binary32, clamped to the largest half, then rounded to fp16 (the INT rule
 * with the FP8 maximum in place of qmax). */
uint16_t rco_fp8_scale_f16_bits(float amax, int format)
{
    float s32 = amax / fp8_max(format);
    if (s32 > 65504.0f) s32 = 65504.0f;
    return rco_f32_to_f16(s32);
}

/* ------------------------------------------------------------------ */
/* bit planes                                                          */
/* ------------------------------------------------------------------ */

static void put_bits(uint8_t *plane, size_t pos, unsigned val, int width)
{
    for (int j = 0; j < width; ++j) {
        size_t p = pos + (size_t)j;
        if ((val >> j) & 1u) plane[p / 8] |= (uint8_t)(1u << (p % 8));
        else                 plane[p / 8] &= (uint8_t)~(1u << (p % 8));
    }
}

static unsigned get_bits(const uint8_t *plane, size_t pos, int width)
{
    unsigned v = 0;
    for (int j = 0; j < width; ++j) {
        size_t p = pos + (size_t)j;
        v |= (unsigned)((plane[p / 8] >> (p % 8)) & 1u) << j;
    }
    return v;
}

/* Bit position, inside the q2w plane of a tile, of the 2-bit magnitude of
 * element e of 32-element group g (tile element 32g + e; the groups do not
 * depend on the scale block size).  The group's 16 element pairs (2p, 2p+1)
 * are dealt alternately to its two 32-bit words: pair p goes to word p%2,
 * nibble p/2, the even element of the pair in the nibble's low two bits. */
static size_t int3_q2w_pos(int g, int e)
{
    int p = e / 2;
    return (size_t)64 * g + 32 * (p % 2) + 4 * (p / 2) + 2 * (e % 2);
}

static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void put_f32(uint8_t *p, float f) { memcpy(p, &f, 4); }
static float get_f32(const uint8_t *p) { float f; memcpy(&f, p, 4); return f; }

/* ------------------------------------------------------------------ */
/* tile encode / decode                                                */
/* ------------------------------------------------------------------ */

static float widen(int dt, const void *in, size_t i)
{
    if (dt == RCO_DT_FP32) return ((const float *)in)[i];
    if (dt == RCO_DT_FP16) return rco_f16_to_f32(((const uint16_t *)in)[i]);
    return rco_bf16_to_f32(((const uint16_t *)in)[i]);
}

static float block_absmax(const float *v, int len)
{
    float a = 0.0f;
    for (int e = 0; e < len; ++e) {
        float m = fabsf(v[e]);
        if (m > a) a = m;
    }
    return a;
}

/* Nearest integer to the exact value y >= 0 (a binary32 value scaled by a
 * power of two, held exactly in a double), ties to even, clamped to qmax. */
static int int_mag_exact(double y, int qmax)
{
    if (!(y < qmax + 0.5)) return qmax;                /* NaN: qmax */
    double k = floor(y), frac = y - k;        /* both exact */
    int m = (int)k;
    if (frac > 0.5 || (frac == 0.5 && m % 2 == 1)) m += 1;
    return m > qmax ? qmax : m;
}

/* Byte offset of element i's FP8 code in the tile's code region.  The pages
 * leave the byte order open; it is fixed as two 1024-byte planes: the first
 * 16 codes of each 32-element group g (tile elements 32g .. 32g+15, whatever
 * the block size) at bytes 16g .., the last 16 at 1024 + 16g .., each in
 * element order. */
static size_t fp8_code_pos(size_t i)
{
    const size_t g = i / 32, e = i % 32;
    return e < 16 ? 16 * g + e : 1024 + 16 * g + (e - 16);
}

static void put_code(rco_codec c, uint8_t *dst, size_t i, unsigned sign, unsigned mag)
{
    switch (c.format) {
    case RCO_FMT_INT4: case RCO_FMT_MXFP4:
        put_bits(dst, 4 * i, (sign << 3) | mag, 4);
        break;
    case RCO_FMT_INT3:
        put_bits(dst, int3_q2w_pos((int)(i / 32), (int)(i % 32)), mag, 2);
        put_bits(dst + 512, i, sign, 1);
        break;
    default:
        dst[fp8_code_pos(i)] = (uint8_t)((sign << 7) | mag);
    }
}

/* Encode the 2048 binary32 values v[] of one tile into dst (tile bytes):
 * per block, the scale by the codec's scale rule, then every element's
 * code.  A block whose FP16 or FP32 scale is 0 stays all-zero bytes; E8M0
 * blocks always keep the element signs. */
static void encode_tile(rco_codec c, const float *v, uint8_t *dst)
{
    const size_t tb = rco_tile_bytes(c), cb = code_bytes(c.format);
    const int B = c.block, nb = RCO_TILE_ELEMS / B;
    memset(dst, 0, tb);
    for (int b = 0; b < nb; ++b) {
        const float *vb = v + (size_t)B * b;
        const float amax = block_absmax(vb, B);
        uint8_t *sdst = dst + cb + (size_t)b * scale_size(c.scale);
        if (is_int(c.format)) {
            const int qmax = (c.format == RCO_FMT_INT4) ? 7 : 3;
            if (c.scale == RCO_SCALE_FP16) {
                uint16_t h = rco_int_scale_bits(amax, qmax);
                float sc = rco_f16_to_f32(h);
                if (sc == 0.0f) continue;                 /* zero block: all bytes 0 */
                put_u16(sdst, h);
                for (int e = 0; e < B; ++e)
                    put_code(c, dst, (size_t)B * b + e, signbit(vb[e]) ? 1u : 0u,
                             (unsigned)rco_int_mag(fabsf(vb[e]), sc, qmax));
            } else {                                       /* E8M0: S = 2^ex */
                int ex = rco_e8m0_exponent(amax, rco_elem_emax(c.format));
                sdst[0] = (uint8_t)(ex + 127);
                for (int e = 0; e < B; ++e)
                    put_code(c, dst, (size_t)B * b + e, signbit(vb[e]) ? 1u : 0u,
                             (unsigned)int_mag_exact(ldexp(fabs((double)vb[e]), -ex), qmax));
            }
        } else if (is_fp8(c.format)) {
            int (*mag_of)(double, double) = (c.format == RCO_FMT_FP8_E5M2)
                                                ? rco_e5m2_mag_of_quotient : rco_e4m3_mag_of_quotient;
            double den;
            if (c.scale == RCO_SCALE_FP32) {
                float sc = rco_fp8_scale_f32(amax, c.format);
                if (sc == 0.0f) continue;
                put_f32(sdst, sc);
                den = sc;
            } else if (c.scale == RCO_SCALE_FP16) {
                uint16_t h = rco_fp8_scale_f16_bits(amax, c.format);
                float sc = rco_f16_to_f32(h);
                if (sc == 0.0f) continue;
                put_u16(sdst, h);
                den = sc;
            } else {
                int ex = rco_e8m0_exponent(amax, rco_elem_emax(c.format));
                sdst[0] = (uint8_t)(ex + 127);
                den = ldexp(1.0, ex);                      /* exact */
            }
            for (int e = 0; e < B; ++e)
                put_code(c, dst, (size_t)B * b + e, signbit(vb[e]) ? 1u : 0u,
                         (unsigned)mag_of(fabs((double)vb[e]), den));
        } else { /* MXFP4: E2M1 elements, E8M0 scale */
            int ex = rco_e8m0_exponent(amax, 2);
            sdst[0] = (uint8_t)(ex + 127);
            for (int e = 0; e < B; ++e) {
                double y = ldexp(fabs((double)vb[e]), -ex);        /* exact */
                put_code(c, dst, (size_t)B * b + e, signbit(vb[e]) ? 1u : 0u, (unsigned)rco_e2m1_mag_of(y));
            }
        }
    }
}

/* Decode element i (0..2047) of one tile to binary32.  Every product of a
 * code value and an FP16 or E8M0 scale is exact in binary32 (at most 15
 * significant bits, no underflow below 2^-149), so the double product
 * rounds to itself; the FP8 x FP32-scale product is one binary32
 * multiplication. */
static float decode_elem(rco_codec c, const uint8_t *src, int i)
{
    const int b = i / c.block;
    const uint8_t *sp = src + code_bytes(c.format) + (size_t)b * scale_size(c.scale);
    double val;                                   /* code value, exact */
    switch (c.format) {
    case RCO_FMT_INT4: {
        unsigned nib = get_bits(src, 4 * (size_t)i, 4);
        val = (nib & 8u) ? -(double)(nib & 7u) : (double)(nib & 7u);
        if ((nib & 8u) && (nib & 7u) == 0) val = -0.0;
        break;
    }
    case RCO_FMT_INT3: {
        unsigned mag = get_bits(src, int3_q2w_pos(i / 32, i % 32), 2);
        unsigned sign = get_bits(src + 512, (size_t)i, 1);
        val = sign ? -(double)mag : (double)mag;
        break;
    }
    case RCO_FMT_FP8_E4M3: val = rco_e4m3_decode(src[fp8_code_pos((size_t)i)]); break;
    case RCO_FMT_FP8_E5M2: val = rco_e5m2_decode(src[fp8_code_pos((size_t)i)]); break;
    default: val = rco_e2m1_decode((uint8_t)get_bits(src, 4 * (size_t)i, 4));
    }
    if (c.scale == RCO_SCALE_FP32) return (float)val * get_f32(sp);       /* RN32 */
    if (c.scale == RCO_SCALE_FP16) return (float)(val * rco_f16_to_f32(get_u16(sp)));
    if (sp[0] == 0xFF) return NAN;
    return (float)ldexp(val, (int)sp[0] - 127);
}

/* ------------------------------------------------------------------ */
/* public operations                                                   */
/* ------------------------------------------------------------------ */

static int dtype_ok(int dt)
{
    return dt == RCO_DT_FP32 || dt == RCO_DT_FP16 || dt == RCO_DT_BF16;
}

int rco_quantize_pack_tiles(rco_codec c, int in_dtype, const void *in, size_t n,
                            void *out, size_t t0, size_t t1)
{
    if (!codec_ok(c) || !dtype_ok(in_dtype)) return RCO_ERR_UNSUPPORTED;
    if (n == 0) return RCO_OK;
    if (!in || !out) return RCO_ERR_NULL;
    size_t tb = rco_tile_bytes(c);
    float v[RCO_TILE_ELEMS];
    for (size_t t = t0; t < t1; ++t) {
        for (int j = 0; j < RCO_TILE_ELEMS; ++j) {
            size_t i = t * RCO_TILE_ELEMS + (size_t)j;
            v[j] = (i < n) ? widen(in_dtype, in, i) : 0.0f;
        }
        encode_tile(c, v, (uint8_t *)out + t * tb);
    }
    return RCO_OK;
}

int rco_quantize_pack(rco_codec c, int in_dtype, const void *in, size_t n, void *out)
{
    size_t tiles = (n + RCO_TILE_ELEMS - 1) / RCO_TILE_ELEMS;
    return rco_quantize_pack_tiles(c, in_dtype, in, n, out, 0, tiles);
}

int rco_unpack_dequant(rco_codec c, const void *in, size_t n, int out_dtype, void *out)
{
    if (!codec_ok(c) || !dtype_ok(out_dtype)) return RCO_ERR_UNSUPPORTED;
    if (n == 0) return RCO_OK;
    if (!in || !out) return RCO_ERR_NULL;
    size_t tb = rco_tile_bytes(c);
    for (size_t i = 0; i < n; ++i) {
        const uint8_t *tile = (const uint8_t *)in + (i / RCO_TILE_ELEMS) * tb;
        float d = decode_elem(c, tile, (int)(i % RCO_TILE_ELEMS));
        if (out_dtype == RCO_DT_FP32)      ((float *)out)[i] = d;
        else if (out_dtype == RCO_DT_FP16) ((uint16_t *)out)[i] = rco_f32_to_f16(d);
        else                               ((uint16_t *)out)[i] = rco_f32_to_bf16(d);
    }
    return RCO_OK;
}

/* acc = d_0, then acc = RN32(acc + d_k) for k = 1..K-1 in stream order
 * (RCCLX ... -- Low-Precision Collectives: computation stays in FP32), then
 * the sums are requantized with the same codec.  Positions beyond n are +0
 * whatever the input codes there say. */
int rco_dequant_reduce_requant_tiles(rco_codec c, const void *const *ins, int k,
                                     size_t n, void *out, float *sum_out,
                                     size_t t0, size_t t1)
{
    if (!codec_ok(c)) return RCO_ERR_UNSUPPORTED;
    if (k < 1 || k > RCO_MAX_STREAMS) return RCO_ERR_RANGE;
    if (n == 0) return RCO_OK;
    if (!ins || !out) return RCO_ERR_NULL;
    for (int s = 0; s < k; ++s) if (!ins[s]) return RCO_ERR_NULL;
    size_t tb = rco_tile_bytes(c);
    float acc[RCO_TILE_ELEMS];
    for (size_t t = t0; t < t1; ++t) {
        for (int j = 0; j < RCO_TILE_ELEMS; ++j) {
            size_t i = t * RCO_TILE_ELEMS + (size_t)j;
            if (i >= n) { acc[j] = 0.0f; continue; }
            float a = decode_elem(c, (const uint8_t *)ins[0] + t * tb, j);
            for (int s = 1; s < k; ++s)
                a = a + decode_elem(c, (const uint8_t *)ins[s] + t * tb, j);
            acc[j] = a;
            if (sum_out) sum_out[i] = a;
        }
        encode_tile(c, acc, (uint8_t *)out + t * tb);
    }
    return RCO_OK;
}

int rco_dequant_reduce_requant(rco_codec c, const void *const *ins, int k, size_t n,
                               void *out, float *sum_out)
{
    size_t tiles = (n + RCO_TILE_ELEMS - 1) / RCO_TILE_ELEMS;
    return rco_dequant_reduce_requant_tiles(c, ins, k, n, out, sum_out, 0, tiles);
}

/* ------------------------------------------------------------------ */
/* element-wise loops (pins)                                           */
/* ------------------------------------------------------------------ */

void rco_map_f32_to_f16(const float *x, uint16_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_f32_to_f16(x[i]); }
void rco_map_f32_to_bf16(const float *x, uint16_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_f32_to_bf16(x[i]); }
void rco_map_f16_to_f32(const uint16_t *x, float *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_f16_to_f32(x[i]); }
void rco_map_bf16_to_f32(const uint16_t *x, float *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_bf16_to_f32(x[i]); }
void rco_map_e4m3_mag(const double *num, const double *den, int32_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_e4m3_mag_of_quotient(num[i], den[i]); }
void rco_map_e2m1_mag(const double *v, int32_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_e2m1_mag_of(v[i]); }
void rco_map_int_mag(const float *v_abs, const float *s, int qmax, int32_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_int_mag(v_abs[i], s[i], qmax); }
void rco_map_int_scale_bits(const float *amax, int qmax, uint16_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_int_scale_bits(amax[i], qmax); }
void rco_map_fp8_scale(const float *amax, float *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_fp8_scale(amax[i]); }
void rco_map_mx_exponent(const float *amax, int32_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_mx_exponent(amax[i]); }
void rco_map_e5m2_mag(const double *num, const double *den, int32_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_e5m2_mag_of_quotient(num[i], den[i]); }
void rco_map_e8m0_exponent(const float *amax, int emax, int32_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_e8m0_exponent(amax[i], emax); }
void rco_map_fp8_scale_f16_bits(const float *amax, int format, uint16_t *y, size_t n)
{ for (size_t i = 0; i < n; ++i) y[i] = rco_fp8_scale_f16_bits(amax[i], format); }
