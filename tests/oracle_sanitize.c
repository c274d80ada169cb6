/*
 * Driver for the sanitizer build of the CPU oracle (test infrastructure).
 *
 * Built by tests/test_oracle_sanitize.py together with oracle/rcodec_oracle.c
 * under AddressSanitizer and UndefinedBehaviorSanitizer; every buffer is
 * allocated at exactly the size the oracle's interface states, so a read or
 * write past it, a use of uninitialised scale bytes, an out-of-range shift
 * or float-to-int conversion stops the run.  It calls every operation for
 * every supported codec, every dtype, ragged lengths and 1..3 streams, then
 * the error paths.  Non-finite inputs (whose codes are unspecified) are fed
 * too: they may give any bytes but must not step outside the buffers or
 * into undefined behaviour.  Exit status 0 = clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rcodec_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform(void) { return ((next_u64() >> 11) + 0.5) * 0x1p-53; }

/* per 32-element block: one kind of values, so every scale path is reached */
static void fill_f32(float *v, size_t n, int with_nonfinite)
{
    for (size_t b = 0; b * 32 < n; ++b) {
        const int kind = (int)(next_u64() % (with_nonfinite ? 10 : 8));
        for (size_t i = b * 32; i < n && i < b * 32 + 32; ++i) {
            const double z = sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform());
            float x;
            switch (kind) {
            case 0: x = 0.0f; break;
            case 1: x = (i % 5 == 0) ? -0.0f : 0.0f; break;
            case 2: x = (float)(z * 1e-40); break;                     /* denormals */
            case 3: x = (float)(z * 1e-6); break;
            case 4: x = (float)((double)((int)(next_u64() % 15) - 7) * 0.25); break;   /* grid, ties */
            case 5: x = (float)(z * 3e4); break;
            case 6: x = (float)(z * 1e38); break;                       /* near the top */
            case 8: x = (i % 3 == 0) ? INFINITY : (float)z; break;
            case 9: x = (i % 4 == 0) ? NAN : (float)z; break;
            default: x = (float)z;
            }
            v[i] = x;
        }
    }
}

static void *xmalloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;

static void expect(int cond, const char *what)
{
    if (!cond) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

/* the input of one dtype, exactly n elements */
static void *make_input(const float *v, size_t n, int dt)
{
    if (dt == RCO_DT_FP32) {
        float *p = xmalloc(n * 4);
        memcpy(p, v, n * 4);
        return p;
    }
    uint16_t *p = xmalloc(n * 2);
    for (size_t i = 0; i < n; ++i) p[i] = dt == RCO_DT_BF16 ? rco_f32_to_bf16(v[i]) : rco_f32_to_f16(v[i]);
    return p;
}

static void run_codec(rco_codec c, size_t n, int with_nonfinite)
{
    const size_t pb = rco_packed_bytes(c, n);
    float *v = xmalloc(n * 4);
    uint8_t *packed[3];
    for (int s = 0; s < 3; ++s) {
        fill_f32(v, n, with_nonfinite);
        packed[s] = xmalloc(pb);
        for (int dt = RCO_DT_FP32; dt <= RCO_DT_BF16; ++dt) {
            void *in = make_input(v, n, dt);
            expect(rco_quantize_pack(c, dt, in, n, packed[s]) == RCO_OK, "quantize_pack");
            free(in);
        }
    }
    for (int dt = RCO_DT_FP32; dt <= RCO_DT_BF16; ++dt) {
        void *out = xmalloc(n * (dt == RCO_DT_FP32 ? 4 : 2));
        expect(rco_unpack_dequant(c, packed[0], n, dt, out) == RCO_OK, "unpack_dequant");
        free(out);
    }
    uint8_t *red = xmalloc(pb);
    float *sums = xmalloc(n * 4);
    for (int k = 1; k <= 3; ++k) {
        const void *ins[3] = {packed[0], packed[1], packed[2]};
        expect(rco_dequant_reduce_requant(c, ins, k, n, red, sums) == RCO_OK, "reduce with sums");
        expect(rco_dequant_reduce_requant(c, ins, k, n, red, NULL) == RCO_OK, "reduce");
    }
    /* tile ranges: the last tile alone, and an empty range */
    const size_t tiles = (n + RCO_TILE_ELEMS - 1) / RCO_TILE_ELEMS;
    {
        const void *ins[2] = {packed[1], packed[2]};
        expect(rco_dequant_reduce_requant_tiles(c, ins, 2, n, red, sums, tiles - 1, tiles) == RCO_OK, "reduce tiles");
        expect(rco_dequant_reduce_requant_tiles(c, ins, 2, n, red, NULL, 0, 0) == RCO_OK, "reduce no tiles");
        void *in = make_input(v, n, RCO_DT_BF16);
        expect(rco_quantize_pack_tiles(c, RCO_DT_BF16, in, n, red, tiles - 1, tiles) == RCO_OK, "quantize tiles");
        free(in);
    }
    free(red);
    free(sums);
    for (int s = 0; s < 3; ++s) free(packed[s]);
    free(v);
}

int main(void)
{
    static const size_t lengths[] = {1, 31, 33, 2047, 2048, 2049, 2 * 2048 + 777};
    int codecs = 0;
    for (int f = 1; f <= 5; ++f)
        for (int s = 1; s <= 3; ++s)
            for (int b = 16; b <= 64; b *= 2) {
                rco_codec c = {f, s, b};
                if (rco_tile_bytes(c) == 0) continue;
                ++codecs;
                for (size_t i = 0; i < sizeof lengths / sizeof lengths[0]; ++i) run_codec(c, lengths[i], 0);
                run_codec(c, 2048 + 100, 1);
            }
    expect(codecs == 33, "33 supported codecs");

    /* error paths: nothing is touched, a status comes back */
    rco_codec bad = {RCO_FMT_MXFP4, RCO_SCALE_FP16, 32};
    float one = 1.0f;
    uint8_t sink[1152];
    expect(rco_quantize_pack(bad, RCO_DT_FP32, &one, 1, sink) != RCO_OK, "unsupported codec");
    rco_codec int4 = {RCO_FMT_INT4, RCO_SCALE_FP16, 32};
    expect(rco_quantize_pack(int4, 99, &one, 1, sink) != RCO_OK, "unsupported dtype");
    expect(rco_quantize_pack(int4, RCO_DT_FP32, NULL, 1, sink) != RCO_OK, "null input");
    const void *ins[1] = {sink};
    expect(rco_dequant_reduce_requant(int4, ins, 0, 1, sink, NULL) != RCO_OK, "k = 0");
    expect(rco_dequant_reduce_requant(int4, ins, RCO_MAX_STREAMS + 1, 1, sink, NULL) != RCO_OK, "k too large");

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle sanitizer run clean: %d codecs\n", codecs);
    return 0;
}
