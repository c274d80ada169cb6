/*
 * rcodec_oracle.h -- plain CPU oracle of the inline-compression codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this code: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no source with the HIP library.
 *
 * What it computes (the spec of record, one definition per step):
 *   - block quantization with one scale per 32-element block, symmetric
 *     integer codes (the exact quotient |v| / s rounded half-even) and an
 *     FP16 block scale, the 3-bit codes split into a low-2-bit plane (q2w)
 *     and a high-bit plane (q1w)
 *       [QuickReduce INT3 Quantization and Benchmarking on MI355 -- Method];
 *   - fixed 2048-element tiles that pack to 1152 B (INT4) and 896 B (INT3)
 *       [same page -- Summary];
 *   - FP8 E4M3 codes with an FP32 block scale, FP32 accumulation of the
 *     dequantized streams
 *       [RCCLX: Innovating GPU communications on AMD platforms --
 *        Low-Precision Collectives];
 *   - E4M3 with no infinities and a single NaN mantissa pattern
 *       [FP8 Formats for Deep Learning -- abstract];
 *   - MX blocks: a shared power-of-two scale over narrow floating-point
 *     and integer elements, and the MXFP4 direct cast
 *       [Microscaling Data Formats for Deep Learning -- abstract;
 *        ML-SpecQD: Multi-Level Speculative Decoding with Quantized Drafts];
 *   - E5M2 with IEEE infinities and NaNs, the second FP8 encoding
 *       [FP8 Formats for Deep Learning -- abstract].
 * Codecs are (element format, scale type, block size): INT4 and INT3 with
 * FP16 or E8M0 scales; E4M3 and E5M2 with FP32, FP16 or E8M0 scales; E2M1
 * (MXFP4) with E8M0 scales; blocks of 16, 32 or 64 elements.  The tile is
 * always 2048 elements: the code region, then 2048/block scales.  FP8
 * codes fill the code region as two 1024-byte planes (the first and the
 * last 16 codes of every 32-element group).
 * Every step the pages leave open is fixed once here and listed as a
 * "reading" in the design notes of the repository.
 *
 * All functions take host pointers, run synchronously on one thread and
 * allocate nothing.  Status codes are numerically identical to the GPU
 * library's; a test checks that they agree.
 */
#ifndef RCODEC_ORACLE_H
#define RCODEC_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RCO_TILE_ELEMS 2048
#define RCO_BLOCK_ELEMS 32
#define RCO_MAX_STREAMS 16

enum { RCO_FMT_INT4 = 1, RCO_FMT_INT3 = 2, RCO_FMT_FP8_E4M3 = 3, RCO_FMT_MXFP4 = 4,
       RCO_FMT_FP8_E5M2 = 5 };
enum { RCO_SCALE_FP16 = 1, RCO_SCALE_FP32 = 2, RCO_SCALE_E8M0 = 3 };
enum { RCO_DT_FP32 = 1, RCO_DT_FP16 = 2, RCO_DT_BF16 = 3 };
enum { RCO_OK = 0, RCO_ERR_NULL = 1, RCO_ERR_UNSUPPORTED = 2, RCO_ERR_ALIGN = 3,
       RCO_ERR_RANGE = 4, RCO_ERR_HIP = 5 };

typedef struct { int32_t format, scale, block; } rco_codec;

/* ---- sizes ---------------------------------------------------------- */
size_t rco_tile_bytes(rco_codec c);               /* 0 when unsupported   */
size_t rco_packed_bytes(rco_codec c, size_t n);   /* ceil(n/2048) * tile  */

/* ---- whole-stream operations (host buffers) ------------------------- */
int rco_quantize_pack(rco_codec c, int in_dtype, const void *in, size_t n, void *out);
int rco_unpack_dequant(rco_codec c, const void *in, size_t n, int out_dtype, void *out);
int rco_dequant_reduce_requant(rco_codec c, const void *const *ins, int k, size_t n,
                               void *out, float *sum_out);
/* Same as above, restricted to tiles [t0, t1): used to time the oracle on a
 * bounded sample and to compute sampled outputs of very large streams.
 * Pointers address the whole stream; only the listed tiles are touched.  */
int rco_quantize_pack_tiles(rco_codec c, int in_dtype, const void *in, size_t n,
                            void *out, size_t t0, size_t t1);
int rco_dequant_reduce_requant_tiles(rco_codec c, const void *const *ins, int k,
                                     size_t n, void *out, float *sum_out,
                                     size_t t0, size_t t1);

/* ---- scalar building blocks, exported so the pins can test them ------ */
float    rco_bf16_to_f32(uint16_t h);
uint16_t rco_f32_to_bf16(float x);                /* RNE, IEEE overflow  */
float    rco_f16_to_f32(uint16_t h);
uint16_t rco_f32_to_f16(float x);                 /* RNE, IEEE overflow  */
float    rco_e4m3_decode(uint8_t code);           /* OCP E4M3 ("FN")     */
float    rco_e2m1_decode(uint8_t nibble);
float    rco_e8m0_decode(uint8_t byte);           /* 2^(byte-127), 0xFF NaN */
float    rco_e5m2_decode(uint8_t code);           /* IEEE-style E5M2     */
/* magnitude code of |num|/den rounded to nearest, ties to even code,
 * saturating; num, den exact doubles, den > 0 */
int      rco_e4m3_mag_of_quotient(double num, double den);   /* 0..126 */
int      rco_e2m1_mag_of(double y_abs);                      /* 0..7   */
int      rco_e5m2_mag_of_quotient(double num, double den);   /* 0..123 */
/* INT magnitude: the integer nearest to the exact quotient v_abs / s (s an
 * fp16 value > 0), ties to even, clamped to qmax */
int      rco_int_mag(float v_abs, float s, int qmax);
/* per-block scale rules; amax >= 0 */
uint16_t rco_int_scale_bits(float amax, int qmax);   /* fp16 bits       */
float    rco_fp8_scale(float amax);                  /* E4M3, 0 when flushed */
int      rco_mx_exponent(float amax);                /* E2M1, -127..127 */
/* the same rules for any element format (RCO_FMT_*) */
int      rco_elem_emax(int format);                  /* largest element exponent */
int      rco_e8m0_exponent(float amax, int emax);    /* -127..127       */
float    rco_fp8_scale_f32(float amax, int format);  /* RN32(a/fmax), 0 below FLT_MIN */
uint16_t rco_fp8_scale_f16_bits(float amax, int format); /* fp16(min(RN32(a/fmax), 65504)) */

/* element-wise loops over the scalar rules above (for the pins) */
void rco_map_f32_to_f16(const float *x, uint16_t *y, size_t n);
void rco_map_f32_to_bf16(const float *x, uint16_t *y, size_t n);
void rco_map_f16_to_f32(const uint16_t *x, float *y, size_t n);
void rco_map_bf16_to_f32(const uint16_t *x, float *y, size_t n);
void rco_map_e4m3_mag(const double *num, const double *den, int32_t *y, size_t n);
void rco_map_e2m1_mag(const double *v, int32_t *y, size_t n);
void rco_map_int_mag(const float *v_abs, const float *s, int qmax, int32_t *y, size_t n);
void rco_map_int_scale_bits(const float *amax, int qmax, uint16_t *y, size_t n);
void rco_map_fp8_scale(const float *amax, float *y, size_t n);
void rco_map_mx_exponent(const float *amax, int32_t *y, size_t n);
void rco_map_e5m2_mag(const double *num, const double *den, int32_t *y, size_t n);
void rco_map_e8m0_exponent(const float *amax, int emax, int32_t *y, size_t n);
void rco_map_fp8_scale_f16_bits(const float *amax, int format, uint16_t *y, size_t n);

#ifdef __cplusplus
}
#endif
#endif
