/*
 * rcodec.h -- C ABI of the MI355X (gfx950) inline-compression codec library
 * (librcodec.so).
 *
 * The codec is the compute half of a quantized all-reduce: block-quantize
 * activations into fixed-size tiles before they travel, then on the receiving
 * side dequantize K incoming streams, add them in FP32 and requantize the sum
 * ("QuickReduce INT3 Quantization and Benchmarking on MI355" -- Summary and
 * Method; "RCCLX: Innovating GPU communications on AMD platforms" --
 * Low-Precision Collectives).  This library is that compute on one GPU; it
 * moves no data between GPUs.
 *
 * Data layout (all formats): the stream of n elements is cut into
 * ceil(n/2048) tiles of 2048 elements, each made of 64 blocks of 32
 * consecutive elements with one scale per block.  Positions of the last tile
 * beyond n are taken as +0.  Packed size = ceil(n/2048) * rc_tile_bytes().
 *
 *   INT4  (1152 B/tile): 1024 B of 4-bit sign/magnitude codes (element i in
 *         nibble i, low nibble first; magnitude 0..7 in bits 0-2, sign in
 *         bit 3), then 64 little-endian fp16 scales.
 *   INT3  (896 B/tile):  q2w plane (512 B, 2-bit magnitudes 0..3), q1w plane
 *         (256 B, sign of element i at bit i), then 64 fp16 scales.  Inside
 *         block b the q2w bits of element e sit at bit 64b + 32*((e/2)%2) +
 *         4*(e/4) + 2*(e%2) of the plane (element pairs dealt alternately to
 *         the block's two 32-bit words).
 *   FP8   (2304 B/tile): 2048 E4M3 codes (OCP "FN": no infinities, NaN =
 *         S.1111.111), then 64 little-endian fp32 scales.
 *   MXFP4 (1088 B/tile): 1024 B of E2M1 codes (element i in nibble i), then
 *         64 E8M0 scale bytes (2^(byte-127)).
 *
 * Numerics (bit-exact with the CPU oracle under oracle/):
 *   INT4/INT3: s = fp16(min(fp32(absmax / qmax), 65504)) with qmax = 7 / 3;
 *     magnitude = min(round-half-even(fp32(|v| * fp32(1 / s))), qmax) (one
 *     binary32 multiply by the correctly rounded reciprocal, then the nearest
 *     integer), sign = sign bit of v; a block whose s is 0 is stored as
 *     all-zero bytes.
 *   FP8: s = fp32(absmax / 448), flushed to 0 below FLT_MIN (block stored as
 *     zeros); code = E4M3 round-to-nearest-even of the exact quotient v / s,
 *     saturating at 448, sign kept.  Decode = fp32(code * s).
 *   MXFP4: e = clamp(floor(log2 absmax) - 2, -127, 127) (-127 for a zero
 *     block); code = E2M1 round-to-nearest-even of v * 2^-e, saturating at 6,
 *     sign kept.
 *   Reduce: acc = d_0; acc = fp32(acc + d_k) for k = 1..K-1 in stream order;
 *     the sums are requantized with the same codec.
 *
 * Conventions shared by every entry point:
 *   - Pointers named in/out/ins[k]/sum_out are device pointers (HIP global
 *     memory), 16-byte aligned; the caller owns all of them.  Inputs and
 *     outputs must not overlap.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     there and completes asynchronously; the library never synchronizes,
 *     allocates nothing and keeps no state, so calls are thread-safe.
 *   - All arguments are validated before any HIP call; nothing aborts and no
 *     exception crosses the ABI.  n = 0 is a successful no-op.
 *   - The GPU does not check inputs for NaN or infinity; their codes are
 *     unspecified (but every access stays in bounds).
 */
#ifndef RCODEC_H
#define RCODEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RC_ABI_VERSION 1
#define RC_TILE_ELEMS 2048
#define RC_BLOCK_ELEMS 32
#define RC_MAX_STREAMS 16

typedef enum { RC_FMT_INT4 = 1, RC_FMT_INT3 = 2, RC_FMT_FP8_E4M3 = 3, RC_FMT_MXFP4 = 4 } rc_format;
typedef enum { RC_SCALE_FP16 = 1, RC_SCALE_FP32 = 2, RC_SCALE_E8M0 = 3 } rc_scale_type;
typedef enum { RC_DT_FP32 = 1, RC_DT_FP16 = 2, RC_DT_BF16 = 3 } rc_dtype;

/* Codec = element format + scale type + block size, passed by value.
 * Supported: {INT4, FP16, 32}, {INT3, FP16, 32}, {FP8_E4M3, FP32, 32},
 * {MXFP4, E8M0, 32}; anything else is RC_ERR_UNSUPPORTED. */
typedef struct { int32_t format, scale, block; } rc_codec;

typedef enum {
    RC_OK = 0,
    RC_ERR_NULL = 1,         /* a required pointer is NULL while n > 0        */
    RC_ERR_UNSUPPORTED = 2,  /* codec or dtype not supported                  */
    RC_ERR_ALIGN = 3,        /* a device pointer is not 16-byte aligned       */
    RC_ERR_RANGE = 4,        /* k outside [1, RC_MAX_STREAMS] or n too large  */
    RC_ERR_HIP = 5           /* the kernel launch failed (hipGetLastError)    */
} rc_status;

/* Bytes of one 2048-element tile (1152 / 896 / 2304 / 1088), 0 when the codec
 * is unsupported.  Tile sizes of INT4 and INT3: QuickReduce INT3 page,
 * Summary. */
size_t rc_tile_bytes(rc_codec c);

/* ceil(n / 2048) * rc_tile_bytes(c). */
size_t rc_packed_bytes(rc_codec c, size_t n);

/* Block-quantize n elements of `in` (dtype in_t: bf16, fp16 or fp32) and pack
 * them into rc_packed_bytes(c, n) bytes at `out`.  Every byte of `out`
 * (including padding of the last tile) is written.
 * Source: QuickReduce INT3 page -- Method (block FP16 scale, symmetric codes,
 * q2w/q1w planes); RCCLX -- Low-Precision Collectives (FP8, FP32/BF16 inputs);
 * Microscaling Data Formats and ML-SpecQD abstracts (MXFP4 direct cast). */
rc_status rc_quantize_pack(rc_codec c, rc_dtype in_t, const void *in, size_t n,
                           void *out, void *stream);

/* Decode n elements of the packed stream `in` to dtype out_t (fp32 exact; bf16
 * and fp16 rounded to nearest even, fp16 overflow to +-inf) at `out`
 * (n * sizeof(out_t) bytes). */
rc_status rc_unpack_dequant(rc_codec c, const void *in, size_t n, rc_dtype out_t,
                            void *out, void *stream);

/* Dequantize k packed streams of n elements (ins: HOST array of k device
 * pointers, 1 <= k <= RC_MAX_STREAMS), add them in FP32 in stream order and
 * requantize the sums into `out` (rc_packed_bytes(c, n) bytes).  If sum_out
 * is not NULL the n FP32 sums are also written there (n * 4 bytes).
 * Source: RCCLX -- Low-Precision Collectives (computation remains in FP32);
 * QuickReduce INT3 page -- Summary (inline-compressed all-reduce). */
rc_status rc_dequant_reduce_requant(rc_codec c, const void *const *ins, int k, size_t n,
                                    void *out, float *sum_out, void *stream);

/* Plain device-to-device copy of `bytes` bytes (multiple of 16) with the same
 * 16-byte vector loads/stores as the codec kernels: the bandwidth baseline
 * the codec kernels are measured against. */
rc_status rc_copy(const void *in, void *out, size_t bytes, void *stream);

/* Static description of a status code; never NULL. */
const char *rc_status_str(rc_status s);

/* RC_ABI_VERSION of the loaded library. */
int rc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
