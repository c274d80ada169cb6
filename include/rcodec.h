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
 * Data layout (all codecs): the stream of n elements is cut into
 * ceil(n/2048) tiles of 2048 elements; each tile is its code region
 * followed by 2048/block scales (one per block of `block` consecutive
 * elements).  Positions of the last tile beyond n are taken as +0.  Packed
 * size = ceil(n/2048) * rc_tile_bytes().  Code regions:
 *
 *   INT4  (1024 B): 4-bit sign/magnitude codes (element i in nibble i, low
 *         nibble first; magnitude 0..7 in bits 0-2, sign in bit 3).
 *   INT3  (768 B):  q2w plane (512 B, 2-bit magnitudes 0..3), then q1w plane
 *         (256 B, sign of element i at bit i).  The q2w bits of element e of
 *         the 32-element group g (tile element 32g + e, whatever the block
 *         size) sit at bit 64g + 32*((e/2)%2) + 4*(e/4) + 2*(e%2) of the plane
 *         (element pairs dealt alternately to the group's two 32-bit words).
 *   FP8_E4M3 (2048 B): E4M3 codes (OCP "FN": no infinities, NaN = S.1111.111).
 *   FP8_E5M2 (2048 B): E5M2 codes (bias 15, IEEE infinities and NaNs).
 *         FP8 byte order: two 1024 B planes; the codes of elements 32g..32g+15
 *         (the first half of the 32-element group g, whatever the block size)
 *         at bytes 16g..16g+15, those of 32g+16..32g+31 at 1024+16g.., so the
 *         codes of 32 consecutive elements are two wave-contiguous 16 B
 *         accesses.
 *   MXFP4 (1024 B): E2M1 codes (element i in nibble i).
 * Scales: fp16 (2 B) or fp32 (4 B) little-endian, or E8M0 bytes
 * (2^(byte-127), 0xFF = NaN).  The default tiles: INT4 1152 B, INT3 896 B,
 * E4M3 + FP32 2304 B, MXFP4 1088 B.
 *
 * Numerics (bit-exact with the CPU oracle under oracle/):
 *   INT4/INT3, FP16 scale: s = fp16(min(fp32(absmax / qmax), 65504)) with
 *     qmax = 7 / 3; magnitude = min(round-half-even(|v| / s), qmax) of the
 *     exact quotient (so |v - q s| <= s / 2 for every unclamped element, and
 *     exact half steps go to the even integer), sign = sign bit of v; a block
 *     whose s is 0 is stored as all-zero bytes.
 *   FP8, FP32 scale: s = fp32(absmax / fmax) (fmax = 448 for E4M3, 57344 for
 *     E5M2), flushed to 0 below FLT_MIN (block stored as zeros); code = the
 *     round-to-nearest-even code of the exact quotient v / s, saturating at
 *     fmax, sign kept.  Decode = fp32(code * s).
 *   FP8, FP16 scale: s = fp16(min(fp32(absmax / fmax), 65504)); codes as with
 *     an FP32 scale; s = 0 stores a zero block.
 *   E8M0 scale (any element format): e = clamp(floor(log2 absmax) - emax,
 *     -127, 127) with emax = 2 (E2M1), 8 (E4M3), 15 (E5M2), 2 (INT4), 1
 *     (INT3); -127 for a zero block; code = the nearest code (ties to even,
 *     saturating at the format's largest magnitude) of v * 2^-e; signs kept.
 *   Reduce: acc = d_0; acc = fp32(acc + d_k) for k = 1..K-1 in stream order;
 *     the sums are requantized with the same codec.
 *   Decode of any bytes: every bit pattern of codes and scales decodes to
 *     fp32(code * scale) (NaN and infinite FP8 codes, negative, subnormal and
 *     non-finite FP16/FP32 scales included), so the decoded values and the
 *     FP32 sums of arbitrary packed data are defined.  With E8M0 scales the
 *     product is rounded, so scale bytes the encoder never writes (2^120 and
 *     up for E4M3, 2^113 for E5M2, 2^126 for INT4 and E2M1, 2^127 for INT3)
 *     give +-inf where it overflows, and 0xFF gives NaN.  The requantized
 *     codes of non-finite sums are unspecified.
 *
 * Conventions shared by every entry point:
 *   - Pointers named in/out/ins[k]/sum_out are device pointers (HIP global
 *     memory), 16-byte aligned; the caller owns all of them.  Inputs and
 *     outputs must not overlap, with two exceptions for in-place use: the
 *     `out` of rc_dequant_reduce_requant may be exactly one of ins[], and the
 *     `out` of rc_allreduce_emulate exactly one of msgs[] (each tile is read
 *     in full before anything of that tile is written).
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

/* 1: the four default codecs; 2: format, scale and block variants, the fused
 * all-reduce emulation and the MXFP4 GEMV; 3: FP8 codes in two 1024-byte
 * planes (packed FP8 data of version 2 reads differently). */
#define RC_ABI_VERSION 3
#define RC_TILE_ELEMS 2048
#define RC_BLOCK_ELEMS 32
#define RC_MAX_STREAMS 16

typedef enum { RC_FMT_INT4 = 1, RC_FMT_INT3 = 2, RC_FMT_FP8_E4M3 = 3, RC_FMT_MXFP4 = 4,
               RC_FMT_FP8_E5M2 = 5 } rc_format;
typedef enum { RC_SCALE_FP16 = 1, RC_SCALE_FP32 = 2, RC_SCALE_E8M0 = 3 } rc_scale_type;
typedef enum { RC_DT_FP32 = 1, RC_DT_FP16 = 2, RC_DT_BF16 = 3 } rc_dtype;

/* Codec = element format + scale type + block size, passed by value.
 * Supported (block 16, 32 or 64 elements in every case):
 *   INT4, INT3          with RC_SCALE_FP16 or RC_SCALE_E8M0
 *   FP8_E4M3, FP8_E5M2  with RC_SCALE_FP32, RC_SCALE_FP16 or RC_SCALE_E8M0
 *   MXFP4 (E2M1)        with RC_SCALE_E8M0
 * anything else is RC_ERR_UNSUPPORTED.  The defaults of the pages are
 * {INT4, FP16, 32}, {INT3, FP16, 32}, {FP8_E4M3, FP32, 32}, {MXFP4, E8M0, 32}. */
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

/* Bytes of a packed stream of n elements: ceil(n / 2048) * rc_tile_bytes(c)
 * (fixed-size tiles, the unit the QuickReduce INT3 page counts in -- Summary:
 * 1152 B per INT4 tile, 896 B per INT3 tile); 0 when the codec is
 * unsupported.  Pure arithmetic: no HIP call, callable without a GPU. */
size_t rc_packed_bytes(rc_codec c, size_t n);

/* Block-quantize n elements of `in` (dtype in_t: bf16, fp16 or fp32) and pack
 * them into rc_packed_bytes(c, n) bytes at `out`.  Every byte of `out`
 * (including padding of the last tile) is written.
 * Source: QuickReduce INT3 page -- Method (block FP16 scale, symmetric codes,
 * q2w/q1w planes); RCCLX -- Low-Precision Collectives (FP8, FP32/BF16 inputs);
 * Microscaling Data Formats and ML-SpecQD abstracts (MXFP4 direct cast). */
rc_status rc_quantize_pack(rc_codec c, rc_dtype in_t, const void *in, size_t n,
                           void *out, void *stream);

/* Decode n elements of the packed stream `in` (rc_packed_bytes(c, n) bytes)
 * to dtype out_t at `out` (n * sizeof(out_t) bytes): each value is code times
 * block scale computed in FP32 (exact with FP16 and E8M0 scales while the
 * product is a binary32 number, one binary32 product for FP8 with an FP32
 * scale; "Decode of any bytes" above), then written as fp32, or rounded to
 * bf16 / fp16 (nearest even, fp16 overflow to +-inf).  This is the receiving
 * side's decode: payloads travel compressed and the arithmetic on them stays
 * in FP32 (RCCLX -- Low-Precision Collectives; QuickReduce INT3 page --
 * Method, FP16 block scale).  Errors as for rc_quantize_pack. */
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

/* Fused single-GPU emulation of a quantized all-reduce over k messages that
 * all sit in this GPU's memory, one per emulated rank ("RCCLX: Innovating
 * GPU communications on AMD platforms" -- Direct Data Access: the flat
 * one-shot and the tree-shaped two-shot all-reduce, with the low-precision
 * payloads of Low-Precision Collectives).  Every message is quantized with
 * codec c and decoded (what a receiving rank decodes), the decoded values
 * are added in FP32 in message order, and then
 *   two_shot != 0 (reduce-scatter and all-gather both carry compressed data):
 *     out = unpack_dequant(requantize(sum)), and the requantized sum (the
 *     all-gather payload, rc_packed_bytes(c, n) bytes) goes to packed_out
 *     when packed_out is not NULL;
 *   two_shot == 0 (every rank reads all compressed messages):
 *     out = the sum rounded to dt (RNE), packed_out unused.
 * Exactly what the separate calls compute (rc_quantize_pack of each message,
 * rc_dequant_reduce_requant with sums, rc_unpack_dequant), in one kernel
 * pass that touches only the messages, out and packed_out.
 *   msgs: host array of k device pointers to n elements of dt each;
 *   out:  n elements of dt.  Every supported codec.  Errors as for
 *   rc_dequant_reduce_requant. */
rc_status rc_allreduce_emulate(rc_codec c, rc_dtype dt, const void *const *msgs, int k, size_t n,
                               int two_shot, void *out, void *packed_out, void *stream);

/* y = W x for a row-major rows x cols matrix W held as an MXFP4 packed stream
 * (rc_quantize_pack of its rows * cols elements with {MXFP4, E8M0, 32}), the
 * consumer of the packed layout ("ML-SpecQD: Multi-Level Speculative Decoding
 * with Quantized Drafts", abstract: MXFP4 weights direct-cast from BF16).
 * cols must be a positive multiple of 2048 (row r = tiles r*cols/2048 ...)
 * with cols * sizeof(x_t) < 2^32 bytes (x is addressed with 32-bit offsets),
 * else RC_ERR_RANGE.  x: cols elements of x_t; y: rows elements of y_t.
 * Accuracy: the pages fix no summation order, so the result is specified by
 * a bound, not an order: the binary32 value s computed for row r satisfies
 *   |s - sum_j W[r][j] x[j]| <= (38 + cols/2048) * 2^-24 * sum_j |W[r][j] x[j]|
 * (plus 2^-143 for block terms below 2^-126), every term passing through at
 * most that many binary32 roundings; y[r] = s rounded to y_t (nearest even).
 * The order is fixed by the kernel, so results are deterministic from call
 * to call.  Pointers are device pointers, 16-byte aligned. */
rc_status rc_mxfp4_gemv(const void *w, size_t rows, size_t cols, rc_dtype x_t, const void *x,
                        rc_dtype y_t, void *y, void *stream);

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
