/*
 * A plain C99 consumer of include/rcodec.h (test infrastructure).
 *
 * Built by tests/test_c_consumer.py with gcc -std=c99 -pedantic -Werror and
 * linked against librcodec.so: the header must be valid C, and the exported
 * functions must behave as declared for a C caller.  Only calls that return
 * before any HIP call are made (sizes, version, status strings, and every
 * validation error), so no GPU is needed.  Exit status 0 = every check held.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rcodec.h"

static int failures = 0;

static void check(int cond, const char *what)
{
    if (!cond) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

int main(void)
{
    const rc_codec int4 = {RC_FMT_INT4, RC_SCALE_FP16, 32};
    const rc_codec int3 = {RC_FMT_INT3, RC_SCALE_FP16, 32};
    const rc_codec fp8 = {RC_FMT_FP8_E4M3, RC_SCALE_FP32, 32};
    const rc_codec mx = {RC_FMT_MXFP4, RC_SCALE_E8M0, 32};
    const rc_codec bad_scale = {RC_FMT_MXFP4, RC_SCALE_FP16, 32};
    const rc_codec bad_block = {RC_FMT_INT4, RC_SCALE_FP16, 48};
    /* never dereferenced: validation rejects the call before any access */
    void *const odd = (void *)(uintptr_t)0x1001;
    void *const even = (void *)(uintptr_t)0x1000;
    const void *ins[2];
    int s;

    check(rc_abi_version() == RC_ABI_VERSION, "rc_abi_version() == RC_ABI_VERSION");

    check(rc_tile_bytes(int4) == 1152, "INT4 tile 1152 B");
    check(rc_tile_bytes(int3) == 896, "INT3 tile 896 B");
    check(rc_tile_bytes(fp8) == 2304, "E4M3 + FP32 tile 2304 B");
    check(rc_tile_bytes(mx) == 1088, "MXFP4 tile 1088 B");
    check(rc_tile_bytes(bad_scale) == 0 && rc_tile_bytes(bad_block) == 0, "unsupported codecs have no size");
    check(rc_packed_bytes(int3, 0) == 0, "packed size of 0 elements");
    check(rc_packed_bytes(int3, 1) == 896 && rc_packed_bytes(int3, 2048) == 896 &&
              rc_packed_bytes(int3, 2049) == 2 * 896, "packed size rounds up to whole tiles");

    for (s = RC_OK; s <= RC_ERR_HIP; ++s) {
        const char *msg = rc_status_str((rc_status)s);
        check(msg != NULL && msg[0] != '\0', "every status has a description");
        if (s > RC_OK) check(strcmp(msg, rc_status_str((rc_status)(s - 1))) != 0, "descriptions differ");
    }
    check(rc_status_str((rc_status)99) != NULL, "unknown status still described");

    /* quantize / unpack */
    check(rc_quantize_pack(bad_scale, RC_DT_BF16, even, 1, even, NULL) == RC_ERR_UNSUPPORTED, "quantize: codec");
    check(rc_quantize_pack(int3, (rc_dtype)7, even, 1, even, NULL) == RC_ERR_UNSUPPORTED, "quantize: dtype");
    check(rc_quantize_pack(int3, RC_DT_BF16, NULL, 0, NULL, NULL) == RC_OK, "quantize: n = 0 is a no-op");
    check(rc_quantize_pack(int3, RC_DT_BF16, NULL, 1, even, NULL) == RC_ERR_NULL, "quantize: null input");
    check(rc_quantize_pack(int3, RC_DT_BF16, odd, 1, even, NULL) == RC_ERR_ALIGN, "quantize: misaligned input");
    check(rc_quantize_pack(int3, RC_DT_BF16, even, (size_t)1 << 41, even, NULL) == RC_ERR_RANGE, "quantize: n");
    check(rc_unpack_dequant(int4, even, 1, RC_DT_FP32, NULL, NULL) == RC_ERR_NULL, "unpack: null output");
    check(rc_unpack_dequant(int4, even, 1, RC_DT_FP32, odd, NULL) == RC_ERR_ALIGN, "unpack: misaligned output");

    /* reduce */
    ins[0] = even;
    ins[1] = odd;
    check(rc_dequant_reduce_requant(int3, ins, 0, 1, even, NULL, NULL) == RC_ERR_RANGE, "reduce: k = 0");
    check(rc_dequant_reduce_requant(int3, ins, RC_MAX_STREAMS + 1, 1, even, NULL, NULL) == RC_ERR_RANGE,
          "reduce: k too large");
    check(rc_dequant_reduce_requant(int3, ins, 2, 0, even, NULL, NULL) == RC_OK, "reduce: n = 0 is a no-op");
    check(rc_dequant_reduce_requant(int3, NULL, 1, 1, even, NULL, NULL) == RC_ERR_NULL, "reduce: null ins");
    check(rc_dequant_reduce_requant(int3, ins, 2, 1, even, NULL, NULL) == RC_ERR_ALIGN, "reduce: misaligned stream");
    check(rc_dequant_reduce_requant(int3, ins, 1, 1, even, (float *)odd, NULL) == RC_ERR_ALIGN,
          "reduce: misaligned sums");

    /* fused all-reduce, GEMV, copy */
    check(rc_allreduce_emulate(bad_block, RC_DT_BF16, ins, 1, 1, 1, even, NULL, NULL) == RC_ERR_UNSUPPORTED,
          "all-reduce: codec");
    check(rc_allreduce_emulate(int4, RC_DT_BF16, ins, 0, 1, 1, even, NULL, NULL) == RC_ERR_RANGE, "all-reduce: k");
    check(rc_mxfp4_gemv(even, 1, 1000, RC_DT_FP32, even, RC_DT_FP32, even, NULL) == RC_ERR_RANGE, "gemv: cols");
    check(rc_mxfp4_gemv(even, 0, 2048, RC_DT_FP32, even, RC_DT_FP32, even, NULL) == RC_OK, "gemv: no rows");
    check(rc_copy(even, even, 17, NULL) == RC_ERR_ALIGN, "copy: size not a multiple of 16");
    check(rc_copy(NULL, even, 16, NULL) == RC_ERR_NULL, "copy: null input");

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("C consumer: all checks held\n");
    return 0;
}
