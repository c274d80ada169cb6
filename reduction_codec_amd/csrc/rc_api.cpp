// rc_api.cpp -- the C ABI of librcodec.so (declared in include/rcodec.h):
// argument validation, then one kernel launch on the caller's stream.
// Validation never touches HIP, so every error path can be exercised on a
// machine without a GPU.
#include "rcodec.h"
#include "rc_launch.hpp"

namespace {

// Largest n accepted: 2^40 elements keeps every tile index, byte offset and
// grid dimension (tiles / 4 workgroups) far inside their types.
constexpr size_t kMaxElems = (size_t)1 << 40;

// Supported codecs: INT4/INT3 with FP16 or E8M0 scales, E4M3/E5M2 with FP32,
// FP16 or E8M0 scales, E2M1 (MXFP4) with E8M0 scales; blocks of 16, 32, 64.
bool codec_ok(rc_codec c)
{
    if (c.block != 16 && c.block != 32 && c.block != 64) return false;
    switch (c.format) {
    case RC_FMT_INT4:
    case RC_FMT_INT3:     return c.scale == RC_SCALE_FP16 || c.scale == RC_SCALE_E8M0;
    case RC_FMT_FP8_E4M3:
    case RC_FMT_FP8_E5M2: return c.scale == RC_SCALE_FP32 || c.scale == RC_SCALE_FP16 || c.scale == RC_SCALE_E8M0;
    case RC_FMT_MXFP4:    return c.scale == RC_SCALE_E8M0;
    default:              return false;
    }
}

bool dtype_ok(int d) { return d == RC_DT_FP32 || d == RC_DT_FP16 || d == RC_DT_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

rc_status from_hip(hipError_t e) { return e == hipSuccess ? RC_OK : RC_ERR_HIP; }

}  // namespace

extern "C" {

size_t rc_tile_bytes(rc_codec c)
{
    if (!codec_ok(c)) return 0;
    size_t code;                                  // code region of 2048 elements
    switch (c.format) {
    case RC_FMT_INT3: code = 768; break;          // 2-bit + 1-bit planes
    case RC_FMT_FP8_E4M3:
    case RC_FMT_FP8_E5M2: code = 2048; break;
    default: code = 1024;                         // 4-bit codes
    }
    const size_t sb = c.scale == RC_SCALE_FP16 ? 2 : (c.scale == RC_SCALE_FP32 ? 4 : 1);
    return code + (size_t)(RC_TILE_ELEMS / c.block) * sb;
}

size_t rc_packed_bytes(rc_codec c, size_t n)
{
    return ((n + RC_TILE_ELEMS - 1) / RC_TILE_ELEMS) * rc_tile_bytes(c);
}

rc_status rc_quantize_pack(rc_codec c, rc_dtype in_t, const void* in, size_t n, void* out, void* stream)
{
    if (!codec_ok(c) || !dtype_ok(in_t)) return RC_ERR_UNSUPPORTED;
    if (n == 0) return RC_OK;
    if (n > kMaxElems) return RC_ERR_RANGE;
    if (!in || !out) return RC_ERR_NULL;
    if (!aligned16(in) || !aligned16(out)) return RC_ERR_ALIGN;
    return from_hip(rc::launch_quantize(c.format, c.scale, c.block, in_t, in, n, out, static_cast<hipStream_t>(stream)));
}

rc_status rc_unpack_dequant(rc_codec c, const void* in, size_t n, rc_dtype out_t, void* out, void* stream)
{
    if (!codec_ok(c) || !dtype_ok(out_t)) return RC_ERR_UNSUPPORTED;
    if (n == 0) return RC_OK;
    if (n > kMaxElems) return RC_ERR_RANGE;
    if (!in || !out) return RC_ERR_NULL;
    if (!aligned16(in) || !aligned16(out)) return RC_ERR_ALIGN;
    return from_hip(rc::launch_unpack(c.format, c.scale, c.block, in, n, out_t, out, static_cast<hipStream_t>(stream)));
}

rc_status rc_dequant_reduce_requant(rc_codec c, const void* const* ins, int k, size_t n, void* out,
                                    float* sum_out, void* stream)
{
    if (!codec_ok(c)) return RC_ERR_UNSUPPORTED;
    if (k < 1 || k > RC_MAX_STREAMS) return RC_ERR_RANGE;
    if (n == 0) return RC_OK;
    if (n > kMaxElems) return RC_ERR_RANGE;
    if (!ins || !out) return RC_ERR_NULL;
    rc::StreamPtrs p = {};
    for (int j = 0; j < k; ++j) {
        if (!ins[j]) return RC_ERR_NULL;
        if (!aligned16(ins[j])) return RC_ERR_ALIGN;
        p.p[j] = static_cast<const uint8_t*>(ins[j]);
    }
    if (!aligned16(out) || (sum_out && !aligned16(sum_out))) return RC_ERR_ALIGN;
    return from_hip(rc::launch_reduce(c.format, c.scale, c.block, p, k, n, out, sum_out, static_cast<hipStream_t>(stream)));
}

rc_status rc_allreduce_emulate(rc_codec c, rc_dtype dt, const void* const* msgs, int k, size_t n, int two_shot,
                               void* out, void* packed_out, void* stream)
{
    if (!codec_ok(c) || !dtype_ok(dt)) return RC_ERR_UNSUPPORTED;
    if (k < 1 || k > RC_MAX_STREAMS) return RC_ERR_RANGE;
    if (n == 0) return RC_OK;
    if (n > kMaxElems) return RC_ERR_RANGE;
    if (!msgs || !out) return RC_ERR_NULL;
    rc::StreamPtrs p = {};
    for (int j = 0; j < k; ++j) {
        if (!msgs[j]) return RC_ERR_NULL;
        if (!aligned16(msgs[j])) return RC_ERR_ALIGN;
        p.p[j] = static_cast<const uint8_t*>(msgs[j]);
    }
    if (!aligned16(out) || (packed_out && !aligned16(packed_out))) return RC_ERR_ALIGN;
    return from_hip(rc::launch_allreduce(c.format, c.scale, c.block, dt, p, k, n, two_shot ? 1 : 0, out,
                                         two_shot ? packed_out : nullptr, static_cast<hipStream_t>(stream)));
}

rc_status rc_mxfp4_gemv(const void* w, size_t rows, size_t cols, rc_dtype x_t, const void* x, rc_dtype y_t,
                         void* y, void* stream)
{
    if (!dtype_ok(x_t) || !dtype_ok(y_t)) return RC_ERR_UNSUPPORTED;
    if (cols == 0 || cols % RC_TILE_ELEMS != 0 || cols > kMaxElems) return RC_ERR_RANGE;
    // x is read through one buffer descriptor with 32-bit byte offsets
    const size_t xbytes = cols * (x_t == RC_DT_FP32 ? 4u : 2u);
    if (xbytes >= ((size_t)1 << 32)) return RC_ERR_RANGE;
    if (rows == 0) return RC_OK;
    if (rows > kMaxElems / cols) return RC_ERR_RANGE;
    if (!w || !x || !y) return RC_ERR_NULL;
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) return RC_ERR_ALIGN;
    return from_hip(rc::launch_mxfp4_gemv(w, rows, cols, x_t, x, y_t, y, static_cast<hipStream_t>(stream)));
}

rc_status rc_copy(const void* in, void* out, size_t bytes, void* stream)
{
    if (bytes == 0) return RC_OK;
    if (!in || !out) return RC_ERR_NULL;
    if (!aligned16(in) || !aligned16(out) || (bytes & 15u)) return RC_ERR_ALIGN;
    return from_hip(rc::launch_copy(in, out, bytes, static_cast<hipStream_t>(stream)));
}

const char* rc_status_str(rc_status s)
{
    switch (s) {
    case RC_OK:              return "ok";
    case RC_ERR_NULL:        return "null pointer";
    case RC_ERR_UNSUPPORTED: return "unsupported codec or dtype";
    case RC_ERR_ALIGN:       return "pointer not 16-byte aligned";
    case RC_ERR_RANGE:       return "argument out of range";
    case RC_ERR_HIP:         return "HIP launch failed";
    default:                 return "unknown status";
    }
}

int rc_abi_version(void) { return RC_ABI_VERSION; }

}  // extern "C"
