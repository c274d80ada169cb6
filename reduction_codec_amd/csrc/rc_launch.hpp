// rc_launch.hpp -- host-side declarations shared by the C-ABI layer, the
// codec dispatch and the kernel instantiation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rc {

// element formats (rc_format values)
enum : int { kInt4 = 1, kInt3 = 2, kFp8 = 3, kMx4 = 4, kBf8 = 5 };
constexpr int kMaxStreams = 16;

// Device pointers of the K input streams, passed by value in the kernel
// argument segment (no device-side pointer array).
struct StreamPtrs { const uint8_t* p[kMaxStreams]; };

// Launcher templates (defined in rc_kernels.hpp, instantiated per codec in
// the rc_inst_*.hip units).  FMT = element format, SC = scale type
// (rc_scale_type), BL = block size.
template <int FMT, int SC, int BL>
hipError_t launch_quantize_t(int dtype, const void* in, size_t n, void* out, hipStream_t st);
template <int FMT, int SC, int BL>
hipError_t launch_unpack_t(const void* in, size_t n, int dtype, void* out, hipStream_t st);
template <int FMT, int SC, int BL>
hipError_t launch_reduce_unrolled_t(const StreamPtrs& p, int k, size_t n, void* out, float* sum, hipStream_t st);
template <int FMT, int SC, int BL>
hipError_t launch_reduce_rt_t(const StreamPtrs& p, int k, size_t n, void* out, float* sum, hipStream_t st);

template <int FMT, int SC, int BL>
hipError_t launch_allreduce_t(int dtype, const StreamPtrs& msgs, int k, size_t n, int two_shot, void* out,
                              void* packed, hipStream_t st);

// Codec dispatch (rc_dispatch.cpp): hipErrorInvalidValue for an unsupported
// (format, scale, block) -- the C ABI checks codecs before calling.
hipError_t launch_quantize(int fmt, int sc, int bl, int dtype, const void* in, size_t n, void* out, hipStream_t st);
hipError_t launch_unpack(int fmt, int sc, int bl, const void* in, size_t n, int dtype, void* out, hipStream_t st);
hipError_t launch_reduce(int fmt, int sc, int bl, const StreamPtrs& p, int k, size_t n, void* out, float* sum,
                         hipStream_t st);
hipError_t launch_allreduce(int fmt, int sc, int bl, int dtype, const StreamPtrs& msgs, int k, size_t n, int two_shot,
                            void* out, void* packed, hipStream_t st);
hipError_t launch_copy(const void* in, void* out, size_t bytes, hipStream_t st);
// y = W x on an MXFP4-packed row-major matrix, cols a multiple of 2048.
hipError_t launch_mxfp4_gemv(const void* w, size_t rows, size_t cols, int x_dtype, const void* x, int y_dtype,
                             void* y, hipStream_t st);

}  // namespace rc
