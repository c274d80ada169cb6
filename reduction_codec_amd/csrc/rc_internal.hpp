// rc_internal.hpp -- declarations shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rc {

enum : int { kInt4 = 1, kInt3 = 2, kFp8 = 3, kMx4 = 4 };   // rc_format values
constexpr int kMaxStreams = 16;

// Device pointers of the K input streams, passed by value in the kernel
// argument segment (no device-side pointer array).
struct StreamPtrs { const uint8_t* p[kMaxStreams]; };

hipError_t launch_quantize(int fmt, int dtype, const void* in, size_t n, void* out, hipStream_t st);
hipError_t launch_unpack(int fmt, const void* in, size_t n, int dtype, void* out, hipStream_t st);
hipError_t launch_reduce(int fmt, const StreamPtrs& p, int k, size_t n, void* out, float* sum, hipStream_t st);
hipError_t launch_copy(const void* in, void* out, size_t bytes, hipStream_t st);

}  // namespace rc
