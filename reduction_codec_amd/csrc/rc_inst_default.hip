// The four default codecs (32-element blocks): INT4 and INT3 with FP16
// scales, E4M3 with FP32 scales, E2M1 with E8M0 scales; the reduce is
// unrolled for every stream count.  Also the copy kernel's launcher.
#include "rc_inst.hpp"

using namespace rc;
RC_INSTANTIATE(kInt4, kS16, 32, launch_reduce_unrolled_t)
RC_INSTANTIATE(kInt3, kS16, 32, launch_reduce_unrolled_t)
RC_INSTANTIATE(kFp8, kS32, 32, launch_reduce_unrolled_t)
RC_INSTANTIATE(kMx4, kSE8, 32, launch_reduce_unrolled_t)

namespace rc {

// Plain 16-byte vector copy with non-temporal hints: the achievable-bandwidth
// reference the codec kernels are measured against.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(in + i), out + i);
}

hipError_t launch_copy(const void* in, void* out, size_t bytes, hipStream_t st)
{
    const size_t n16 = bytes / 16;
    size_t blocks = (n16 + 255) / 256;         // one 16-byte chunk per thread
    if (blocks > (1u << 20)) blocks = 1u << 20;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const u32x4*>(in),
                       static_cast<u32x4*>(out), n16);
    return hipGetLastError();
}
}  // namespace rc
