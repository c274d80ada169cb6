// MXFP4 GEMV kernels (x and y in fp32, fp16 or bf16).
#include "rc_kernels.hpp"

namespace rc {
hipError_t launch_mxfp4_gemv(const void* w, size_t rows, size_t cols, int x_dtype, const void* x, int y_dtype,
                             void* y, hipStream_t st)
{
    return launch_gemv_impl(w, rows, cols, x_dtype, x, y_dtype, y, st);
}
}  // namespace rc
