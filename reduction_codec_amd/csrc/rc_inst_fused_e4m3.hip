// Fused all-reduce emulation kernels of the E4M3 variant codecs (FP32 scales
// on 16- and 64-element blocks, FP16 and E8M0 scales).
#include "rc_inst.hpp"

using namespace rc;
#define RC_INSTANTIATE_AR(FMT, SC, BL)                                                                       \
    template hipError_t rc::launch_allreduce_t<FMT, SC, BL>(int, const rc::StreamPtrs&, int, size_t, int, void*, \
                                                            void*, hipStream_t);
RC_INSTANTIATE_AR(kFp8, kS32, 16)
RC_INSTANTIATE_AR(kFp8, kS32, 64)
RC_INSTANTIATE_AR(kFp8, kS16, 16)
RC_INSTANTIATE_AR(kFp8, kS16, 32)
RC_INSTANTIATE_AR(kFp8, kS16, 64)
RC_INSTANTIATE_AR(kFp8, kSE8, 16)
RC_INSTANTIATE_AR(kFp8, kSE8, 32)
RC_INSTANTIATE_AR(kFp8, kSE8, 64)
