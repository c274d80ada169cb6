// Fused all-reduce emulation kernels of the four default codecs (the variant
// codecs' are in rc_inst_fused_int/e4m3/e5m2.hip).
#include "rc_inst.hpp"

using namespace rc;
#define RC_INSTANTIATE_AR(FMT, SC, BL)                                                                       \
    template hipError_t rc::launch_allreduce_t<FMT, SC, BL>(int, const rc::StreamPtrs&, int, size_t, int, void*, \
                                                            void*, hipStream_t);
RC_INSTANTIATE_AR(kInt4, kS16, 32)
RC_INSTANTIATE_AR(kInt3, kS16, 32)
RC_INSTANTIATE_AR(kFp8, kS32, 32)
RC_INSTANTIATE_AR(kMx4, kSE8, 32)
