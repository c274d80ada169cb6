// Fused all-reduce emulation kernels of the INT4, INT3 and E2M1 variant
// codecs (16- and 64-element blocks, E8M0 scales on INT elements).
#include "rc_inst.hpp"

using namespace rc;
#define RC_INSTANTIATE_AR(FMT, SC, BL)                                                                       \
    template hipError_t rc::launch_allreduce_t<FMT, SC, BL>(int, const rc::StreamPtrs&, int, size_t, int, void*, \
                                                            void*, hipStream_t);
RC_INSTANTIATE_AR(kInt4, kS16, 16)
RC_INSTANTIATE_AR(kInt4, kS16, 64)
RC_INSTANTIATE_AR(kInt4, kSE8, 16)
RC_INSTANTIATE_AR(kInt4, kSE8, 32)
RC_INSTANTIATE_AR(kInt4, kSE8, 64)
RC_INSTANTIATE_AR(kInt3, kS16, 16)
RC_INSTANTIATE_AR(kInt3, kS16, 64)
RC_INSTANTIATE_AR(kInt3, kSE8, 16)
RC_INSTANTIATE_AR(kInt3, kSE8, 32)
RC_INSTANTIATE_AR(kInt3, kSE8, 64)
RC_INSTANTIATE_AR(kMx4, kSE8, 16)
RC_INSTANTIATE_AR(kMx4, kSE8, 64)
