// INT4 / INT3 variants: FP16 scales on 16- and 64-element blocks, E8M0
// scales on every block size; reduce unrolled for 2, 4 and 8 streams.
#include "rc_inst.hpp"

using namespace rc;
RC_INSTANTIATE(kInt4, kS16, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kInt4, kS16, 64, launch_reduce_rt_t)
RC_INSTANTIATE(kInt4, kSE8, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kInt4, kSE8, 32, launch_reduce_rt_t)
RC_INSTANTIATE(kInt4, kSE8, 64, launch_reduce_rt_t)
RC_INSTANTIATE(kInt3, kS16, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kInt3, kS16, 64, launch_reduce_rt_t)
RC_INSTANTIATE(kInt3, kSE8, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kInt3, kSE8, 32, launch_reduce_rt_t)
RC_INSTANTIATE(kInt3, kSE8, 64, launch_reduce_rt_t)
