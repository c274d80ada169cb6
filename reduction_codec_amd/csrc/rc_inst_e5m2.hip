// E5M2 with FP32, FP16 and E8M0 scales on every block size; reduce
// unrolled for 2, 4 and 8 streams.
#include "rc_inst.hpp"

using namespace rc;
RC_INSTANTIATE(kBf8, kS32, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kS32, 32, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kS32, 64, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kS16, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kS16, 32, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kS16, 64, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kSE8, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kSE8, 32, launch_reduce_rt_t)
RC_INSTANTIATE(kBf8, kSE8, 64, launch_reduce_rt_t)
