// E4M3 variants: FP32 scales on 16- and 64-element blocks, FP16 and E8M0
// scales on every block size; reduce unrolled for 2, 4 and 8 streams.
#include "rc_inst.hpp"

using namespace rc;
RC_INSTANTIATE(kFp8, kS32, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kFp8, kS32, 64, launch_reduce_rt_t)
RC_INSTANTIATE(kFp8, kS16, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kFp8, kS16, 32, launch_reduce_rt_t)
RC_INSTANTIATE(kFp8, kS16, 64, launch_reduce_rt_t)
RC_INSTANTIATE(kFp8, kSE8, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kFp8, kSE8, 32, launch_reduce_rt_t)
RC_INSTANTIATE(kFp8, kSE8, 64, launch_reduce_rt_t)
