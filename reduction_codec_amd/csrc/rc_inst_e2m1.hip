// E2M1 (MXFP4 elements) with E8M0 scales on 16- and 64-element blocks;
// reduce unrolled for 2, 4 and 8 streams.
#include "rc_inst.hpp"

using namespace rc;
RC_INSTANTIATE(kMx4, kSE8, 16, launch_reduce_rt_t)
RC_INSTANTIATE(kMx4, kSE8, 64, launch_reduce_rt_t)
