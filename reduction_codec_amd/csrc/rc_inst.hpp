// rc_inst.hpp -- explicit instantiation of one codec's launchers.
#pragma once
#include "rc_kernels.hpp"

#define RC_INSTANTIATE(FMT, SC, BL, REDUCE)                                                             \
    template hipError_t rc::launch_quantize_t<FMT, SC, BL>(int, const void*, size_t, void*, hipStream_t); \
    template hipError_t rc::launch_unpack_t<FMT, SC, BL>(const void*, size_t, int, void*, hipStream_t);   \
    template hipError_t rc::REDUCE<FMT, SC, BL>(const rc::StreamPtrs&, int, size_t, void*, float*, hipStream_t);
