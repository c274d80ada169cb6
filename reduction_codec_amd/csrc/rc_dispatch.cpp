// rc_dispatch.cpp -- (format, scale type, block size) -> the codec's
// launchers.  Host code only; the launchers are instantiated in the
// rc_inst_*.hip units.
#include "rc_launch.hpp"

namespace rc {
namespace {

enum : int { S16 = 1, S32 = 2, SE8 = 3 };

typedef hipError_t (*QuantizeFn)(int, const void*, size_t, void*, hipStream_t);
typedef hipError_t (*UnpackFn)(const void*, size_t, int, void*, hipStream_t);
typedef hipError_t (*ReduceFn)(const StreamPtrs&, int, size_t, void*, float*, hipStream_t);
typedef hipError_t (*AllreduceFn)(int, const StreamPtrs&, int, size_t, int, void*, void*, hipStream_t);

struct Entry {
    int fmt, sc, bl;
    QuantizeFn q;
    UnpackFn u;
    ReduceFn r;
    AllreduceFn a;
};

#define RC_ENTRY(F, S, B, R)                                                                  \
    {F, S, B, &launch_quantize_t<F, S, B>, &launch_unpack_t<F, S, B>, &R<F, S, B>, &launch_allreduce_t<F, S, B>}

const Entry kCodecs[] = {
    RC_ENTRY(kInt4, S16, 32, launch_reduce_unrolled_t),
    RC_ENTRY(kInt3, S16, 32, launch_reduce_unrolled_t),
    RC_ENTRY(kFp8, S32, 32, launch_reduce_unrolled_t),
    RC_ENTRY(kMx4, SE8, 32, launch_reduce_unrolled_t),
    RC_ENTRY(kInt4, S16, 16, launch_reduce_rt_t),
    RC_ENTRY(kInt4, S16, 64, launch_reduce_rt_t),
    RC_ENTRY(kInt4, SE8, 16, launch_reduce_rt_t),
    RC_ENTRY(kInt4, SE8, 32, launch_reduce_rt_t),
    RC_ENTRY(kInt4, SE8, 64, launch_reduce_rt_t),
    RC_ENTRY(kInt3, S16, 16, launch_reduce_rt_t),
    RC_ENTRY(kInt3, S16, 64, launch_reduce_rt_t),
    RC_ENTRY(kInt3, SE8, 16, launch_reduce_rt_t),
    RC_ENTRY(kInt3, SE8, 32, launch_reduce_rt_t),
    RC_ENTRY(kInt3, SE8, 64, launch_reduce_rt_t),
    RC_ENTRY(kFp8, S32, 16, launch_reduce_rt_t),
    RC_ENTRY(kFp8, S32, 64, launch_reduce_rt_t),
    RC_ENTRY(kFp8, S16, 16, launch_reduce_rt_t),
    RC_ENTRY(kFp8, S16, 32, launch_reduce_rt_t),
    RC_ENTRY(kFp8, S16, 64, launch_reduce_rt_t),
    RC_ENTRY(kFp8, SE8, 16, launch_reduce_rt_t),
    RC_ENTRY(kFp8, SE8, 32, launch_reduce_rt_t),
    RC_ENTRY(kFp8, SE8, 64, launch_reduce_rt_t),
    RC_ENTRY(kBf8, S32, 16, launch_reduce_rt_t),
    RC_ENTRY(kBf8, S32, 32, launch_reduce_rt_t),
    RC_ENTRY(kBf8, S32, 64, launch_reduce_rt_t),
    RC_ENTRY(kBf8, S16, 16, launch_reduce_rt_t),
    RC_ENTRY(kBf8, S16, 32, launch_reduce_rt_t),
    RC_ENTRY(kBf8, S16, 64, launch_reduce_rt_t),
    RC_ENTRY(kBf8, SE8, 16, launch_reduce_rt_t),
    RC_ENTRY(kBf8, SE8, 32, launch_reduce_rt_t),
    RC_ENTRY(kBf8, SE8, 64, launch_reduce_rt_t),
    RC_ENTRY(kMx4, SE8, 16, launch_reduce_rt_t),
    RC_ENTRY(kMx4, SE8, 64, launch_reduce_rt_t),
};

const Entry* find(int fmt, int sc, int bl)
{
    for (const Entry& e : kCodecs)
        if (e.fmt == fmt && e.sc == sc && e.bl == bl) return &e;
    return nullptr;
}

}  // namespace

hipError_t launch_quantize(int fmt, int sc, int bl, int dtype, const void* in, size_t n, void* out, hipStream_t st)
{
    const Entry* e = find(fmt, sc, bl);
    return e ? e->q(dtype, in, n, out, st) : hipErrorInvalidValue;
}

hipError_t launch_unpack(int fmt, int sc, int bl, const void* in, size_t n, int dtype, void* out, hipStream_t st)
{
    const Entry* e = find(fmt, sc, bl);
    return e ? e->u(in, n, dtype, out, st) : hipErrorInvalidValue;
}

hipError_t launch_reduce(int fmt, int sc, int bl, const StreamPtrs& p, int k, size_t n, void* out, float* sum,
                         hipStream_t st)
{
    const Entry* e = find(fmt, sc, bl);
    return e ? e->r(p, k, n, out, sum, st) : hipErrorInvalidValue;
}

hipError_t launch_allreduce(int fmt, int sc, int bl, int dtype, const StreamPtrs& msgs, int k, size_t n, int two_shot,
                            void* out, void* packed, hipStream_t st)
{
    const Entry* e = find(fmt, sc, bl);
    return e ? e->a(dtype, msgs, k, n, two_shot, out, packed, st) : hipErrorInvalidValue;
}

}  // namespace rc
