// rc_kernels.hip -- gfx950 kernels of the codec and their launchers.
//
// One wave64 per 2048-element tile, lane l = block l; 256-thread workgroups
// (four tiles).  Every per-lane load and store is a contiguous span across
// the wave: code words at lane * (bytes per block), scales at lane * (scale
// bytes), input elements at lane * 32.
#include "rc_device.hpp"
#include "rc_internal.hpp"

namespace rc {

template <int FMT> struct TileBytes;
template <> struct TileBytes<kInt4> { static constexpr int v = 1152; };
template <> struct TileBytes<kInt3> { static constexpr int v = 896; };
template <> struct TileBytes<kFp8> { static constexpr int v = 2304; };
template <> struct TileBytes<kMx4> { static constexpr int v = 1088; };

__device__ __forceinline__ size_t tile_index() { return (size_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ------------------------------------------------------------- stores ----

template <int FMT>
__device__ __forceinline__ void encode_store(const float (&v)[32], uint8_t* __restrict__ t, int lane)
{
    if constexpr (FMT == kInt3) {
        const Int3Words w = int3_encode_block(v);
        *reinterpret_cast<uint2*>(t + 8 * lane) = make_uint2(w.w0, w.w1);
        *reinterpret_cast<uint32_t*>(t + 512 + 4 * lane) = w.h;
        *reinterpret_cast<uint16_t*>(t + 768 + 2 * lane) = (uint16_t)w.sbits;
    } else if constexpr (FMT == kInt4) {
        const Int4Words w = int4_encode_block(v);
        *reinterpret_cast<uint4*>(t + 16 * lane) = make_uint4(w.d[0], w.d[1], w.d[2], w.d[3]);
        *reinterpret_cast<uint16_t*>(t + 1024 + 2 * lane) = (uint16_t)w.sbits;
    } else if constexpr (FMT == kFp8) {
        const Fp8Words w = fp8_encode_block(v);
        uint4* p = reinterpret_cast<uint4*>(t + 32 * lane);
        p[0] = make_uint4(w.d[0], w.d[1], w.d[2], w.d[3]);
        p[1] = make_uint4(w.d[4], w.d[5], w.d[6], w.d[7]);
        *reinterpret_cast<float*>(t + 2048 + 4 * lane) = w.s;
    } else {
        const MxWords w = mx_encode_block(v);
        *reinterpret_cast<uint4*>(t + 16 * lane) = make_uint4(w.d[0], w.d[1], w.d[2], w.d[3]);
        t[1024 + lane] = (uint8_t)w.e8;
    }
}

// Per-lane code words of one block of one stream.
template <int FMT> struct LaneCodes;
template <> struct LaneCodes<kInt3> { uint2 q2; uint32_t h; uint32_t s; };
template <> struct LaneCodes<kInt4> { uint4 d; uint32_t s; };
template <> struct LaneCodes<kFp8> { uint4 d0, d1; float s; };
template <> struct LaneCodes<kMx4> { uint4 d; uint32_t e8; };

template <int FMT>
__device__ __forceinline__ LaneCodes<FMT> load_codes(const uint8_t* __restrict__ t, int lane)
{
    LaneCodes<FMT> c;
    if constexpr (FMT == kInt3) {
        c.q2 = *reinterpret_cast<const uint2*>(t + 8 * lane);
        c.h = *reinterpret_cast<const uint32_t*>(t + 512 + 4 * lane);
        c.s = *reinterpret_cast<const uint16_t*>(t + 768 + 2 * lane);
    } else if constexpr (FMT == kInt4) {
        c.d = *reinterpret_cast<const uint4*>(t + 16 * lane);
        c.s = *reinterpret_cast<const uint16_t*>(t + 1024 + 2 * lane);
    } else if constexpr (FMT == kFp8) {
        const uint4* p = reinterpret_cast<const uint4*>(t + 32 * lane);
        c.d0 = p[0];
        c.d1 = p[1];
        c.s = *reinterpret_cast<const float*>(t + 2048 + 4 * lane);
    } else {
        c.d = *reinterpret_cast<const uint4*>(t + 16 * lane);
        c.e8 = t[1024 + lane];
    }
    return c;
}

template <int FMT, bool FIRST>
__device__ __forceinline__ void accumulate(const LaneCodes<FMT>& c, float (&acc)[32])
{
    if constexpr (FMT == kInt3) {
        int3_accumulate<FIRST>(c.q2.x, c.q2.y, c.h, c.s, acc);
    } else if constexpr (FMT == kInt4) {
        const uint32_t d[4] = {c.d.x, c.d.y, c.d.z, c.d.w};
        int4_accumulate<FIRST>(d, c.s, acc);
    } else if constexpr (FMT == kFp8) {
        const uint32_t d[8] = {c.d0.x, c.d0.y, c.d0.z, c.d0.w, c.d1.x, c.d1.y, c.d1.z, c.d1.w};
        fp8_accumulate<FIRST>(d, c.s, acc);
    } else {
        const uint32_t d[4] = {c.d.x, c.d.y, c.d.z, c.d.w};
        mx_accumulate<FIRST>(d, c.e8, acc);
    }
}

// ------------------------------------------------------------ kernels ----

__device__ __forceinline__ void tail_zero(float (&acc)[32], size_t base, size_t n)
{
    const size_t valid = (base >= n) ? 0 : n - base;
#pragma unroll
    for (int e = 0; e < 32; ++e)
        if ((size_t)e >= valid) acc[e] = 0.0f;
}

__device__ __forceinline__ void store_sums_tail(float* __restrict__ sum_out, size_t base, size_t n, const float (&acc)[32])
{
#pragma unroll
    for (int e = 0; e < 32; ++e)
        if (base + e < n) sum_out[base + e] = acc[e];
}

template <int FMT, int DT>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ in, size_t n,
                                                       uint8_t* __restrict__ out, size_t tiles)
{
    const size_t tile = tile_index();
    if (tile >= tiles) return;
    const int lane = lane_id();
    float v[32];
    load_block<DT>(in, tile * kTile + (size_t)lane * kBlock, n, v);
    encode_store<FMT>(v, out + tile * TileBytes<FMT>::v, lane);
}

template <int FMT, int K>
__global__ __launch_bounds__(256) void reduce_kernel(StreamPtrs ins, size_t n, uint8_t* __restrict__ out,
                                                     float* __restrict__ sum_out, size_t tiles)
{
    const size_t tile = tile_index();
    if (tile >= tiles) return;
    const int lane = lane_id();
    const size_t off = tile * TileBytes<FMT>::v;
    LaneCodes<FMT> c[K];
#pragma unroll
    for (int k = 0; k < K; ++k) c[k] = load_codes<FMT>(ins.p[k] + off, lane);
    float acc[32];
    accumulate<FMT, true>(c[0], acc);
#pragma unroll
    for (int k = 1; k < K; ++k) accumulate<FMT, false>(c[k], acc);
    const size_t base = tile * kTile + (size_t)lane * kBlock;
    if (tile == tiles - 1 && (n % kTile) != 0) {   // wave-uniform: only the last tile
        tail_zero(acc, base, n);                   // positions >= n are +0
        if (sum_out) store_sums_tail(sum_out, base, n, acc);
    } else if (sum_out) {
        float4* p = reinterpret_cast<float4*>(sum_out + base);
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    }
    encode_store<FMT>(acc, out + off, lane);
}

// binary32 -> binary16 bits, RNE.  The empty asm pins x in a register so the
// compiler cannot fold the producing multiply into the conversion (an fma
// into f16 with a +0 addend would turn -0 products into +0).
__device__ __forceinline__ uint32_t f16_bits(float x)
{
    __asm__("" : "+v"(x));
    return __half_as_ushort(__float2half_rn(x));
}

template <int ODT>
__device__ __forceinline__ void store_block(void* __restrict__ out, size_t base, size_t n, const float (&d)[32])
{
    if (base + kBlock <= n) {
        if constexpr (ODT == kF32) {
            float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + base);
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = make_float4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
        } else {
            uint32_t w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (ODT == kBF16) {
                    __hip_bfloat162 b = __float22bfloat162_rn(make_float2(d[2 * i], d[2 * i + 1]));
                    w[i] = *reinterpret_cast<uint32_t*>(&b);
                } else {
                    w[i] = f16_bits(d[2 * i]) | (f16_bits(d[2 * i + 1]) << 16);
                }
            }
            uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + base);
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            if (base + e >= n) continue;
            if constexpr (ODT == kF32) static_cast<float*>(out)[base + e] = d[e];
            else if constexpr (ODT == kBF16)
                static_cast<uint16_t*>(out)[base + e] = __bfloat16_as_ushort(__float2bfloat16(d[e]));
            else static_cast<uint16_t*>(out)[base + e] = (uint16_t)f16_bits(d[e]);
        }
    }
}

template <int FMT, int ODT>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ in, size_t n,
                                                     void* __restrict__ out, size_t tiles)
{
    const size_t tile = tile_index();
    if (tile >= tiles) return;
    const int lane = lane_id();
    const LaneCodes<FMT> c = load_codes<FMT>(in + tile * TileBytes<FMT>::v, lane);
    float d[32];
    accumulate<FMT, true>(c, d);
    store_block<ODT>(out, tile * kTile + (size_t)lane * kBlock, n, d);
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ in, uint4* __restrict__ out, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = in[i], b = in[i + stride], c = in[i + 2 * stride], d = in[i + 3 * stride];
        out[i] = a; out[i + stride] = b; out[i + 2 * stride] = c; out[i + 3 * stride] = d;
    }
    for (; i < n16; i += stride) out[i] = in[i];
}

// ---------------------------------------------------------- launchers ----

static inline dim3 tile_grid(size_t tiles) { return dim3((unsigned)((tiles + kWavesPerGroup - 1) / kWavesPerGroup)); }

template <int FMT>
static hipError_t launch_quantize_fmt(int dt, const void* in, size_t n, void* out, size_t tiles, hipStream_t st)
{
    uint8_t* o = static_cast<uint8_t*>(out);
    switch (dt) {
    case kF32: hipLaunchKernelGGL((quantize_kernel<FMT, kF32>), tile_grid(tiles), dim3(256), 0, st, in, n, o, tiles); break;
    case kF16: hipLaunchKernelGGL((quantize_kernel<FMT, kF16>), tile_grid(tiles), dim3(256), 0, st, in, n, o, tiles); break;
    default:   hipLaunchKernelGGL((quantize_kernel<FMT, kBF16>), tile_grid(tiles), dim3(256), 0, st, in, n, o, tiles); break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize(int fmt, int dt, const void* in, size_t n, void* out, hipStream_t st)
{
    const size_t tiles = (n + kTile - 1) / kTile;
    switch (fmt) {
    case kInt4: return launch_quantize_fmt<kInt4>(dt, in, n, out, tiles, st);
    case kInt3: return launch_quantize_fmt<kInt3>(dt, in, n, out, tiles, st);
    case kFp8:  return launch_quantize_fmt<kFp8>(dt, in, n, out, tiles, st);
    default:    return launch_quantize_fmt<kMx4>(dt, in, n, out, tiles, st);
    }
}

template <int FMT, int K>
static hipError_t launch_reduce_k(const StreamPtrs& p, size_t n, void* out, float* sum, size_t tiles, hipStream_t st)
{
    hipLaunchKernelGGL((reduce_kernel<FMT, K>), tile_grid(tiles), dim3(256), 0, st, p, n,
                       static_cast<uint8_t*>(out), sum, tiles);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_reduce_fmt(const StreamPtrs& p, int k, size_t n, void* out, float* sum, size_t tiles,
                                    hipStream_t st)
{
    switch (k) {
    case 1:  return launch_reduce_k<FMT, 1>(p, n, out, sum, tiles, st);
    case 2:  return launch_reduce_k<FMT, 2>(p, n, out, sum, tiles, st);
    case 3:  return launch_reduce_k<FMT, 3>(p, n, out, sum, tiles, st);
    case 4:  return launch_reduce_k<FMT, 4>(p, n, out, sum, tiles, st);
    case 5:  return launch_reduce_k<FMT, 5>(p, n, out, sum, tiles, st);
    case 6:  return launch_reduce_k<FMT, 6>(p, n, out, sum, tiles, st);
    case 7:  return launch_reduce_k<FMT, 7>(p, n, out, sum, tiles, st);
    case 8:  return launch_reduce_k<FMT, 8>(p, n, out, sum, tiles, st);
    case 9:  return launch_reduce_k<FMT, 9>(p, n, out, sum, tiles, st);
    case 10: return launch_reduce_k<FMT, 10>(p, n, out, sum, tiles, st);
    case 11: return launch_reduce_k<FMT, 11>(p, n, out, sum, tiles, st);
    case 12: return launch_reduce_k<FMT, 12>(p, n, out, sum, tiles, st);
    case 13: return launch_reduce_k<FMT, 13>(p, n, out, sum, tiles, st);
    case 14: return launch_reduce_k<FMT, 14>(p, n, out, sum, tiles, st);
    case 15: return launch_reduce_k<FMT, 15>(p, n, out, sum, tiles, st);
    default: return launch_reduce_k<FMT, 16>(p, n, out, sum, tiles, st);
    }
}

hipError_t launch_reduce(int fmt, const StreamPtrs& p, int k, size_t n, void* out, float* sum, hipStream_t st)
{
    const size_t tiles = (n + kTile - 1) / kTile;
    switch (fmt) {
    case kInt4: return launch_reduce_fmt<kInt4>(p, k, n, out, sum, tiles, st);
    case kInt3: return launch_reduce_fmt<kInt3>(p, k, n, out, sum, tiles, st);
    case kFp8:  return launch_reduce_fmt<kFp8>(p, k, n, out, sum, tiles, st);
    default:    return launch_reduce_fmt<kMx4>(p, k, n, out, sum, tiles, st);
    }
}

template <int FMT>
static hipError_t launch_unpack_fmt(const void* in, size_t n, int dt, void* out, size_t tiles, hipStream_t st)
{
    const uint8_t* i = static_cast<const uint8_t*>(in);
    switch (dt) {
    case kF32: hipLaunchKernelGGL((unpack_kernel<FMT, kF32>), tile_grid(tiles), dim3(256), 0, st, i, n, out, tiles); break;
    case kF16: hipLaunchKernelGGL((unpack_kernel<FMT, kF16>), tile_grid(tiles), dim3(256), 0, st, i, n, out, tiles); break;
    default:   hipLaunchKernelGGL((unpack_kernel<FMT, kBF16>), tile_grid(tiles), dim3(256), 0, st, i, n, out, tiles); break;
    }
    return hipGetLastError();
}

hipError_t launch_unpack(int fmt, const void* in, size_t n, int dt, void* out, hipStream_t st)
{
    const size_t tiles = (n + kTile - 1) / kTile;
    switch (fmt) {
    case kInt4: return launch_unpack_fmt<kInt4>(in, n, dt, out, tiles, st);
    case kInt3: return launch_unpack_fmt<kInt3>(in, n, dt, out, tiles, st);
    case kFp8:  return launch_unpack_fmt<kFp8>(in, n, dt, out, tiles, st);
    default:    return launch_unpack_fmt<kMx4>(in, n, dt, out, tiles, st);
    }
}

hipError_t launch_copy(const void* in, void* out, size_t bytes, hipStream_t st)
{
    const size_t n16 = bytes / 16;
    size_t blocks = (n16 + 4 * 256 - 1) / (4 * 256);
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint4*>(in),
                       static_cast<uint4*>(out), n16);
    return hipGetLastError();
}

}  // namespace rc
