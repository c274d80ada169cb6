// rc_kernels.hip -- gfx950 kernels of the codec and their launchers.
//
// One wave64 per 2048-element tile, lane l = block l; 256-thread workgroups
// (four waves).  Packed tiles are read and written with per-lane buffer
// accesses that are contiguous across the wave (code words at lane * bytes
// per block, scales at lane * scale bytes); the 64- or 128-byte element rows
// of quantize input and unpack output are regrouped through LDS so that HBM
// sees wave-coalesced 16-byte chunks.
#include "rc_device.hpp"
#include "rc_internal.hpp"

#ifndef RC_GROUPS_PER_CU
#define RC_GROUPS_PER_CU 256                       // grid cap, workgroups per CU
#endif
#ifndef RC_REDUCE_WAVES
#define RC_REDUCE_WAVES 8                          // reduce occupancy target (waves per SIMD), INT / MX
#endif
#ifndef RC_REDUCE_BATCH
#define RC_REDUCE_BATCH 2                          // streams loaded together, INT / MX
#endif
#ifndef RC_FP8_REDUCE_BATCH
#define RC_FP8_REDUCE_BATCH 4                      // streams loaded together, FP8
#endif
#ifndef RC_FP8_REDUCE_WAVES
#define RC_FP8_REDUCE_WAVES 4                      // reduce occupancy target, FP8
#endif
#ifndef RC_REDUCE_SCHED_BARRIER
#define RC_REDUCE_SCHED_BARRIER 1                  // keep each batch's loads below the previous batch
#endif
#ifndef RC_QUANT_WAVES
#define RC_QUANT_WAVES 8                           // quantize occupancy target, waves per SIMD
#endif
#ifndef RC_QUANT_LDS
#define RC_QUANT_LDS 1                             // quantize input regrouped through LDS
#endif
#ifndef RC_UNPACK_LDS
#define RC_UNPACK_LDS 1                            // unpack output regrouped through LDS
#endif

namespace rc {

template <int FMT> struct TileBytes;
template <> struct TileBytes<kInt4> { static constexpr int v = 1152; };
template <> struct TileBytes<kInt3> { static constexpr int v = 896; };
template <> struct TileBytes<kFp8> { static constexpr int v = 2304; };
template <> struct TileBytes<kMx4> { static constexpr int v = 1088; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Per-lane code words of one block of one stream.
template <int FMT> struct LaneCodes;
template <> struct LaneCodes<kInt3> { uint2 q2; uint32_t h; uint32_t s; };
template <> struct LaneCodes<kInt4> { uint4 d; uint32_t s; };
template <> struct LaneCodes<kFp8> { uint4 d0, d1; float s; };
template <> struct LaneCodes<kMx4> { uint4 d; uint32_t e8; };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------ buffer access ----
// Tiles are addressed through a buffer descriptor built in scalar registers
// from the (wave-uniform) tile address, and a per-lane byte offset that
// does not change from tile to tile: no per-lane 64-bit address arithmetic.
// Loads and stores carry the non-temporal hint.

constexpr int kNT = 2;                              // aux bits: nt
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc span_rsrc(const void* base, size_t off, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint8_t*>(base) + off), (short)0,
                                             (int)bytes, 0x00020000);
}

// The per-lane code words of one block, read from a stream's tile.
template <int FMT>
__device__ __forceinline__ LaneCodes<FMT> load_codes_buf(Rsrc r, uint32_t lane)
{
    LaneCodes<FMT> c;
    if constexpr (FMT == kInt3) {
        const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8u, 0, kNT);
        c.q2 = make_uint2(q.x, q.y);
        c.h = __builtin_amdgcn_raw_buffer_load_b32(r, 512u + lane * 4u, 0, kNT);
        c.s = __builtin_amdgcn_raw_buffer_load_b16(r, 768u + lane * 2u, 0, kNT);
    } else if constexpr (FMT == kInt4) {
        const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 0, kNT);
        c.d = make_uint4(d.x, d.y, d.z, d.w);
        c.s = __builtin_amdgcn_raw_buffer_load_b16(r, 1024u + lane * 2u, 0, kNT);
    } else if constexpr (FMT == kFp8) {
        const u32x4 d0 = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 32u, 0, kNT);
        const u32x4 d1 = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 32u + 16u, 0, kNT);
        c.d0 = make_uint4(d0.x, d0.y, d0.z, d0.w);
        c.d1 = make_uint4(d1.x, d1.y, d1.z, d1.w);
        c.s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 2048u + lane * 4u, 0, kNT));
    } else {
        const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 0, kNT);
        c.d = make_uint4(d.x, d.y, d.z, d.w);
        c.e8 = __builtin_amdgcn_raw_buffer_load_b8(r, 1024u + lane, 0, kNT);
    }
    return c;
}

// Requantize the 32 values of lane's block and store its code words.
template <int FMT>
__device__ __forceinline__ void encode_store_buf(const float (&v)[32], Rsrc r, uint32_t lane)
{
    if constexpr (FMT == kInt3) {
        const Int3Words w = int3_encode_block(v);
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){w.w0, w.w1}, r, lane * 8u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b32(w.h, r, 512u + lane * 4u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w.sbits, r, 768u + lane * 2u, 0, kNT);
    } else if constexpr (FMT == kInt4) {
        const Int4Words w = int4_encode_block(v);
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){w.d[0], w.d[1], w.d[2], w.d[3]}, r, lane * 16u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w.sbits, r, 1024u + lane * 2u, 0, kNT);
    } else if constexpr (FMT == kFp8) {
        const Fp8Words w = fp8_encode_block(v);
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){w.d[0], w.d[1], w.d[2], w.d[3]}, r, lane * 32u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){w.d[4], w.d[5], w.d[6], w.d[7]}, r, lane * 32u + 16u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(w.s), r, 2048u + lane * 4u, 0, kNT);
    } else {
        const MxWords w = mx_encode_block(v);
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){w.d[0], w.d[1], w.d[2], w.d[3]}, r, lane * 16u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)w.e8, r, 1024u + lane, 0, kNT);
    }
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

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// ------------------------------------------------------------ kernels ----

// Tile walk: each wave processes tiles first, first + stride, ...; `first`
// and `stride` are wave-uniform (scalar registers), so tile addresses and
// buffer descriptors are built with scalar arithmetic.
struct TileWalk {
    size_t first, stride;
    int lane, w;
};

__device__ __forceinline__ TileWalk tile_walk()
{
    TileWalk t;
    t.w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    t.lane = lane_id();
    t.first = (size_t)blockIdx.x * kWavesPerGroup + (size_t)t.w;
    t.stride = (size_t)gridDim.x * kWavesPerGroup;
    return t;
}

// The 32 input elements of lane's block from the CPB 16-byte chunks of its
// row, widened exactly to binary32.
template <int DT, int CPB>
__device__ __forceinline__ void widen_chunks(const u32x4 (&c)[CPB], float (&v)[32])
{
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[4 * i] = __uint_as_float(c[i].x); v[4 * i + 1] = __uint_as_float(c[i].y);
            v[4 * i + 2] = __uint_as_float(c[i].z); v[4 * i + 3] = __uint_as_float(c[i].w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) widen8<DT>(c[i], v + 8 * i);
    }
}

// One wave quantizes one whole tile per iteration.  With RC_QUANT_LDS the
// tile's input is read as wave-coalesced 16-byte chunks (chunk c by lane
// c % 64) and regrouped through a padded LDS row per block; otherwise each
// lane reads its own block's 16-byte chunks directly.  Codes and scales go
// out through buffer stores.  Latency is covered by the other waves of the
// SIMD (no in-wave prefetch).  The partial last tile, if any, is done after
// the loop by the wave whose walk would reach it.
template <int FMT, int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RC_QUANT_WAVES)))
void quantize_kernel(const void* __restrict__ in, size_t n, uint8_t* __restrict__ out, size_t tiles)
{
    constexpr int ES = (DT == kF32) ? 4 : 2;
    constexpr int TIB = kTile * ES;            // input bytes of one tile
    constexpr int BB = kBlock * ES;            // input bytes of one block
    constexpr int CPB = BB / 16;               // 16-byte chunks per block
    constexpr int TB = TileBytes<FMT>::v;
    const TileWalk tw = tile_walk();
    const uint32_t lane = (uint32_t)tw.lane;
    const size_t full = n / kTile;
#if RC_QUANT_LDS
    constexpr int ROW = BB + 16;               // padded LDS row: conflict-free 16-byte reads
    __shared__ __attribute__((aligned(16))) uint8_t sm[kWavesPerGroup][64 * ROW];
    uint8_t* lds = sm[tw.w];
#endif
    for (size_t tile = tw.first; tile < full; tile += tw.stride) {
        const Rsrc src = span_rsrc(in, tile * TIB, TIB);
        u32x4 c[CPB];
        float v[32];
#if RC_QUANT_LDS
#pragma unroll
        for (int i = 0; i < CPB; ++i) c[i] = __builtin_amdgcn_raw_buffer_load_b128(src, (64u * i + lane) * 16u, 0, kNT);
        wave_lds_sync();                       // the previous tile's rows are fully read
#pragma unroll
        for (int i = 0; i < CPB; ++i) {
            const uint32_t ch = 64u * i + lane;
            *reinterpret_cast<u32x4*>(lds + (ch / CPB) * ROW + (ch % CPB) * 16) = c[i];
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < CPB; ++i) c[i] = *reinterpret_cast<const u32x4*>(lds + lane * ROW + 16 * i);
#else
#pragma unroll
        for (int i = 0; i < CPB; ++i) c[i] = __builtin_amdgcn_raw_buffer_load_b128(src, lane * BB + 16u * i, 0, kNT);
#endif
        widen_chunks<DT, CPB>(c, v);
        encode_store_buf<FMT>(v, span_rsrc(out, tile * TB, TB), lane);
    }
    if (full != tiles && full % tw.stride == tw.first) {     // the partial last tile
        float v[32];
        load_block<DT>(in, full * kTile + (size_t)lane * kBlock, n, v);
        encode_store_buf<FMT>(v, span_rsrc(out, full * TB, TB), lane);
    }
}

// Streams whose codes are loaded together before they are accumulated.
// FP8's encoder holds more registers: it runs at fewer waves per SIMD.
template <int FMT> struct ReduceBatch { static constexpr int v = (FMT == kFp8) ? RC_FP8_REDUCE_BATCH : RC_REDUCE_BATCH; };
template <int FMT> struct ReduceWaves { static constexpr int v = (FMT == kFp8) ? RC_FP8_REDUCE_WAVES : RC_REDUCE_WAVES; };

// acc = the K streams' decoded values of lane's block of `tile`, added in
// stream order in binary32.
template <int FMT, int K>
__device__ __forceinline__ void reduce_tile(const StreamPtrs& ins, size_t tile, uint32_t lane, float (&acc)[32])
{
    constexpr int TB = TileBytes<FMT>::v;
    constexpr int B = (K < ReduceBatch<FMT>::v) ? K : ReduceBatch<FMT>::v;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += B) {
        LaneCodes<FMT> c[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (k0 + j < K) c[j] = load_codes_buf<FMT>(span_rsrc(ins.p[k0 + j], tile * TB, TB), lane);
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (k0 + j >= K) break;
            if (k0 + j == 0) accumulate<FMT, true>(c[j], acc);
            else accumulate<FMT, false>(c[j], acc);
        }
        // keep the next batch's loads below this batch's arithmetic (bounds
        // the registers held by codes in flight)
        if (RC_REDUCE_SCHED_BARRIER && k0 + B < K) __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ void store_sums(float* __restrict__ sum_out, size_t tile, uint32_t lane, const float (&acc)[32])
{
    const Rsrc r = span_rsrc(sum_out, tile * (kTile * 4), kTile * 4);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){__float_as_uint(acc[4 * i]), __float_as_uint(acc[4 * i + 1]),
                                                       __float_as_uint(acc[4 * i + 2]), __float_as_uint(acc[4 * i + 3])},
                                               r, lane * 128u + 16u * i, 0, kNT);
}

// Each wave reduces whole tiles: the codes of the K streams are read with
// per-lane coalesced loads (ReduceBatch streams at a time), decoded and
// accumulated in registers, and the sums requantized in place.  No LDS and
// no in-wave prefetch: latency is covered by the other waves of the SIMD.
// The partial last tile (if any) is done after the loop by the wave whose
// walk would reach it.
template <int FMT, int K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ReduceWaves<FMT>::v)))
void reduce_kernel(StreamPtrs ins, size_t n, uint8_t* __restrict__ out, float* __restrict__ sum_out, size_t tiles)
{
    constexpr int TB = TileBytes<FMT>::v;
    const TileWalk tw = tile_walk();
    const uint32_t lane = (uint32_t)tw.lane;
    const size_t full = n / kTile;
    if (sum_out) {
        for (size_t tile = tw.first; tile < full; tile += tw.stride) {
            float acc[32];
            reduce_tile<FMT, K>(ins, tile, lane, acc);
            store_sums(sum_out, tile, lane, acc);
            encode_store_buf<FMT>(acc, span_rsrc(out, tile * TB, TB), lane);
        }
    } else {
        for (size_t tile = tw.first; tile < full; tile += tw.stride) {
            float acc[32];
            reduce_tile<FMT, K>(ins, tile, lane, acc);
            encode_store_buf<FMT>(acc, span_rsrc(out, tile * TB, TB), lane);
        }
    }
    if (full != tiles && full % tw.stride == tw.first) {
        float acc[32];
        reduce_tile<FMT, K>(ins, full, lane, acc);
        const size_t base = full * kTile + (size_t)lane * kBlock;
        tail_zero(acc, base, n);                   // positions >= n are +0
        if (sum_out) store_sums_tail(sum_out, base, n, acc);
        encode_store_buf<FMT>(acc, span_rsrc(out, full * TB, TB), lane);
    }
}

// binary32 -> binary16 bits, RNE.  The empty asm pins x in a register so the
// compiler cannot fold the producing multiply into the conversion (an fma
// into f16 with a +0 addend would turn -0 products into +0).
__device__ __forceinline__ uint32_t f16_bits(float x)
{
    __asm__("" : "+v"(x));
    return __half_as_ushort(__float2half_rn(x));
}

// The 32 decoded values of one block as output words (16 for 2-byte dtypes).
template <int ODT>
__device__ __forceinline__ void out_words(const float (&d)[32], uint32_t (&w)[32])
{
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if constexpr (ODT == kF32) w[i] = __float_as_uint(d[i]);
        else if (i < 16) {
            if constexpr (ODT == kBF16) {
                __hip_bfloat162 b = __float22bfloat162_rn(make_float2(d[2 * i], d[2 * i + 1]));
                w[i] = *reinterpret_cast<uint32_t*>(&b);
            } else {
                w[i] = f16_bits(d[2 * i]) | (f16_bits(d[2 * i + 1]) << 16);
            }
        }
    }
}

template <int ODT>
__device__ __forceinline__ void store_block_guarded(void* __restrict__ out, size_t base, size_t n, const float (&d)[32])
{
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        if (base + e >= n) continue;
        if constexpr (ODT == kF32) static_cast<float*>(out)[base + e] = d[e];
        else if constexpr (ODT == kBF16)
            static_cast<uint16_t*>(out)[base + e] = __bfloat16_as_ushort(__float2bfloat16(d[e]));
        else static_cast<uint16_t*>(out)[base + e] = (uint16_t)f16_bits(d[e]);
    }
}

// One wave unpacks one tile per iteration: codes in through per-lane buffer
// loads, decoded values out either through a padded LDS row per block and
// wave-coalesced 16-byte stores (RC_UNPACK_LDS) or straight from each lane.
template <int FMT, int ODT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8)))
void unpack_kernel(const uint8_t* __restrict__ in, size_t n, void* __restrict__ out, size_t tiles)
{
    constexpr int TB = TileBytes<FMT>::v;
    constexpr int ES = (ODT == kF32) ? 4 : 2;
    constexpr int OB = kBlock * ES;            // output bytes of one block
    constexpr int CPB = OB / 16;
    const TileWalk tw = tile_walk();
    const uint32_t lane = (uint32_t)tw.lane;
    const size_t full = n / kTile;
#if RC_UNPACK_LDS
    constexpr int ROW = OB + 16;
    __shared__ __attribute__((aligned(16))) uint8_t sm[kWavesPerGroup][64 * ROW];
    uint8_t* lds = sm[tw.w];
#endif
    for (size_t tile = tw.first; tile < full; tile += tw.stride) {
        float d[32];
        accumulate<FMT, true>(load_codes_buf<FMT>(span_rsrc(in, tile * TB, TB), lane), d);
        uint32_t wd[32];
        out_words<ODT>(d, wd);
        const Rsrc dst = span_rsrc(out, tile * (size_t)(kTile * ES), kTile * ES);
#if RC_UNPACK_LDS
        wave_lds_sync();                       // the previous tile's rows are fully read
#pragma unroll
        for (int i = 0; i < CPB; ++i)
            *reinterpret_cast<u32x4*>(lds + lane * ROW + 16 * i) =
                (u32x4){wd[4 * i], wd[4 * i + 1], wd[4 * i + 2], wd[4 * i + 3]};
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < CPB; ++i) {
            const uint32_t ch = 64u * i + lane;
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(lds + (ch / CPB) * ROW + (ch % CPB) * 16),
                                                   dst, ch * 16u, 0, kNT);
        }
#else
#pragma unroll
        for (int i = 0; i < CPB; ++i)
            __builtin_amdgcn_raw_buffer_store_b128((u32x4){wd[4 * i], wd[4 * i + 1], wd[4 * i + 2], wd[4 * i + 3]},
                                                   dst, lane * OB + 16u * i, 0, kNT);
#endif
    }
    if (full != tiles && full % tw.stride == tw.first) {     // the partial last tile
        float d[32];
        accumulate<FMT, true>(load_codes_buf<FMT>(span_rsrc(in, full * TB, TB), lane), d);
        store_block_guarded<ODT>(out, full * kTile + (size_t)lane * kBlock, n, d);
    }
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(in + i), out + i);
}

// ---------------------------------------------------------- launchers ----


// Grid of four-wave workgroups: one tile per wave up to RC_GROUPS_PER_CU
// workgroups per compute unit (1 GiB of bf16 input on 256 CUs; measured
// faster there than a 4x smaller grid walking 4 tiles per wave); beyond that
// each wave walks several tiles.
static inline dim3 tile_grid(size_t tiles)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const size_t groups = (tiles + kWavesPerGroup - 1) / kWavesPerGroup;
    const size_t cap = (size_t)RC_GROUPS_PER_CU * (size_t)(cus > 0 ? cus : 256);
    return dim3((unsigned)(groups < cap ? groups : cap));
}

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
    size_t blocks = (n16 + 255) / 256;         // one 16-byte chunk per thread
    if (blocks > (1u << 20)) blocks = 1u << 20;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const u32x4*>(in),
                       static_cast<u32x4*>(out), n16);
    return hipGetLastError();
}

}  // namespace rc
