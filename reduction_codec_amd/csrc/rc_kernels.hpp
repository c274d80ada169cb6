// rc_kernels.hpp -- kernel templates of the codec and their launcher
// templates, for every (element format, scale type, block size).  Included
// only by the instantiation units (rc_inst_*.hip); everything else sees the
// launcher declarations of rc_launch.hpp.
//
// One wave64 per 2048-element tile, lane l = elements 32l..32l+31;
// 256-thread workgroups (four waves), one-wave ones for the INT reduce.
// Packed tiles are read and written with per-lane buffer accesses that are
// contiguous across the wave (code words at lane * bytes per 32 elements,
// FP8 codes as two 16-byte planes, scales at lane * scale bytes per lane);
// the 64- or 128-byte element rows of quantize input and unpack output are
// regrouped through LDS so that HBM sees wave-coalesced 16-byte chunks.
#pragma once

#include "rc_device.hpp"
#include "rc_launch.hpp"

#ifndef RC_GROUPS_PER_CU
#define RC_GROUPS_PER_CU 256                       // grid cap, four-wave workgroups per CU
#endif
#ifndef RC_REDUCE_GROUPS_PER_CU
#define RC_REDUCE_GROUPS_PER_CU RC_GROUPS_PER_CU   // reduce grid cap, in four-wave-group units per CU
#endif
#ifndef RC_QUANT_GROUPS_PER_CU
#define RC_QUANT_GROUPS_PER_CU RC_GROUPS_PER_CU    // quantize grid cap, four-wave groups per CU
#endif
#ifndef RC_REDUCE_WAVES
#define RC_REDUCE_WAVES 8                          // reduce occupancy target (waves per SIMD), INT / MX
#endif
#ifndef RC_MX_REDUCE_WAVES
#define RC_MX_REDUCE_WAVES 6                       // the same, MXFP4 with 4 or more streams (see ReduceWaves)
#endif
#ifndef RC_REDUCE_ROLL
#define RC_REDUCE_ROLL 1                           // rolling stream loads in the unrolled INT / MX reduce (ReduceRoll)
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
#ifndef RC_QUANT_F32_HALVES
#define RC_QUANT_F32_HALVES 1                      // fp32 quantize input regrouped in two halves
#endif
#ifndef RC_QUANT_F32_WAVES
#define RC_QUANT_F32_WAVES 4                       // fp32 quantize occupancy target (5, 6: no gain)
#endif
#ifndef RC_QUANT_LDS
#define RC_QUANT_LDS 1                             // quantize input regrouped through LDS
#endif
#ifndef RC_RT_UNROLL_COMMON
#define RC_RT_UNROLL_COMMON 1                      // variants: 2, 4, 8 streams unrolled too
#endif
#ifndef RC_GEMV_ROWS
#define RC_GEMV_ROWS 2                             // rows per wave of the GEMV
#endif
#ifndef RC_GEMV_DOT2
#define RC_GEMV_DOT2 1                             // bf16 x: v_dot2_f32_bf16 on bf16 weight pairs
#endif
#ifndef RC_UNPACK_LDS
#define RC_UNPACK_LDS 1                            // unpack output regrouped through LDS
#endif

namespace rc {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Per-lane code words of 32 elements of one stream (scales load separately).
// FP8 codes sit in two 1024-byte planes (the first and the last 16 codes of
// every 32-element group), so each of a lane's two 16-byte accesses is
// contiguous across the wave.
template <int FMT> struct LaneCodes;
template <> struct LaneCodes<kInt3> { uint32_t w0, w1, h; };
template <> struct LaneCodes<kInt4> { uint32_t d[4]; };
template <> struct LaneCodes<kFp8> { uint32_t d[8]; };
template <> struct LaneCodes<kBf8> { uint32_t d[8]; };
template <> struct LaneCodes<kMx4> { uint32_t d[4]; };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------ buffer access ----
// Tiles are addressed through a buffer descriptor built in scalar registers
// from the (wave-uniform) tile address, and a per-lane byte offset that
// does not change from tile to tile: no per-lane 64-bit address arithmetic.
// Loads and stores carry the non-temporal hint.

constexpr int kNT = 2;                              // aux bits: nt
// Element rows written by unpack: nt with sc1 (device scope), measured
// 2-4 % faster than nt alone there (and slower for the packed outputs of
// quantize and reduce, and for the fused all-reduce's output rows).
constexpr int kRowStore = 18;
// Packed tiles read by unpack: where the packed input is small next to the
// output (the 3- and 4-bit formats, at most 0.5625 packed bytes per element
// against 2-4 bytes written, and FP8 into fp32) plain loads beat nt ones
// from 65,536 tiles on (INT3 to bf16 at 1 GiB: 243 -> 215 us; FP8 to fp32:
// 5-7 %), and lose 4-6 % below 96 MiB; FP8 into bf16 or fp16 keeps nt loads
// at every size.
// Quantize and reduce keep nt loads (plain ones measured 2-9 % slower).
constexpr int kPlainLoad = 0;
constexpr size_t kUnpackPlainLoadTiles = size_t(1) << 16;
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc span_rsrc(const void* base, size_t off, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint8_t*>(base) + off), (short)0,
                                             (int)bytes, 0x00020000);
}

// The per-lane code words of 32 elements, read from a stream's tile.
template <int FMT, int AUX = kNT>
__device__ __forceinline__ LaneCodes<FMT> load_codes_buf(Rsrc r, uint32_t lane)
{
    LaneCodes<FMT> c;
    if constexpr (FMT == kInt3) {
        const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8u, 0, AUX);
        c.w0 = q.x;
        c.w1 = q.y;
        c.h = __builtin_amdgcn_raw_buffer_load_b32(r, 512u + lane * 4u, 0, AUX);
    } else if constexpr (FMT == kFp8 || FMT == kBf8) {
        const u32x4 d0 = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 0, AUX);
        const u32x4 d1 = __builtin_amdgcn_raw_buffer_load_b128(r, 1024u + lane * 16u, 0, AUX);
        c.d[0] = d0.x; c.d[1] = d0.y; c.d[2] = d0.z; c.d[3] = d0.w;
        c.d[4] = d1.x; c.d[5] = d1.y; c.d[6] = d1.z; c.d[7] = d1.w;
    } else {
        const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 0, AUX);
        c.d[0] = d.x; c.d[1] = d.y; c.d[2] = d.z; c.d[3] = d.w;
    }
    return c;
}

// Raw scale bits of the lane's blocks: one scale (32-element blocks), two
// adjacent scales (16), or the pair's shared scale (64), read at the
// scale region's offset.
template <int FMT, int SC, int BL, int AUX = kNT>
__device__ __forceinline__ void load_scale_bits(Rsrc r, uint32_t lane, uint32_t (&bits)[Halves<BL>::v])
{
    constexpr uint32_t base = Fmt<FMT>::code_bytes;
    constexpr uint32_t SB = ScaleBytes<SC>::v;
    if constexpr (BL == 16) {
        if constexpr (SB == 2) {
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, base + lane * 4u, 0, AUX);
            bits[0] = w & 0xFFFFu; bits[1] = w >> 16;
        } else if constexpr (SB == 4) {
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, base + lane * 8u, 0, AUX);
            bits[0] = w.x; bits[1] = w.y;
        } else {
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b16(r, base + lane * 2u, 0, AUX);
            bits[0] = w & 0xFFu; bits[1] = w >> 8;
        }
    } else {
        const uint32_t idx = (BL == 64) ? (lane >> 1) : lane;
        if constexpr (SB == 2) bits[0] = __builtin_amdgcn_raw_buffer_load_b16(r, base + idx * 2u, 0, AUX);
        else if constexpr (SB == 4) bits[0] = __builtin_amdgcn_raw_buffer_load_b32(r, base + idx * 4u, 0, AUX);
        else bits[0] = __builtin_amdgcn_raw_buffer_load_b8(r, base + idx, 0, AUX);
    }
}

// Codes and decode multipliers of 32 elements of one stream.
template <int FMT, int SC, int BL>
struct LaneBlock {
    LaneCodes<FMT> c;
    uint32_t sbits[Halves<BL>::v];
};

template <int FMT, int SC, int BL, int AUX = kNT>
__device__ __forceinline__ LaneBlock<FMT, SC, BL> load_lane_block(Rsrc r, uint32_t lane)
{
    LaneBlock<FMT, SC, BL> b;
    b.c = load_codes_buf<FMT, AUX>(r, lane);
    load_scale_bits<FMT, SC, BL, AUX>(r, lane, b.sbits);
    return b;
}

// Exponent P at which the reduce holds its FP32 sums: value * 2^-P.  INT
// codes with FP16 scales decode as q/2 (INT3) or q 2^-9 (INT4); keeping the
// sums at that scale makes the decode multiplier the fp16 scale itself and
// the requantize multiplier the reciprocal itself.  Exact: every sum is a
// multiple of at least 2^-34 (codes times fp16 scales >= 2^-24, then 2^-9),
// far above the binary32 subnormal range, so the scaling commutes with every
// rounding.
template <int FMT, int SC> struct SumScale {
    static constexpr int v = SC == kS16 ? (FMT == kInt3 ? 1 : (FMT == kInt4 ? 9 : 0)) : 0;
};

// acc (+)= decoded values of the lane's 32 elements (times 2^-P).  ROUNDED,
// the default with E8M0 scales: every product is rounded before it is added,
// and INT3 codes decode as q with multiplier 2^e.  The same result as the fma
// while code * 2^e is a binary32 number, and still the definition where it is
// not: E8M0 bytes from 2^120 (E4M3), 2^113 (E5M2), 2^126 (INT4, E2M1) or
// 2^127 (INT3, whose usual multiplier 2^(e + 1) would itself be infinite) on.
// The encoder never writes those, but any packed bytes can hold them.  E2M1
// codes take 2^e as the conversion's scale operand, which rounds the product
// itself (one add per element, as with the fma); the other formats pay a
// multiply and an add.  The fused kernel, which decodes only its own codes,
// keeps the fma.
template <int FMT, int SC, int BL, bool FIRST, int P = 0, bool ROUNDED = (SC == kSE8)>
__device__ __forceinline__ void accumulate(const LaneBlock<FMT, SC, BL>& b, float (&acc)[32])
{
    constexpr int H = Halves<BL>::v;
    if constexpr (SC == kSE8 && ROUNDED) {
        float dm[H];
#pragma unroll
        for (int h = 0; h < H; ++h) dm[h] = e8m0_mult<0>(b.sbits[h]);       // 2^e
        if constexpr (FMT == kInt3) int3_accumulate<FIRST, H, true>(b.c.w0, b.c.w1, b.c.h, dm, acc);
        else if constexpr (FMT == kInt4) int4_accumulate<FIRST, H, true>(b.c.d, 512.0f, dm, acc);
        else if constexpr (FMT == kFp8 || FMT == kBf8) fp8_accumulate<FMT, SC, FIRST, H, true>(b.c.d, dm, acc);
        else mx_accumulate<FIRST, H, true>(b.c.d, dm, acc);
        return;
    }
    float dm[H];
#pragma unroll
    for (int h = 0; h < H; ++h) dm[h] = dec_mult<FMT, SC, P>(b.sbits[h]);
    if constexpr (FMT == kInt3) {
        int3_accumulate<FIRST, H>(b.c.w0, b.c.w1, b.c.h, dm, acc);
    } else if constexpr (FMT == kInt4) {
        // E8M0: the codes decode as q through the conversion's scale operand
        // 512 (2^(e+9) overflows for e > 118); FP16: as q 2^-9.
        int4_accumulate<FIRST, H>(b.c.d, SC == kSE8 ? 512.0f : 1.0f, dm, acc);
    } else if constexpr (FMT == kFp8 || FMT == kBf8) {
        fp8_accumulate<FMT, SC, FIRST, H>(b.c.d, dm, acc);
    } else {
        mx_accumulate<FIRST, H>(b.c.d, dm, acc);
    }
}

// Quantize the lane's 32 values (held at 2^-P of their value) into its code
// words and scale bits (in registers).  NARROW: the values are widened bf16
// or fp16 (at most 11 significant bits), which the FP8 encoder exploits.
template <int FMT, int SC, int BL, int P = 0, bool NARROW = false>
__device__ __forceinline__ LaneBlock<FMT, SC, BL> encode_lane(const float (&v)[32])
{
    constexpr int H = Halves<BL>::v;
    float a[H];
    lane_absmax<BL>(v, a);
    EncScale sc[H];
#pragma unroll
    for (int h = 0; h < H; ++h) sc[h] = enc_scale<FMT, SC>(P ? a[h] * (float)(1u << P) : a[h]);   // exact
    LaneBlock<FMT, SC, BL> b;
#pragma unroll
    for (int h = 0; h < H; ++h) b.sbits[h] = sc[h].bits;
    if constexpr (FMT == kInt3) {
        const Int3Words w = int3_encode<H, SC == kSE8, P>(v, sc);
        b.c.w0 = w.w0; b.c.w1 = w.w1; b.c.h = w.h;
    } else if constexpr (FMT == kInt4) {
        int4_encode<H, P>(v, sc, b.c.d);
    } else if constexpr (FMT == kFp8 || FMT == kBf8) {
        fp8_encode<FMT, SC, H, NARROW>(v, sc, b.c.d);
    } else {
        mx_encode<H>(v, sc, b.c.d);
    }
    return b;
}

// Store the lane's code words and scale(s) into a tile.
template <int FMT, int SC, int BL>
__device__ __forceinline__ void store_lane_block(const LaneBlock<FMT, SC, BL>& b, Rsrc r, uint32_t lane)
{
    if constexpr (FMT == kInt3) {
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){b.c.w0, b.c.w1}, r, lane * 8u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b32(b.c.h, r, 512u + lane * 4u, 0, kNT);
    } else if constexpr (FMT == kFp8 || FMT == kBf8) {
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){b.c.d[0], b.c.d[1], b.c.d[2], b.c.d[3]}, r, lane * 16u, 0, kNT);
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){b.c.d[4], b.c.d[5], b.c.d[6], b.c.d[7]}, r, 1024u + lane * 16u, 0, kNT);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){b.c.d[0], b.c.d[1], b.c.d[2], b.c.d[3]}, r, lane * 16u, 0, kNT);
    }
    constexpr uint32_t base = Fmt<FMT>::code_bytes;
    constexpr uint32_t SB = ScaleBytes<SC>::v;
    if constexpr (BL == 16) {
        if constexpr (SB == 2) __builtin_amdgcn_raw_buffer_store_b32(b.sbits[0] | (b.sbits[1] << 16), r, base + lane * 4u, 0, kNT);
        else if constexpr (SB == 4) __builtin_amdgcn_raw_buffer_store_b64((u32x2){b.sbits[0], b.sbits[1]}, r, base + lane * 8u, 0, kNT);
        else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(b.sbits[0] | (b.sbits[1] << 8)), r, base + lane * 2u, 0, kNT);
    } else if constexpr (BL == 32) {
        if constexpr (SB == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b.sbits[0], r, base + lane * 2u, 0, kNT);
        else if constexpr (SB == 4) __builtin_amdgcn_raw_buffer_store_b32(b.sbits[0], r, base + lane * 4u, 0, kNT);
        else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b.sbits[0], r, base + lane, 0, kNT);
    } else if ((lane & 1u) == 0u) {                  // 64: the even lane of the pair stores
        const uint32_t idx = lane >> 1;
        if constexpr (SB == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b.sbits[0], r, base + idx * 2u, 0, kNT);
        else if constexpr (SB == 4) __builtin_amdgcn_raw_buffer_store_b32(b.sbits[0], r, base + idx * 4u, 0, kNT);
        else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b.sbits[0], r, base + idx, 0, kNT);
    }
}

template <int FMT, int SC, int BL, int P = 0, bool NARROW = false>
__device__ __forceinline__ void encode_store_buf(const float (&v)[32], Rsrc r, uint32_t lane)
{
    store_lane_block<FMT, SC, BL>(encode_lane<FMT, SC, BL, P, NARROW>(v), r, lane);
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

template <int P>
__device__ __forceinline__ void store_sums_tail(float* __restrict__ sum_out, size_t base, size_t n, const float (&acc)[32])
{
#pragma unroll
    for (int e = 0; e < 32; ++e)
        if (base + e < n) sum_out[base + e] = acc[e] * (float)(1u << P);
}

// ------------------------------------------------------------ kernels ----

// Tile walk: each wave processes tiles first, first + stride, ...; `first`
// and `stride` are wave-uniform (scalar registers), so tile addresses and
// buffer descriptors are built with scalar arithmetic.
struct TileWalk {
    size_t first, stride;
    int lane, w;
};

template <int W = kWavesPerGroup>
__device__ __forceinline__ TileWalk tile_walk()
{
    TileWalk t;
    t.w = W == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    t.lane = lane_id();
    t.first = (size_t)blockIdx.x * W + (size_t)t.w;
    t.stride = (size_t)gridDim.x * W;
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

// Waves per workgroup of quantize and unpack: one when the packed tile is
// whole 128-byte lines (INT4 1152 B, INT3 896 B, E4M3 with FP32 scales
// 2304 B, ...), so that a freed wave slot is refilled at once; four when
// neighbouring tiles share a line (MXFP4's 1088 B), which one-wave groups
// would deal to different XCDs.  Measured against four-wave groups with
// bf16 and fp32 messages: quantize -0.3 to +1.8 points of HBM peak from
// 256 MiB on (+0.9 on average), unpack -0.3 to +2.7, both within about 1
// point at 64 MiB; MXFP4 unpack 1.2 points slower at 64 MiB.
template <int FMT, int SC, int BL> struct LineGroupWaves {
    static constexpr int v = TileGeom<FMT, SC, BL>::bytes % 128 == 0 ? 1 : kWavesPerGroup;
};

// Occupancy targets of the quantize kernel: fp32 input needs 36 KiB of LDS
// per workgroup (4 waves per SIMD fit); FP8 codes from 16-bit input run at 7
// (its exact-quotient encoder then holds its values without spilling:
// measured 3 % faster than 8 at 64 MiB); the others at RC_QUANT_WAVES.
template <int FMT, int DT> struct QuantWaves {
    static constexpr int v = DT == kF32 ? RC_QUANT_F32_WAVES : ((FMT == kFp8 || FMT == kBf8) ? 7 : RC_QUANT_WAVES);
};

// One wave quantizes one whole tile per iteration (fp32 input: the padded
// 128-byte rows pass through LDS in two halves of 32 rows, 4.5 KiB per wave;
// measured 2-3 % faster at 64 MiB than all 64 rows at once).
// With RC_QUANT_LDS the
// tile's input is read as wave-coalesced 16-byte chunks (chunk c by lane
// c % 64) and regrouped through a padded LDS row per lane; otherwise each
// lane reads its own 16-byte chunks directly.  Codes and scales go out
// through buffer stores.  Latency is covered by the other waves of the SIMD
// (no in-wave prefetch).  The partial last tile, if any, is done after the
// loop by the wave whose walk would reach it.
template <int FMT, int SC, int BL, int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QuantWaves<FMT, DT>::v)))
void quantize_kernel(const void* __restrict__ in, size_t n, uint8_t* __restrict__ out, size_t tiles)
{
    constexpr int ES = (DT == kF32) ? 4 : 2;
    constexpr int TIB = kTile * ES;            // input bytes of one tile
    constexpr int BB = 32 * ES;                // input bytes of one lane
    constexpr int CPB = BB / 16;               // 16-byte chunks per lane
    constexpr int TB = TileGeom<FMT, SC, BL>::bytes;
    constexpr int GW = LineGroupWaves<FMT, SC, BL>::v;
    const TileWalk tw = tile_walk<GW>();
    const uint32_t lane = (uint32_t)tw.lane;
    const size_t full = n / kTile;
#if RC_QUANT_LDS
    constexpr int ROW = BB + 16;               // padded LDS row: conflict-free 16-byte reads
    // fp32 (RC_QUANT_F32_HALVES): the rows of lanes 0-31, then of lanes
    // 32-63, pass through one 32-row buffer (half the LDS per wave)
    constexpr bool HALVES = RC_QUANT_F32_HALVES && DT == kF32;
    constexpr int ROWS = HALVES ? 32 : 64;
    __shared__ __attribute__((aligned(16))) uint8_t sm[GW][ROWS * ROW];
    uint8_t* lds = sm[tw.w];
#endif
    for (size_t tile = tw.first; tile < full; tile += tw.stride) {
        const Rsrc src = span_rsrc(in, tile * TIB, TIB);
        u32x4 c[CPB];
        float v[32];
#if RC_QUANT_LDS
#pragma unroll
        for (int i = 0; i < CPB; ++i) c[i] = __builtin_amdgcn_raw_buffer_load_b128(src, (64u * i + lane) * 16u, 0, kNT);
        if constexpr (HALVES) {
            // loads 0..CPB/2-1 hold the chunks of rows 0-31, the rest rows 32-63
            u32x4 r[CPB];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                wave_lds_sync();               // the buffer's previous rows are fully read
#pragma unroll
                for (int i = 0; i < CPB / 2; ++i) {
                    const uint32_t ch = 64u * i + lane;              // chunk within the half
                    *reinterpret_cast<u32x4*>(lds + (ch / CPB) * ROW + (ch % CPB) * 16) = c[h * (CPB / 2) + i];
                }
                wave_lds_sync();
                if ((lane >> 5) == (uint32_t)h) {
#pragma unroll
                    for (int i = 0; i < CPB; ++i) r[i] = *reinterpret_cast<const u32x4*>(lds + (lane & 31u) * ROW + 16 * i);
                }
            }
#pragma unroll
            for (int i = 0; i < CPB; ++i) c[i] = r[i];
        } else {
            wave_lds_sync();                   // the previous tile's rows are fully read
#pragma unroll
            for (int i = 0; i < CPB; ++i) {
                const uint32_t ch = 64u * i + lane;
                *reinterpret_cast<u32x4*>(lds + (ch / CPB) * ROW + (ch % CPB) * 16) = c[i];
            }
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < CPB; ++i) c[i] = *reinterpret_cast<const u32x4*>(lds + lane * ROW + 16 * i);
        }
#else
#pragma unroll
        for (int i = 0; i < CPB; ++i) c[i] = __builtin_amdgcn_raw_buffer_load_b128(src, lane * BB + 16u * i, 0, kNT);
#endif
        widen_chunks<DT, CPB>(c, v);
        encode_store_buf<FMT, SC, BL, 0, DT != kF32>(v, span_rsrc(out, tile * TB, TB), lane);
    }
    if (full != tiles && full % tw.stride == tw.first) {     // the partial last tile
        float v[32];
        load_block<DT>(in, full * kTile + (size_t)lane * 32, n, v);
        encode_store_buf<FMT, SC, BL, 0, DT != kF32>(v, span_rsrc(out, full * TB, TB), lane);
    }
}

// Streams whose codes are loaded together before they are accumulated.
// FP8's encoder holds more registers: it runs at fewer waves per SIMD.
// Rolling loads in the unrolled INT / MX reduce (stream j loaded once stream
// j - 2 is decoded; the same two streams in flight as batches of two, but
// each load issued earlier): 1.4-4.9 % faster at 64 MiB, neutral from
// 256 MiB.  Not for INT with E8M0 scales, whose decode holds more registers
// (there it spilled: 8-11 % slower), nor FP8 (batches of four; rolling
// four deep measured within +-1 %).
template <int FMT, int SC> struct ReduceRoll {
    static constexpr bool v = RC_REDUCE_ROLL && FMT != kFp8 && FMT != kBf8 &&
                              !((FMT == kInt3 || FMT == kInt4) && SC == kSE8);
};

template <int FMT> struct ReduceBatch {
    static constexpr int v = (FMT == kFp8 || FMT == kBf8) ? RC_FP8_REDUCE_BATCH : RC_REDUCE_BATCH;
};
// Waves per workgroup of the reduce.  INT codecs whose tiles are whole
// 128-byte lines run one-wave workgroups: a freed wave slot is refilled at
// once, which shortens the ramp and the drain of these ALU-bound kernels
// (measured at 64 MiB: INT3 4 streams -6 %, 2 streams -12 %; 1 GiB -5 %).
// So do FP8 codecs whose tiles are whole 256-byte pairs of lines (2304 B
// with FP32 scales: +0.3-3.2 points of HBM peak from 256 MiB on, within
// +-0.6 at 64 MiB; 2176-byte tiles, 17 lines, measured up to 1.3 points
// slower).  Tiles that are not whole lines (MXFP4's 1088 B, the E8M0 and
// 64-block INT variants) keep four-wave groups: one-wave groups deal
// neighbouring tiles to different XCDs, which then both fetch the line the
// two tiles share (MXFP4 measured 7-12 % slower).
template <int FMT, int SC, int BL> struct ReduceGroupWaves {
    static constexpr int TB = TileGeom<FMT, SC, BL>::bytes;
    static constexpr int v = ((FMT == kInt3 || FMT == kInt4) && TB % 128 == 0) ||
                                     ((FMT == kFp8 || FMT == kBf8) && TB % 256 == 0)
                                 ? 1 : kWavesPerGroup;
};

// Occupancy target of the reduce (amdgpu_waves_per_eu: waves per SIMD, 8 =
// at most 64 VGPRs), which also sets the register budget the compiler
// schedules for.  At 8, the INT kernels with two scales per lane or shared
// across a lane pair (16- and 64-element blocks) and with E8M0 scales spill
// registers once more than four streams are unrolled or k is a run-time
// count; they run at 6 (measured 1.2-1.5x faster at k = 8), INT with E8M0
// scales at 7 below that (their rounded decode needs more than 64
// registers).  MXFP4 from 4 streams on: with a target of 6 the compiler's
// schedule fits in 64 registers without spills (so 8 waves still run), with
// a target of 8 it spills some.  FP8 runs at RC_FP8_REDUCE_WAVES.
template <int FMT, int SC, int BL, int K> struct ReduceWaves {
    static constexpr bool kInt = FMT == kInt3 || FMT == kInt4;
    static constexpr bool kVar = BL != 32 || SC == kSE8;
    static constexpr int v = (FMT == kFp8 || FMT == kBf8) ? RC_FP8_REDUCE_WAVES
                           : (kInt && kVar && (K == 0 || K > 4)) ? 6
                           : (kInt && SC == kSE8) ? 7
                           : (FMT == kMx4 && (K == 0 || K > 3)) ? RC_MX_REDUCE_WAVES : RC_REDUCE_WAVES;
};

// acc = the K streams' decoded values of the lane's 32 elements of `tile`,
// added in stream order in binary32.  K > 0: K known at compile time, loads
// in batches; K == 0: k streams at run time, loads two at a time.
template <int FMT, int SC, int BL, int K>
__device__ __forceinline__ void reduce_tile(const StreamPtrs& ins, int k, size_t tile, uint32_t lane, float (&acc)[32])
{
    constexpr int TB = TileGeom<FMT, SC, BL>::bytes;
    constexpr int P = SumScale<FMT, SC>::v;
    if constexpr (ReduceRoll<FMT, SC>::v && K > 2) {
        // rolling: stream j is loaded as soon as stream j - 2 is decoded, so
        // two streams' codes are in flight at any time
        LaneBlock<FMT, SC, BL> c[K];
        c[0] = load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[0], tile * TB, TB), lane);
        __builtin_amdgcn_sched_barrier(0);
        c[1] = load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[1], tile * TB, TB), lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (j == 0) accumulate<FMT, SC, BL, true, P>(c[0], acc);
            else accumulate<FMT, SC, BL, false, P>(c[j], acc);
            if (j + 2 < K) {
                __builtin_amdgcn_sched_barrier(0);
                c[j + 2] = load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[j + 2], tile * TB, TB), lane);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else if constexpr (K > 0) {
        constexpr int B = (K < ReduceBatch<FMT>::v) ? K : ReduceBatch<FMT>::v;
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += B) {
            LaneBlock<FMT, SC, BL> c[B];
#pragma unroll
            for (int j = 0; j < B; ++j)
                if (k0 + j < K) c[j] = load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[k0 + j], tile * TB, TB), lane);
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (k0 + j >= K) break;
                if (k0 + j == 0) accumulate<FMT, SC, BL, true, P>(c[j], acc);
                else accumulate<FMT, SC, BL, false, P>(c[j], acc);
            }
            // keep the next batch's loads below this batch's arithmetic (bounds
            // the registers held by codes in flight)
            if (RC_REDUCE_SCHED_BARRIER && k0 + B < K) __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        accumulate<FMT, SC, BL, true, P>(load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[0], tile * TB, TB), lane), acc);
        int j = 1;
        for (; j + 1 < k; j += 2) {
            const LaneBlock<FMT, SC, BL> c0 = load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[j], tile * TB, TB), lane);
            const LaneBlock<FMT, SC, BL> c1 = load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[j + 1], tile * TB, TB), lane);
            accumulate<FMT, SC, BL, false, P>(c0, acc);
            accumulate<FMT, SC, BL, false, P>(c1, acc);
        }
        if (j < k)
            accumulate<FMT, SC, BL, false, P>(load_lane_block<FMT, SC, BL>(span_rsrc(ins.p[j], tile * TB, TB), lane), acc);
    }
}

// The FP32 sums (held at 2^-P of their value) written out at their value.
template <int P>
__device__ __forceinline__ void store_sums(float* __restrict__ sum_out, size_t tile, uint32_t lane, const float (&acc)[32])
{
    const Rsrc r = span_rsrc(sum_out, tile * (kTile * 4), kTile * 4);
    constexpr float k = (float)(1u << P);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){__float_as_uint(acc[4 * i] * k), __float_as_uint(acc[4 * i + 1] * k),
                                                       __float_as_uint(acc[4 * i + 2] * k), __float_as_uint(acc[4 * i + 3] * k)},
                                               r, lane * 128u + 16u * i, 0, kNT);
}

// Each wave reduces whole tiles: the codes of the K streams are read with
// per-lane coalesced loads, decoded and accumulated in registers, and the
// sums requantized in place.  No LDS and no in-wave prefetch: latency is
// covered by the other waves of the SIMD.  The partial last tile (if any)
// is done after the loop by the wave whose walk would reach it.
template <int FMT, int SC, int BL, int K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ReduceWaves<FMT, SC, BL, K>::v)))
void reduce_kernel(StreamPtrs ins, int k, size_t n, uint8_t* __restrict__ out, float* __restrict__ sum_out,
                   size_t tiles)
{
    constexpr int TB = TileGeom<FMT, SC, BL>::bytes;
    constexpr int P = SumScale<FMT, SC>::v;
    const TileWalk tw = tile_walk<ReduceGroupWaves<FMT, SC, BL>::v>();
    const uint32_t lane = (uint32_t)tw.lane;
    const size_t full = n / kTile;
    if (sum_out) {
        for (size_t tile = tw.first; tile < full; tile += tw.stride) {
            float acc[32];
            reduce_tile<FMT, SC, BL, K>(ins, k, tile, lane, acc);
            store_sums<P>(sum_out, tile, lane, acc);
            encode_store_buf<FMT, SC, BL, P>(acc, span_rsrc(out, tile * TB, TB), lane);
        }
    } else {
        for (size_t tile = tw.first; tile < full; tile += tw.stride) {
            float acc[32];
            reduce_tile<FMT, SC, BL, K>(ins, k, tile, lane, acc);
            encode_store_buf<FMT, SC, BL, P>(acc, span_rsrc(out, tile * TB, TB), lane);
        }
    }
    if (full != tiles && full % tw.stride == tw.first) {
        float acc[32];
        reduce_tile<FMT, SC, BL, K>(ins, k, full, lane, acc);
        const size_t base = full * kTile + (size_t)lane * 32;
        tail_zero(acc, base, n);                   // positions >= n are +0
        if (sum_out) store_sums_tail<P>(sum_out, base, n, acc);
        encode_store_buf<FMT, SC, BL, P>(acc, span_rsrc(out, full * TB, TB), lane);
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
// loads (cache policy LDA), decoded values out either through a padded LDS
// row per lane and wave-coalesced 16-byte stores (RC_UNPACK_LDS) or straight
// from each lane.
template <int FMT, int SC, int BL, int ODT, int LDA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ODT == kF32 ? 4 : 8)))
void unpack_kernel(const uint8_t* __restrict__ in, size_t n, void* __restrict__ out, size_t tiles)
{
    constexpr int TB = TileGeom<FMT, SC, BL>::bytes;
    constexpr int ES = (ODT == kF32) ? 4 : 2;
    constexpr int OB = 32 * ES;                // output bytes of one lane
    constexpr int CPB = OB / 16;
    constexpr int GW = LineGroupWaves<FMT, SC, BL>::v;
    const TileWalk tw = tile_walk<GW>();
    const uint32_t lane = (uint32_t)tw.lane;
    const size_t full = n / kTile;
#if RC_UNPACK_LDS
    constexpr int ROW = OB + 16;
    __shared__ __attribute__((aligned(16))) uint8_t sm[GW][64 * ROW];
    uint8_t* lds = sm[tw.w];
#endif
    for (size_t tile = tw.first; tile < full; tile += tw.stride) {
        float d[32];
        accumulate<FMT, SC, BL, true>(load_lane_block<FMT, SC, BL, LDA>(span_rsrc(in, tile * TB, TB), lane), d);
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
                                                   dst, ch * 16u, 0, kRowStore);
        }
#else
#pragma unroll
        for (int i = 0; i < CPB; ++i)
            __builtin_amdgcn_raw_buffer_store_b128((u32x4){wd[4 * i], wd[4 * i + 1], wd[4 * i + 2], wd[4 * i + 3]},
                                                   dst, lane * OB + 16u * i, 0, kRowStore);
#endif
    }
    if (full != tiles && full % tw.stride == tw.first) {     // the partial last tile
        float d[32];
        accumulate<FMT, SC, BL, true>(load_lane_block<FMT, SC, BL, LDA>(span_rsrc(in, full * TB, TB), lane), d);
        store_block_guarded<ODT>(out, full * kTile + (size_t)lane * 32, n, d);
    }
}

// ------------------------------------------- fused all-reduce emulation ----
//
// A quantized all-reduce of k messages that all sit in this GPU's memory,
// one per emulated rank, in one pass: for every tile each message is
// quantized and decoded in registers (what a receiver decodes), the decoded
// values are added in stream order in binary32, and then either the sum is
// requantized and decoded once more (two-shot: reduce-scatter and
// all-gather both carry compressed data) or written as is (one-shot: every
// rank reads all compressed messages).  Nothing but the inputs, the output
// and (optionally) the requantized sum touches memory.

// The lane's 32 input elements of one tile, regrouped through LDS like the
// quantize kernel's input.
template <int DT>
__device__ __forceinline__ void load_lane_row(const void* base, size_t tile, uint32_t lane, uint8_t* lds, float (&v)[32])
{
    constexpr int ES = (DT == kF32) ? 4 : 2;
    constexpr int TIB = kTile * ES;
    constexpr int BB = 32 * ES;
    constexpr int CPB = BB / 16;
    constexpr int ROW = BB + 16;
    const Rsrc src = span_rsrc(base, tile * TIB, TIB);
    u32x4 c[CPB];
#pragma unroll
    for (int i = 0; i < CPB; ++i) c[i] = __builtin_amdgcn_raw_buffer_load_b128(src, (64u * i + lane) * 16u, 0, kNT);
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
        const uint32_t ch = 64u * i + lane;
        *reinterpret_cast<u32x4*>(lds + (ch / CPB) * ROW + (ch % CPB) * 16) = c[i];
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < CPB; ++i) c[i] = *reinterpret_cast<const u32x4*>(lds + lane * ROW + 16 * i);
    wave_lds_sync();                             // rows read before the next reuse of the buffer
    widen_chunks<DT, CPB>(c, v);
}

// The lane's 32 output values of one tile, regrouped through LDS like the
// unpack kernel's output.
template <int DT>
__device__ __forceinline__ void store_lane_row(void* base, size_t tile, uint32_t lane, uint8_t* lds, const float (&d)[32])
{
    constexpr int ES = (DT == kF32) ? 4 : 2;
    constexpr int OB = 32 * ES;
    constexpr int CPB = OB / 16;
    constexpr int ROW = OB + 16;
    uint32_t wd[32];
    out_words<DT>(d, wd);
    const Rsrc dst = span_rsrc(base, tile * (size_t)(kTile * ES), kTile * ES);
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < CPB; ++i)
        *reinterpret_cast<u32x4*>(lds + lane * ROW + 16 * i) = (u32x4){wd[4 * i], wd[4 * i + 1], wd[4 * i + 2], wd[4 * i + 3]};
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
        const uint32_t ch = 64u * i + lane;
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(lds + (ch / CPB) * ROW + (ch % CPB) * 16),
                                               dst, ch * 16u, 0, kNT);
    }
    wave_lds_sync();
}

// Built for 4 waves per SIMD (up to 128 VGPRs): the message row, the FP32
// sums and the codes are live together.
template <int FMT, int SC, int BL, int DT, bool TWO_SHOT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void allreduce_kernel(StreamPtrs msgs, int k, size_t n, void* __restrict__ out, uint8_t* __restrict__ packed_out,
                      size_t tiles)
{
    constexpr int ES = (DT == kF32) ? 4 : 2;
    constexpr int ROW = 32 * ES + 16;
    constexpr int TB = TileGeom<FMT, SC, BL>::bytes;
    __shared__ __attribute__((aligned(16))) uint8_t sm[kWavesPerGroup][64 * ROW];
    const TileWalk tw = tile_walk();
    const uint32_t lane = (uint32_t)tw.lane;
    uint8_t* lds = sm[tw.w];
    const size_t full = n / kTile;
    for (size_t tile = tw.first; tile < tiles; tile += tw.stride) {
        const bool partial = tile >= full;        // wave-uniform: only the last tile
        float acc[32];
        for (int j = 0; j < k; ++j) {
            float v[32];
            if (!partial) load_lane_row<DT>(msgs.p[j], tile, lane, lds, v);
            else load_block<DT>(msgs.p[j], tile * kTile + (size_t)lane * 32, n, v);
            const LaneBlock<FMT, SC, BL> b = encode_lane<FMT, SC, BL, 0, DT != kF32>(v);
            if (j == 0) accumulate<FMT, SC, BL, true, 0, false>(b, acc);
            else accumulate<FMT, SC, BL, false, 0, false>(b, acc);
        }
        float d[32];
        if constexpr (TWO_SHOT) {
            const LaneBlock<FMT, SC, BL> r = encode_lane<FMT, SC, BL>(acc);
            if (packed_out) store_lane_block<FMT, SC, BL>(r, span_rsrc(packed_out, tile * TB, TB), lane);
            accumulate<FMT, SC, BL, true, 0, false>(r, d);
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) d[e] = acc[e];
        }
        if (!partial) store_lane_row<DT>(out, tile, lane, lds, d);
        else store_block_guarded<DT>(out, tile * kTile + (size_t)lane * 32, n, d);
    }
}

// ------------------------------------------------------------ MXFP4 GEMV ----
//
// y = W x on an MXFP4-packed row-major matrix (row r = tiles r*T .. r*T+T-1).
// The result is specified by a rounding bound, not by an order; the order
// used here: lane l of a wave holds block l of every tile of R rows (the
// same 32 columns for all R rows, so the lane's x values are loaded once and
// used R times); a block term is four interleaved fma chains of 8 elements,
// added pairwise, times 2^e (one ldexp); the lane adds its block terms over
// the tiles; then the 64 lane sums of a row are added within quads and rows
// of 16 lanes (DPP) and the four row sums read out (readlane) and added.
// Every term passes through at most 8 + 2 + T + 6 binary32 roundings.

// The lane's 32 x values of tile j (elements j*2048 + 32 lane .. + 31).
template <int XT>
__device__ __forceinline__ void load_x32(Rsrc xr, int j, uint32_t lane, float (&xv)[32])
{
    constexpr uint32_t ES = (XT == kF32) ? 4 : 2;
    const uint32_t off = ((uint32_t)j * kTile + lane * 32u) * ES;
    if constexpr (XT == kF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16u * i, 0, 0);
            xv[4 * i] = __uint_as_float(u.x); xv[4 * i + 1] = __uint_as_float(u.y);
            xv[4 * i + 2] = __uint_as_float(u.z); xv[4 * i + 3] = __uint_as_float(u.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) widen8<XT>(__builtin_amdgcn_raw_buffer_load_b128(xr, off + 16u * i, 0, 0), xv + 8 * i);
    }
}

// The lane's block of one tile: 32 E2M1 codes and the E8M0 byte.
struct GemvBlock { uint32_t d[4]; uint32_t sb; };

__device__ __forceinline__ GemvBlock gemv_load(Rsrc wt, uint32_t lane)
{
    GemvBlock b;
    const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(wt, lane * 16u, 0, kNT);
    b.d[0] = c.x; b.d[1] = c.y; b.d[2] = c.z; b.d[3] = c.w;
    b.sb = __builtin_amdgcn_raw_buffer_load_b8(wt, 1024u + lane, 0, kNT);
    return b;
}

// Block term 2^e * sum over the block's 32 elements of code * x: four
// interleaved chains (elements 8c + 2b and 8c + 2b + 1 of word c go to chains
// 2(c%2) and 2(c%2) + 1), added pairwise.
__device__ __forceinline__ float gemv_block_term(const GemvBlock& b, const float (&xv)[32])
{
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f2 v = fp4_dec(b.d[w], 1.0f, k);            // elements 8w+2k, 8w+2k+1
            p[2 * (w & 1)] = __builtin_fmaf(v.x, xv[8 * w + 2 * k], p[2 * (w & 1)]);
            p[2 * (w & 1) + 1] = __builtin_fmaf(v.y, xv[8 * w + 2 * k + 1], p[2 * (w & 1) + 1]);
        }
    }
    const float t = (p[0] + p[1]) + (p[2] + p[3]);
    return (b.sb == 255u) ? __builtin_nanf("") : __builtin_ldexpf(t, (int)b.sb - 127);
}

// bf16 x: the lane's 32 x values of tile j kept as 16 packed bf16 pairs, and
// the block term from bf16 pairs of decoded weights (E2M1 values are exact in
// bf16) with v_dot2_f32_bf16: two exact products and the running sum per
// instruction, four interleaved chains of four, added pairwise, times 2^e.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load_x32_bf16(Rsrc xr, int j, uint32_t lane, uint32_t (&xw)[16])
{
    const uint32_t off = ((uint32_t)j * kTile + lane * 32u) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16u * i, 0, 0);
        xw[4 * i] = u.x; xw[4 * i + 1] = u.y; xw[4 * i + 2] = u.z; xw[4 * i + 3] = u.w;
    }
}

__device__ __forceinline__ bf16x2 fp4_dec_bf16(uint32_t w, int sel)
{
    switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    }
}

__device__ __forceinline__ float gemv_block_term_bf16(const GemvBlock& b, const uint32_t (&xw)[16])
{
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = 2 * (w & 1) + (k & 1);
            p[c] = __builtin_amdgcn_fdot2_f32_bf16(fp4_dec_bf16(b.d[w], k), __builtin_bit_cast(bf16x2, xw[4 * w + k]),
                                                    p[c], false);
        }
    }
    const float t = (p[0] + p[1]) + (p[2] + p[3]);
    return (b.sb == 255u) ? __builtin_nanf("") : __builtin_ldexpf(t, (int)b.sb - 127);
}

// v + the value of the lane named by the DPP control (a quad permutation or
// a rotation within a row of 16 lanes), all lanes active.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The sum of v over the 64 lanes of the wave, as a wave-uniform value.
__device__ __forceinline__ float wave_sum(float v)
{
    v = dpp_add<0xB1>(v);        // quad_perm [1,0,3,2]: pairs
    v = dpp_add<0x4E>(v);        // quad_perm [2,3,0,1]: quads
    v = dpp_add<0x124>(v);       // row_ror:4  : two quads
    v = dpp_add<0x128>(v);       // row_ror:8  : the row of 16
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (a + b) + (c + d);
}

template <int YT>
__device__ __forceinline__ void store_y(void* y, size_t r, float v)
{
    if constexpr (YT == kF32) static_cast<float*>(y)[r] = v;
    else if constexpr (YT == kBF16) static_cast<uint16_t*>(y)[r] = __bfloat16_as_ushort(__float2bfloat16(v));
    else static_cast<uint16_t*>(y)[r] = (uint16_t)f16_bits(v);
}

// One wave per R consecutive rows (a group of four waves per 4R rows).  TC =
// T when T <= 2: x and all R x T weight blocks are loaded before any
// arithmetic; TC = 0: any T, tile by tile.
template <int XT, int YT, int TC, int R>
__global__ __launch_bounds__(256) void mxfp4_gemv_kernel(const uint8_t* __restrict__ w, size_t rows, int T,
                                                         const void* __restrict__ x, void* __restrict__ y)
{
    constexpr int TB = TileGeom<kMx4, kSE8, 32>::bytes;
    constexpr uint32_t ES = (XT == kF32) ? 4 : 2;
    const TileWalk tw = tile_walk();
    const uint32_t lane = (uint32_t)tw.lane;
    const Rsrc xr = span_rsrc(x, 0, (uint32_t)T * kTile * ES);
    for (size_t r0 = tw.first * R; r0 < rows; r0 += tw.stride * R) {
        float L[R];
        if constexpr (TC > 0 && XT == kBF16 && RC_GEMV_DOT2) {
            uint32_t xw[TC][16];
            GemvBlock b[R][TC];
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < TC; ++j)
                    if (r0 + i < rows) b[i][j] = gemv_load(span_rsrc(w, ((r0 + i) * TC + j) * TB, TB), lane);
#pragma unroll
            for (int j = 0; j < TC; ++j) load_x32_bf16(xr, j, lane, xw[j]);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                L[i] = 0.0f;
#pragma unroll
                for (int j = 0; j < TC; ++j) {
                    const float t = (r0 + i < rows) ? gemv_block_term_bf16(b[i][j], xw[j]) : 0.0f;
                    L[i] = (j == 0) ? t : L[i] + t;
                }
            }
        } else if constexpr (TC > 0) {
            float xv[TC][32];
            GemvBlock b[R][TC];
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < TC; ++j)
                    if (r0 + i < rows) b[i][j] = gemv_load(span_rsrc(w, ((r0 + i) * TC + j) * TB, TB), lane);
#pragma unroll
            for (int j = 0; j < TC; ++j) load_x32<XT>(xr, j, lane, xv[j]);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                L[i] = 0.0f;
#pragma unroll
                for (int j = 0; j < TC; ++j) {
                    const float t = (r0 + i < rows) ? gemv_block_term(b[i][j], xv[j]) : 0.0f;
                    L[i] = (j == 0) ? t : L[i] + t;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < R; ++i) L[i] = 0.0f;
            for (int j = 0; j < T; ++j) {
                float xv[32];
                GemvBlock b[R];
#pragma unroll
                for (int i = 0; i < R; ++i)
                    if (r0 + i < rows) b[i] = gemv_load(span_rsrc(w, ((r0 + i) * (size_t)T + j) * TB, TB), lane);
                load_x32<XT>(xr, j, lane, xv);
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float t = (r0 + i < rows) ? gemv_block_term(b[i], xv) : 0.0f;
                    L[i] = (j == 0) ? t : L[i] + t;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float s = wave_sum(L[i]);
            if (lane == 0 && r0 + i < rows) store_y<YT>(y, r0 + i, s);
        }
    }
}

// ---------------------------------------------------------- launchers ----

// Grid of `waves`-wave workgroups (four, or one where the packed tiles are
// whole 128-byte lines: LineGroupWaves, ReduceGroupWaves): one
// tile per wave up to 4 * RC_GROUPS_PER_CU waves per compute unit (1 GiB of
// bf16 input on 256 CUs; measured faster there than a 4x smaller grid
// walking 4 tiles per wave); beyond that each wave walks several tiles.
static inline dim3 tile_grid(size_t tiles, int waves = kWavesPerGroup, int groups_per_cu = RC_GROUPS_PER_CU)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const size_t groups = (tiles + waves - 1) / waves;
    const size_t cap = (size_t)groups_per_cu * (size_t)(cus > 0 ? cus : 256) * (size_t)(kWavesPerGroup / waves);
    return dim3((unsigned)(groups < cap ? groups : cap));
}

template <int FMT, int SC, int BL>
hipError_t launch_quantize_t(int dt, const void* in, size_t n, void* out, hipStream_t st)
{
    constexpr int GW = LineGroupWaves<FMT, SC, BL>::v;
    const size_t tiles = (n + kTile - 1) / kTile;
    uint8_t* o = static_cast<uint8_t*>(out);
    switch (dt) {
    case kF32: hipLaunchKernelGGL((quantize_kernel<FMT, SC, BL, kF32>), tile_grid(tiles, GW, RC_QUANT_GROUPS_PER_CU), dim3(64 * GW), 0, st, in, n, o, tiles); break;
    case kF16: hipLaunchKernelGGL((quantize_kernel<FMT, SC, BL, kF16>), tile_grid(tiles, GW, RC_QUANT_GROUPS_PER_CU), dim3(64 * GW), 0, st, in, n, o, tiles); break;
    default:   hipLaunchKernelGGL((quantize_kernel<FMT, SC, BL, kBF16>), tile_grid(tiles, GW, RC_QUANT_GROUPS_PER_CU), dim3(64 * GW), 0, st, in, n, o, tiles); break;
    }
    return hipGetLastError();
}

template <int FMT, int SC, int BL>
hipError_t launch_unpack_t(const void* in, size_t n, int dt, void* out, hipStream_t st)
{
    constexpr int GW = LineGroupWaves<FMT, SC, BL>::v;
    const size_t tiles = (n + kTile - 1) / kTile;
    const uint8_t* i = static_cast<const uint8_t*>(in);
#define RC_UNPACK(LDA)                                                                                                   \
    switch (dt) {                                                                                                        \
    case kF32: hipLaunchKernelGGL((unpack_kernel<FMT, SC, BL, kF32, LDA>), tile_grid(tiles, GW), dim3(64 * GW), 0, st, i, n, out, tiles); break; \
    case kF16: hipLaunchKernelGGL((unpack_kernel<FMT, SC, BL, kF16, LDA>), tile_grid(tiles, GW), dim3(64 * GW), 0, st, i, n, out, tiles); break; \
    default:   hipLaunchKernelGGL((unpack_kernel<FMT, SC, BL, kBF16, LDA>), tile_grid(tiles, GW), dim3(64 * GW), 0, st, i, n, out, tiles); break; \
    }
    constexpr bool F8 = FMT == kFp8 || FMT == kBf8;
    if (tiles >= kUnpackPlainLoadTiles && (!F8 || dt == kF32)) {
        RC_UNPACK(kPlainLoad)
    } else {
        RC_UNPACK(kNT)
    }
#undef RC_UNPACK
    return hipGetLastError();
}

template <int FMT, int SC, int BL, int K>
static hipError_t launch_reduce_k(const StreamPtrs& p, int k, size_t n, void* out, float* sum, hipStream_t st)
{
    const size_t tiles = (n + kTile - 1) / kTile;
    constexpr int W = ReduceGroupWaves<FMT, SC, BL>::v;
    hipLaunchKernelGGL((reduce_kernel<FMT, SC, BL, K>), tile_grid(tiles, W, RC_REDUCE_GROUPS_PER_CU), dim3(64 * W), 0, st, p, k, n,
                       static_cast<uint8_t*>(out), sum, tiles);
    return hipGetLastError();
}

// Reduce with K unrolled at compile time (K = 1..16).
template <int FMT, int SC, int BL>
hipError_t launch_reduce_unrolled_t(const StreamPtrs& p, int k, size_t n, void* out, float* sum, hipStream_t st)
{
    switch (k) {
    case 1:  return launch_reduce_k<FMT, SC, BL, 1>(p, k, n, out, sum, st);
    case 2:  return launch_reduce_k<FMT, SC, BL, 2>(p, k, n, out, sum, st);
    case 3:  return launch_reduce_k<FMT, SC, BL, 3>(p, k, n, out, sum, st);
    case 4:  return launch_reduce_k<FMT, SC, BL, 4>(p, k, n, out, sum, st);
    case 5:  return launch_reduce_k<FMT, SC, BL, 5>(p, k, n, out, sum, st);
    case 6:  return launch_reduce_k<FMT, SC, BL, 6>(p, k, n, out, sum, st);
    case 7:  return launch_reduce_k<FMT, SC, BL, 7>(p, k, n, out, sum, st);
    case 8:  return launch_reduce_k<FMT, SC, BL, 8>(p, k, n, out, sum, st);
    case 9:  return launch_reduce_k<FMT, SC, BL, 9>(p, k, n, out, sum, st);
    case 10: return launch_reduce_k<FMT, SC, BL, 10>(p, k, n, out, sum, st);
    case 11: return launch_reduce_k<FMT, SC, BL, 11>(p, k, n, out, sum, st);
    case 12: return launch_reduce_k<FMT, SC, BL, 12>(p, k, n, out, sum, st);
    case 13: return launch_reduce_k<FMT, SC, BL, 13>(p, k, n, out, sum, st);
    case 14: return launch_reduce_k<FMT, SC, BL, 14>(p, k, n, out, sum, st);
    case 15: return launch_reduce_k<FMT, SC, BL, 15>(p, k, n, out, sum, st);
    default: return launch_reduce_k<FMT, SC, BL, 16>(p, k, n, out, sum, st);
    }
}

template <int FMT, int SC, int BL>
hipError_t launch_allreduce_t(int dt, const StreamPtrs& msgs, int k, size_t n, int two_shot, void* out, void* packed,
                              hipStream_t st)
{
    const size_t tiles = (n + kTile - 1) / kTile;
    uint8_t* po = static_cast<uint8_t*>(packed);
#define RC_AR(DT, TS) hipLaunchKernelGGL((allreduce_kernel<FMT, SC, BL, DT, TS>), tile_grid(tiles), dim3(256), 0, st, \
                                         msgs, k, n, out, po, tiles)
    if (two_shot) {
        if (dt == kF32) RC_AR(kF32, true); else if (dt == kF16) RC_AR(kF16, true); else RC_AR(kBF16, true);
    } else {
        if (dt == kF32) RC_AR(kF32, false); else if (dt == kF16) RC_AR(kF16, false); else RC_AR(kBF16, false);
    }
#undef RC_AR
    return hipGetLastError();
}


template <int XT, int YT>
static hipError_t launch_gemv_xy(const void* w, size_t rows, int T, const void* x, void* y, hipStream_t st)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    constexpr int R = RC_GEMV_ROWS;
    // R rows per wave, four waves per group, at most 16 groups per CU (rows loop beyond)
    size_t groups = (rows + 4 * R - 1) / (4 * R);
    const size_t cap = (size_t)16 * (size_t)(cus > 0 ? cus : 256);
    if (groups > cap) groups = cap;
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    if (T == 1) hipLaunchKernelGGL((mxfp4_gemv_kernel<XT, YT, 1, R>), dim3((unsigned)groups), dim3(256), 0, st, wp, rows, T, x, y);
    else if (T == 2) hipLaunchKernelGGL((mxfp4_gemv_kernel<XT, YT, 2, R>), dim3((unsigned)groups), dim3(256), 0, st, wp, rows, T, x, y);
    else hipLaunchKernelGGL((mxfp4_gemv_kernel<XT, YT, 0, R>), dim3((unsigned)groups), dim3(256), 0, st, wp, rows, T, x, y);
    return hipGetLastError();
}

inline hipError_t launch_gemv_impl(const void* w, size_t rows, size_t cols, int xt, const void* x, int yt, void* y,
                                   hipStream_t st)
{
    const int T = (int)(cols / kTile);
#define RC_G(XT) (yt == kF32 ? launch_gemv_xy<XT, kF32>(w, rows, T, x, y, st) : \
                  yt == kF16 ? launch_gemv_xy<XT, kF16>(w, rows, T, x, y, st) : launch_gemv_xy<XT, kBF16>(w, rows, T, x, y, st))
    return xt == kF32 ? RC_G(kF32) : (xt == kF16 ? RC_G(kF16) : RC_G(kBF16));
#undef RC_G
}

// Reduce for the variant codecs: unrolled for 2, 4 and 8 streams (the usual
// tensor-parallel degrees; 2-9 % faster than the loop, measured), the
// stream count a run-time loop otherwise (one kernel for every other k).
template <int FMT, int SC, int BL>
hipError_t launch_reduce_rt_t(const StreamPtrs& p, int k, size_t n, void* out, float* sum, hipStream_t st)
{
#if RC_RT_UNROLL_COMMON
    switch (k) {
    case 2: return launch_reduce_k<FMT, SC, BL, 2>(p, k, n, out, sum, st);
    case 4: return launch_reduce_k<FMT, SC, BL, 4>(p, k, n, out, sum, st);
    case 8: return launch_reduce_k<FMT, SC, BL, 8>(p, k, n, out, sum, st);
    default: break;
    }
#endif
    return launch_reduce_k<FMT, SC, BL, 0>(p, k, n, out, sum, st);
}

}  // namespace rc
