// rc_device.hpp -- device-side building blocks of the gfx950 codec kernels.
//
// Work decomposition used by every kernel: one wave64 owns one 2048-element
// tile and lane l owns block l (32 consecutive elements), so the per-block
// absmax, scale and code packing all stay inside one lane's registers, and
// the per-lane code words of a tile are contiguous across lanes in every
// format (each load / store instruction of a wave covers one contiguous span).
//
// Element codes are produced and consumed with gfx950's FP4 (E2M1) and FP8
// (E4M3) conversion instructions:
//   * INT3 magnitudes 0..3 are the E2M1 codes of 0, 0.5, 1, 1.5, so a
//     sign/magnitude INT3 code is an E2M1 nibble of value q/2 with bit 2
//     clear.  Quantize = E2M1 conversion of x / (2s) (formed as below);
//     dequantize = E2M1 conversion back, times 2s.
//   * INT4 magnitudes 0..7 are the E4M3 subnormals m * 2^-9, so a sign /
//     magnitude INT4 code is an E4M3 byte with exponent 0.
// Both conversions round their binary32 input to nearest even.  The INT rule
// is round-half-even of the exact quotient |x| / s; the conversions are fed
// y = fma(x, r, x * r_lo), where r = 1/s rounded down and r_lo ~ 1/s - r
// (>= 0, so y keeps the sign of x, -0 included): y is within 2^-44 |x|/s of
// the quotient before its one
// rounding, while a quotient that is not exactly a half-integer lies more
// than half a binary32 ulp (plus that margin) away from one, so y sits on the
// same side of every half step as the quotient, and exact half steps stay
// exact (then ties go to even: below the clamp the code's low bit is the
// parity of the integer).  For a normal, unsaturated fp16 scale y <= qmax +
// 1/2, so no clamp is needed; for a subnormal or saturated scale the clamp
// is applied to the packed codes (every code above qmax becomes qmax).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace rc {

typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 2048;
constexpr int kBlock = 32;
constexpr int kWavesPerGroup = 4;          // 256-thread workgroups, one tile per wave

// ------------------------------------------------- conversion helpers ----
// The byte / word selectors of these instructions must be literals; the
// switches fold away once the callers' loops are unrolled.

// Two binary32 -> two E2M1 codes (RNE, saturating at 6, sign kept) of
// a / 2^k and b / 2^k, 2^k = the power-of-two part of `scale`; a goes to the
// low nibble of byte `sel` of `old`, b to its high nibble.
__device__ __forceinline__ uint32_t fp4_enc(uint32_t old, float a, float b, float scale, int sel)
{
    switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, 3);
    }
}

// The two E2M1 codes of byte `sel` of w (low nibble first), times the
// power-of-two part of `scale`, exactly.
__device__ __forceinline__ f2 fp4_dec(uint32_t w, float scale, int sel)
{
    switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
    }
}

// Two binary32 -> two E4M3 codes (RNE; exact for |x| <= 448, NaN above 464:
// callers clamp) into 16-bit word `hi` of `old`.
__device__ __forceinline__ uint32_t fp8_pair(float a, float b, uint32_t old, bool hi)
{
    return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
              : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}

// The two E4M3 codes of 16-bit word `hi` of w, exactly.
__device__ __forceinline__ f2 fp8_dec(uint32_t w, bool hi)
{
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// The two E4M3 codes of 16-bit word `hi` of w, times the power-of-two part
// of `scale`, exactly.
__device__ __forceinline__ f2 fp8_dec_scaled(uint32_t w, float scale, bool hi)
{
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w, scale, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w, scale, false);
}

// Two binary32 -> two E5M2 codes (RNE; exact for |x| <= 57344, infinity from
// 61440 up: callers clamp) into 16-bit word `hi` of `old`.
__device__ __forceinline__ uint32_t bf8_pair(float a, float b, uint32_t old, bool hi)
{
    return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, true)
              : (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, false);
}

// The two E5M2 codes of 16-bit word `hi` of w, exactly.
__device__ __forceinline__ f2 bf8_dec(uint32_t w, bool hi)
{
    return hi ? __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
}

// ---------------------------------------------------------------- loads ----

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xFFFFu))); }
__device__ __forceinline__ float f16hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }

// dtype codes as in the C ABI
enum : int { kF32 = 1, kF16 = 2, kBF16 = 3 };

template <int DT>
__device__ __forceinline__ void widen8(const u32x4 u, float* v)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (DT == kBF16) { v[2 * i] = bf16lo(w[i]); v[2 * i + 1] = bf16hi(w[i]); }
        else             { v[2 * i] = f16lo(w[i]);  v[2 * i + 1] = f16hi(w[i]); }
    }
}

// Load the 32 elements of one block, widened exactly to binary32.  `base` is
// the element index of the block; elements >= n read as +0.
template <int DT>
__device__ __forceinline__ void load_block(const void* __restrict__ in, size_t base, size_t n, float (&v)[32])
{
    if (base + 32 <= n) {
        if (DT == kF32) {
            const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(in) + base);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 u = __builtin_nontemporal_load(p + i);
                v[4 * i] = __uint_as_float(u.x); v[4 * i + 1] = __uint_as_float(u.y);
                v[4 * i + 2] = __uint_as_float(u.z); v[4 * i + 3] = __uint_as_float(u.w);
            }
        } else {
            const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(in) + base);
#pragma unroll
            for (int i = 0; i < 4; ++i) widen8<DT>(__builtin_nontemporal_load(p + i), v + 8 * i);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            size_t i = base + e;
            float x = 0.0f;
            if (i < n) {
                if (DT == kF32) x = static_cast<const float*>(in)[i];
                else {
                    uint32_t h = static_cast<const uint16_t*>(in)[i];
                    x = (DT == kBF16) ? bf16lo(h) : f16lo(h);
                }
            }
            v[e] = x;
        }
    }
}

// max |v[e]| over e in [B, E)
template <int B, int E>
__device__ __forceinline__ float absmax_range(const float (&v)[32])
{
    float a = 0.0f;
#pragma unroll
    for (int e = B; e < E; e += 2) a = fmaxf(fmaxf(fabsf(v[e]), fabsf(v[e + 1])), a);
    return a;
}

__device__ __forceinline__ float absmax32(const float (&v)[32]) { return absmax_range<0, 32>(v); }

// The value held by the other lane of this lane's pair (lanes 2m, 2m+1):
// a DPP quad permutation [1,0,3,2].
__device__ __forceinline__ float pair_swap(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// ------------------------------------------------------- INT scale rule ----

struct IntScale {
    float s;          // fp16 scale as binary32 (exact)
    uint32_t bits;    // fp16 bit pattern
    float r;          // 1/s rounded down, 0 for a zero block
    float r_lo;       // RN((1 - s r) r) ~ 1/s - r >= 0, 0 for a zero block
    bool zero;        // s == 0: the block is stored as zeros
    bool abnormal;    // subnormal fp16 or saturated: codes need the clamp
};

// Correctly rounded a / b for a constant b: q = a * RN(1/b), then one
// residual correction.  For b = 3, 7, 448 and 57344 this equals the IEEE
// quotient for every finite a >= 0 (448, 57344: wherever the quotient is
// normal), which an exhaustive run over all binary32 inputs confirms; an
// infinite a gives NaN.
template <int B>
__device__ __forceinline__ float div_by(float a)
{
    constexpr float y = 1.0f / (float)B;
    const float q = a * y;
    return __builtin_fmaf(__builtin_fmaf(-q, (float)B, a), y, q);
}

// RN(1/s) for a positive fp16 scale s (as binary32): the hardware
// reciprocal (within 1 ulp) plus one Newton step, which is correctly rounded
// for every fp16 value and every starting point within 1 ulp.
__device__ __forceinline__ float recip_f16_scale(float s)
{
    const float y0 = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
}

// s = fp16(min(fp32(a / qmax), 65504)) with the IEEE binary32 quotient.
template <int QMAX>
__device__ __forceinline__ IntScale int_scale(float a)
{
    IntScale r;
    float s32 = div_by<QMAX>(a);
    const bool sat = !(s32 <= 65504.0f);            // also an infinite a (NaN quotient)
    s32 = fminf(s32, 65504.0f);
    __half h = __float2half_rn(s32);
    r.bits = __half_as_ushort(h);
    r.s = __half2float(h);
    r.zero = (r.s == 0.0f);
    r.abnormal = sat || (!r.zero && r.s < 0x1p-14f);
    r.r = r.zero ? 0.0f : recip_f16_scale(r.s);
    // The high part is taken rounded down, r <= 1/s, so that the low part is
    // never negative: then x r_lo keeps the sign of x even for x = -0 (a
    // negative r_lo would turn -0 * r_lo into +0 and lose the sign of a -0
    // element).  1 - s r is exact (at most 10 significant bits, |.| < 2^-22);
    // times r it gives the low part of 1/s to within 2^-45 / s in all.
    float e = __builtin_fmaf(-r.s, r.r, 1.0f);
    r.r = __uint_as_float(__float_as_uint(r.r) - (e < 0.0f ? 1u : 0u));
    e = __builtin_fmaf(-r.s, r.r, 1.0f);
    r.r_lo = e * r.r;
    return r;
}

__device__ __forceinline__ uint32_t signbit_u(float x) { return __float_as_uint(x) >> 31; }

// floor(log2 a) of a positive binary32, subnormals included (128 for inf).
__device__ __forceinline__ int ilog2f(float a)
{
    const uint32_t b = __float_as_uint(a);
    const int ef = (int)(b >> 23);
    return ef ? ef - 127 : (31 - (int)__builtin_clz(b)) - 149;
}

// ============================================================ codecs ====
//
// A codec is (element format, scale type, block size).  Each lane holds 32
// consecutive elements of a tile; with 32-element blocks that is one block,
// with 16-element blocks two (elements 0-15 and 16-31, "halves"), and with
// 64-element blocks lanes 2m and 2m+1 share one block (absmax exchanged
// across the pair, the even lane stores the scale).

enum : int { kS16 = 1, kS32 = 2, kSE8 = 3 };   // scale types (rc_scale_type)

template <int FMT> struct Fmt;
template <> struct Fmt<1> { static constexpr int code_bytes = 1024, emax = 2, qmax = 7; };       // INT4
template <> struct Fmt<2> { static constexpr int code_bytes = 768, emax = 1, qmax = 3; };        // INT3
template <> struct Fmt<3> { static constexpr int code_bytes = 2048, emax = 8, fmax = 448; };     // E4M3
template <> struct Fmt<4> { static constexpr int code_bytes = 1024, emax = 2; };                // E2M1
template <> struct Fmt<5> { static constexpr int code_bytes = 2048, emax = 15, fmax = 57344; }; // E5M2

template <int SC> struct ScaleBytes { static constexpr int v = SC == kS16 ? 2 : (SC == kS32 ? 4 : 1); };
template <int BL> struct Halves { static constexpr int v = (BL == 16) ? 2 : 1; };  // scale blocks per lane

template <int FMT, int SC, int BL> struct TileGeom {
    static constexpr int code = Fmt<FMT>::code_bytes;
    static constexpr int bytes = code + (2048 / BL) * ScaleBytes<SC>::v;
};

// MX shared exponent: floor(log2 a) minus the element format's largest
// exponent, clamped to the E8M0 range; -127 for a zero block.
template <int EMAX>
__device__ __forceinline__ int e8m0_exponent(float a)
{
    int e = (a == 0.0f) ? -127 : ilog2f(a) - EMAX;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Per-block encode data: the stored scale bits and the element multiplier
// (INT/FP16: 1/s rounded down, with m_lo >= 0 its low part; E8M0: 2^-e; FP8 with
// FP32/FP16 scale: s itself; E2M1: 2^e, the conversion's scale operand).
struct EncScale {
    uint32_t bits;
    float m;
    float m_lo;      // INT/FP16: low part of the reciprocal; FP8/FP32: a - s fmax
                     // (exact: its sign says which way s was rounded)
    bool zero;       // FP16/FP32 scale 0: the block is stored as zeros
    bool clamp;      // codes may exceed the format's largest magnitude
};

template <int FMT, int SC>
__device__ __forceinline__ EncScale enc_scale(float a)
{
    EncScale r;
    r.zero = false;
    r.clamp = false;
    r.m_lo = 0.0f;
    if constexpr (FMT == 1 || FMT == 2) {
        if constexpr (SC == kS16) {
            const IntScale sc = int_scale<Fmt<FMT>::qmax>(a);
            r.bits = sc.bits;                            // +0 for a zero block (a >= 0)
            r.m = sc.r;
            r.m_lo = sc.r_lo;
            r.zero = sc.zero;
            r.clamp = sc.abnormal;
        } else {
            const int e = e8m0_exponent<Fmt<FMT>::emax>(a);
            r.bits = (uint32_t)(e + 127);
            r.m = __builtin_ldexpf(1.0f, -e);
            r.clamp = true;                              // a / 2^e lies in [2^k, 2^(k+1))
        }
    } else if constexpr (FMT == 3 || FMT == 5) {
        if constexpr (SC == kS32) {
            const float s = (a == __builtin_inff()) ? a : div_by<Fmt<FMT>::fmax>(a);   // inf / fmax = inf
            r.zero = !(s >= 0x1p-126f);
            r.bits = r.zero ? 0u : __float_as_uint(s);
            r.m = s;
            r.m_lo = __builtin_fmaf(-s, (float)Fmt<FMT>::fmax, a);
        } else if constexpr (SC == kS16) {
            const float s32 = fminf(div_by<Fmt<FMT>::fmax>(a), 65504.0f);            // NaN (inf a) -> 65504
            const __half h = __float2half_rn(s32);
            const float s = __half2float(h);
            r.zero = (s == 0.0f);
            r.bits = r.zero ? 0u : (uint32_t)__half_as_ushort(h);
            r.m = s;
        } else {
            const int e = e8m0_exponent<Fmt<FMT>::emax>(a);
            r.bits = (uint32_t)(e + 127);
            r.m = __builtin_ldexpf(1.0f, -e);
        }
    } else {
        const int e = e8m0_exponent<2>(a);
        r.bits = (uint32_t)(e + 127);
        r.m = __builtin_ldexpf(1.0f, e);                 // 2^e, subnormal for e < -126
    }
    return r;
}

// The lane's block maxima: two halves, one block, or the pair's block.
template <int BL>
__device__ __forceinline__ void lane_absmax(const float (&v)[32], float (&a)[Halves<BL>::v])
{
    if constexpr (BL == 16) {
        a[0] = absmax_range<0, 16>(v);
        a[1] = absmax_range<16, 32>(v);
    } else {
        float m = absmax32(v);
        if constexpr (BL == 64) m = fmaxf(m, pair_swap(m));
        a[0] = m;
    }
}

// All-ones unless the block (or half h of a 16-element-block lane) is a
// zero-scale block; `lo`/`hi` select which 16 of the word's bits belong to
// the first half for word layouts that mix halves (INT3 group words).
template <int H>
__device__ __forceinline__ uint32_t keep_mask(const EncScale (&sc)[H], int half)
{
    return sc[H == 2 ? half : 0].zero ? 0u : 0xFFFFFFFFu;
}

// ----------------------------------------------------------------- INT3 ----
// Group word g (g = 0..3) of a lane's 32 elements holds in nibble j the code
// of element 4j + g: (sign << 3) | magnitude.  Plane words:
//   q2w word 0 = (N0 & 0x33333333) | ((N1 & 0x33333333) << 2)
//   q2w word 1 = (N2 & 0x33333333) | ((N3 & 0x33333333) << 2)
//   q1w word   = sign of element e at bit e.
// Nibbles 0-3 of a group word are elements 0..15, nibbles 4-7 elements
// 16..31; byte b holds nibbles 2b, 2b+1 (elements 8b+g, 8b+4+g).

struct Int3Words { uint32_t w0, w1, h; };

__device__ __forceinline__ Int3Words int3_planes(const uint32_t (&N)[4])
{
    Int3Words o;
    o.w0 = (N[0] & 0x33333333u) | ((N[1] << 2) & 0xCCCCCCCCu);
    o.w1 = (N[2] & 0x33333333u) | ((N[3] << 2) & 0xCCCCCCCCu);
    o.h = (N[3] & 0x88888888u) | ((N[2] >> 1) & 0x44444444u) | ((N[1] >> 2) & 0x22222222u) |
          ((N[0] >> 3) & 0x11111111u);
    return o;
}

__device__ __forceinline__ uint32_t int3_group(uint32_t w0, uint32_t w1, uint32_t h, int g)
{
    uint32_t w = (g < 2) ? w0 : w1;
    return ((w >> (2 * (g & 1))) & 0x33333333u) | ((h << (3 - g)) & 0x88888888u);
}

// min(magnitude, 3) on E2M1 nibbles: a magnitude code with bit 2 set (an E2M1
// value of 2 or more, i.e. an INT3 magnitude of 4 or more) becomes 3.
__device__ __forceinline__ uint32_t int3_clamp_word(uint32_t w)
{
    const uint32_t big = (w >> 2) & 0x11111111u;
    return (w & 0x88888888u) | (w & 0x33333333u) | (big * 3u);
}

// INT3 codes: E2M1 nibbles of x / (2 s), formed as fma(x, r/2, x r_lo/2)
// (FP16 scale) or x 2^-e / 2 (E8M0): RNE, the low code bit is the integer's
// parity below 2; clamped when a block may exceed 3.
// E8M0 scales (P2): the multiplier 2^-e is a power of two, so the
// conversion's own scale operand 2^(e+1) divides exactly and no multiply is
// needed (e <= 126 for finite data, so the operand is finite).
// With P = 1 the values come in halved (sums held at 2^-1 of their value),
// so x / (2 s) is formed with r and r_lo themselves.
template <int H, bool P2, int P = 0>
__device__ __forceinline__ Int3Words int3_encode(const float (&v)[32], const EncScale (&sc)[H])
{
    static_assert(P == 0 || (P == 1 && !P2), "pre-scaled values only with FP16 scales");
    constexpr float k = P == 1 ? 1.0f : 0.5f;
    float r2[H], l2[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        r2[h] = P2 ? __builtin_ldexpf(2.0f, (int)sc[h].bits - 127)   // 2^(e+1), the operand
                   : k * sc[h].m;                                     // r/2 (or r), exact
        l2[h] = k * sc[h].m_lo;                                       // r_lo/2 (or r_lo), exact
    }
    uint32_t N[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t w = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float r = r2[H == 2 ? b / 2 : 0], l = l2[H == 2 ? b / 2 : 0];
            const float y0 = v[8 * b + g], y1 = v[8 * b + 4 + g];
            const float x0 = P2 ? y0 : __builtin_fmaf(y0, r, y0 * l);
            const float x1 = P2 ? y1 : __builtin_fmaf(y1, r, y1 * l);
            // the first conversion starts from x0's own bits: every byte of w
            // is written by the four conversions, and no register is cleared
            w = fp4_enc(b == 0 ? __float_as_uint(x0) : w, x0, x1, P2 ? r : 1.0f, b);
        }
        N[g] = w;
    }
    bool clamp = sc[0].clamp;
    if constexpr (H == 2) clamp = clamp || sc[1].clamp;
    if (clamp) {
#pragma unroll
        for (int g = 0; g < 4; ++g) N[g] = int3_clamp_word(N[g]);
    }
    // A zero block (FP16 scale 0) has multiplier 0, so its magnitudes are
    // already 0; only the signs of its negative elements (x * 0 = -0) remain,
    // and they all sit in the sign plane: elements 0-15 in bits 0-15.
    uint32_t keep = sc[0].zero ? 0u : 0xFFFFFFFFu;
    if constexpr (H == 2) keep = (sc[0].zero ? 0u : 0x0000FFFFu) | (sc[1].zero ? 0u : 0xFFFF0000u);
    Int3Words o = int3_planes(N);
    o.h &= keep;
    return o;
}

// acc[e] (+)= q_e * S for the 32 elements: E2M1 decode of the nibble (q/2)
// times dm = 2S (exact products, one rounding per add); with sums held at
// half their value, dm = S.  The first term is an fma with a -0 addend,
// which is the product itself, signed zeros included.
// ROUNDED (E8M0 exponents whose products can exceed binary32): the nibbles
// decode as q (conversion scale 2), dm = 2^e, and each product is rounded
// before it is added.
template <bool FIRST, int H, bool ROUNDED = false>
__device__ __forceinline__ void int3_accumulate(uint32_t w0, uint32_t w1, uint32_t h, const float (&dm)[H],
                                                float (&acc)[32])
{
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t Ng = int3_group(w0, w1, h, g);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float m = dm[H == 2 ? b / 2 : 0];
            const f2 c = fp4_dec(Ng, ROUNDED ? 2.0f : 1.0f, b);
            if constexpr (ROUNDED) {
                const float vx = __fmul_rn(c.x, m), vy = __fmul_rn(c.y, m);
                acc[8 * b + g] = FIRST ? vx : __fadd_rn(acc[8 * b + g], vx);
                acc[8 * b + 4 + g] = FIRST ? vy : __fadd_rn(acc[8 * b + 4 + g], vy);
            } else if (FIRST) {
                acc[8 * b + g] = __builtin_fmaf(c.x, m, -0.0f);
                acc[8 * b + 4 + g] = __builtin_fmaf(c.y, m, -0.0f);
            }
            else {
                acc[8 * b + g] = __builtin_fmaf(c.x, m, acc[8 * b + g]);
                acc[8 * b + 4 + g] = __builtin_fmaf(c.y, m, acc[8 * b + 4 + g]);
            }
        }
    }
}

// ----------------------------------------------------------------- INT4 ----
// Word d (d = 0..3) holds elements 8d..8d+7, element 8d+j in nibble j:
// (sign << 3) | magnitude.  E4M3 view: byte = (sign << 7) | m.

// min(magnitude, 7) on four E4M3 bytes of INT4 codes: a byte with a nonzero
// exponent field (value 8 * 2^-9 or more) gets mantissa bits 111; only the
// mantissa and sign bits are packed afterwards.
__device__ __forceinline__ uint32_t int4_clamp_bytes(uint32_t x)
{
    const uint32_t big = (((x & 0x78787878u) + 0x78787878u) >> 7) & 0x01010101u;
    return x | big | (big << 1) | (big << 2);
}

// INT4 codes: E4M3 subnormal bytes of x / s * 2^-9 (RNE), formed as
// fma(x, r 2^-9, x r_lo 2^-9) (FP16 scale) or x 2^-e 2^-9 (E8M0, m_lo = 0),
// clamped when a block may exceed 7.
// With P = 9 the values come in at 2^-9 of their value (pre-scaled sums), so
// the multipliers are r and r_lo themselves.
template <int H, int P = 0>
__device__ __forceinline__ void int4_encode(const float (&v)[32], const EncScale (&sc)[H], uint32_t (&D)[4])
{
    static_assert(P == 0 || P == 9, "INT4 values are pre-scaled by 2^-9 or not at all");
    constexpr float k = P == 9 ? 1.0f : 0x1p-9f;
    float r9[H], l9[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        r9[h] = sc[h].m * k;                                             // exact
        l9[h] = sc[h].m_lo * k;                                          // exact (>= 2^-50 or 0)
    }
    // word d's even elements 0,2,4,6 in the bytes of xe[d], odd 1,3,5,7 in xo[d]
    uint32_t xe[4], xo[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float r = r9[H == 2 ? d / 2 : 0], l = l9[H == 2 ? d / 2 : 0];
        const float* y = v + 8 * d;
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = __builtin_fmaf(y[j], r, y[j] * l);
        // first conversions start from their own bits
        xe[d] = fp8_pair(q[4], q[6], fp8_pair(q[0], q[2], __float_as_uint(q[0]), false), true);
        xo[d] = fp8_pair(q[5], q[7], fp8_pair(q[1], q[3], __float_as_uint(q[1]), false), true);
    }
    bool clamp = sc[0].clamp;
    if constexpr (H == 2) clamp = clamp || sc[1].clamp;
    if (clamp) {
#pragma unroll
        for (int d = 0; d < 4; ++d) { xe[d] = int4_clamp_bytes(xe[d]); xo[d] = int4_clamp_bytes(xo[d]); }
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
        D[d] = ((xe[d] & 0x07070707u) | ((xe[d] >> 4) & 0x08080808u) | ((xo[d] << 4) & 0x70707070u) |
                (xo[d] & 0x80808080u)) & keep_mask(sc, d / 2);
}

// acc[e] (+)= q_e * S: the nibbles rebuilt as E4M3 subnormal bytes, decoded
// times the power-of-two part of `cs` (1 for an FP16 scale, giving q 2^-9,
// with dm = 512 s; 512 for E8M0, giving q, with dm = 2^e).  ROUNDED (E8M0
// exponents whose products can exceed binary32): each product is rounded
// before it is added.
template <bool FIRST, int H, bool ROUNDED = false>
__device__ __forceinline__ void int4_accumulate(const uint32_t (&D)[4], float cs, const float (&dm)[H],
                                                float (&acc)[32])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float m = dm[H == 2 ? d / 2 : 0];
        const uint32_t xe = (D[d] & 0x07070707u) | ((D[d] << 4) & 0x80808080u);
        const uint32_t xo = ((D[d] >> 4) & 0x07070707u) | (D[d] & 0x80808080u);
        f2 e01, e23, o01, o23;
        if (cs == 1.0f) {
            e01 = fp8_dec(xe, false); e23 = fp8_dec(xe, true);
            o01 = fp8_dec(xo, false); o23 = fp8_dec(xo, true);
        } else {
            e01 = fp8_dec_scaled(xe, cs, false); e23 = fp8_dec_scaled(xe, cs, true);
            o01 = fp8_dec_scaled(xo, cs, false); o23 = fp8_dec_scaled(xo, cs, true);
        }
        const float c[8] = {e01.x, o01.x, e01.y, o01.y, e23.x, o23.x, e23.y, o23.y};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (ROUNDED) {
                const float v = __fmul_rn(c[j], m);
                acc[8 * d + j] = FIRST ? v : __fadd_rn(acc[8 * d + j], v);
            } else if (FIRST) {
                acc[8 * d + j] = __builtin_fmaf(c[j], m, -0.0f);   // the product, signed zeros kept
            } else {
                acc[8 * d + j] = __builtin_fmaf(c[j], m, acc[8 * d + j]);
            }
        }
    }
}

// ------------------------------------------------------------------ FP8 ----
// Byte e of the lane's 32 code bytes = E4M3 or E5M2 code of element e;
// word d holds elements 4d..4d+3.

template <int FMT>
__device__ __forceinline__ uint32_t f8_pair(float a, float b, uint32_t old, bool hi)
{
    if constexpr (FMT == 5) return bf8_pair(a, b, old, hi);
    else return fp8_pair(a, b, old, hi);
}

template <int FMT>
__device__ __forceinline__ f2 f8_dec(uint32_t w, bool hi)
{
    if constexpr (FMT == 5) return bf8_dec(w, hi);
    else return fp8_dec(w, hi);
}

// Round-to-odd binary32 value of the exact quotient |x| / s, with the sign
// of x and clamped to FMAX; its round-to-nearest-even conversion to E4M3 or
// E5M2 equals that of the exact quotient (binary32 carries more than 4 + 2
// significant bits).  rs is the hardware reciprocal of s (within 1 ulp) and
// rl = fma(-s, rs, 1) * rs its low part, so that
//   y1 = fma(|x|, rs, |x| * rl) lies within 1 ulp of the quotient q, and
//   r = fma(-y1, s, |x|) is exact, zero only when y1 = q, negative when q
//   lies below y1: its sign bit steps y1 down to the binary32 value just
//   below q, and a nonzero r sets the last bit (round to odd).
// An overflowed y1 = inf gives r = -inf and so the largest finite value.
// The residuals must not underflow: callers pass s >= 2^-64 (smaller block
// scales are handled by multiplying x and s by 2^64).
template <int FMAX, bool CLAMP>
__device__ __forceinline__ float fp8_ro_quotient(float x, float s, float rs, float rl)
{
    const float ax = fabsf(x);
    const float y1 = __builtin_fmaf(ax, rs, ax * rl);
    const uint32_t rb = __float_as_uint(__builtin_fmaf(-y1, s, ax));
    const uint32_t t = (__float_as_uint(y1) - (rb >> 31)) | min(rb, 1u);
    const float yo = CLAMP ? fminf(__uint_as_float(t), (float)FMAX) : __uint_as_float(t);
    return __uint_as_float(__float_as_uint(yo) | (__float_as_uint(x) & 0x80000000u));
}

// Codes of the exact quotients x / s (scales as multipliers m = s), with x
// and s both multiplied by k (an exact power of two).  CLAMP = false when
// every quotient is known to round to at most the format's largest value
// (see fp8_encode).
template <int FMT, int H, bool CLAMP>
__device__ __forceinline__ void fp8_quotient_codes(const float (&v)[32], const float (&sk)[H], float k,
                                                   uint32_t (&d)[8])
{
    float rs[H], rl[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        rs[h] = __builtin_amdgcn_rcpf(sk[h]);
        rl[h] = __builtin_fmaf(-sk[h], rs[h], 1.0f) * rs[h];
    }
    constexpr int FM = Fmt<FMT>::fmax;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int h = H == 2 ? i / 4 : 0;
        const float* x = v + 4 * i;
        const float q0 = fp8_ro_quotient<FM, CLAMP>(x[0] * k, sk[h], rs[h], rl[h]);
        const uint32_t w = f8_pair<FMT>(q0, fp8_ro_quotient<FM, CLAMP>(x[1] * k, sk[h], rs[h], rl[h]),
                                        __float_as_uint(q0), false);     // starts from q0's own bits
        d[i] = f8_pair<FMT>(fp8_ro_quotient<FM, CLAMP>(x[2] * k, sk[h], rs[h], rl[h]),
                            fp8_ro_quotient<FM, CLAMP>(x[3] * k, sk[h], rs[h], rl[h]), w, true);
    }
}

// Codes of x * r (r = the reciprocal rounded down by 2^-21) and of x * R
// (rounded up by 2^-21), clamped to the largest magnitude when CLAMP.
// Against the hardware reciprocal's 1 ulp and the roundings of r and of the
// products, the two products enclose the quotient x / s; the conversion
// (nearest even, after the clamp) is monotone, so where both give one code
// that is the code of the quotient.  Where they differ (adjacent codes) the
// quotient lies within 2^-20 of the midpoint m between them:
//   - NARROW (x and the block maximum a carry at most 11 significant bits,
//     as bf16 and fp16 values do): then the quotient is an exact tie of
//     fmax x = m a (FP32 scale; s = a / fmax rounded, so the quotient lies
//     above m when s was rounded down, dir = a - s fmax > 0, below when up,
//     on it when exact) or of x = m s (FP16 scale, dir = 0), because any
//     other distance from a midpoint is at least 2^-16 relative.  The code
//     is taken per byte: the upper one, the lower one, or the even one.
//   - otherwise, where some lane of the wave has such an element in a word
//     of four codes, the exact sequence recomputes that word (fp32 sums and
//     messages seldom need it; sums of two streams, often a single decoded
//     term, do for about one word in eight).
// Callers pass s >= 2^-64 in every lane.
template <int FMT, int H, bool CLAMP, bool NARROW>
__device__ __forceinline__ void fp8_bracket_codes(const float (&v)[32], const float (&s)[H], const float (&dir)[H],
                                                  uint32_t (&d)[8])
{
    constexpr float FM = (float)Fmt<FMT>::fmax;
    constexpr int FMI = Fmt<FMT>::fmax;
    float rs[H], rl[H], rlo[H], rhi[H];
    uint32_t up[H], tie[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        rs[h] = __builtin_amdgcn_rcpf(s[h]);
        rl[h] = __builtin_fmaf(-s[h], rs[h], 1.0f) * rs[h];
        rlo[h] = rs[h] * 0x1.fffffp-1f;         // 1 - 2^-21
        rhi[h] = rs[h] * 0x1.000008p0f;         // 1 + 2^-21
        up[h] = dir[h] > 0.0f ? 0x01010101u : 0u;
        tie[h] = dir[h] == 0.0f ? 0x01010101u : 0u;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int h = H == 2 ? i / 4 : 0;
        float a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = v[4 * i + j] * rlo[h];
            b[j] = v[4 * i + j] * rhi[h];
            if constexpr (CLAMP) {
                a[j] = __builtin_amdgcn_fmed3f(a[j], -FM, FM);
                b[j] = __builtin_amdgcn_fmed3f(b[j], -FM, FM);
            }
        }
        uint32_t lo = f8_pair<FMT>(a[2], a[3], f8_pair<FMT>(a[0], a[1], __float_as_uint(a[0]), false), true);
        const uint32_t hi = f8_pair<FMT>(b[2], b[3], f8_pair<FMT>(b[0], b[1], __float_as_uint(b[0]), false), true);
        if constexpr (NARROW) {
            // byte k from hi where the lower code is odd (ties) or dir > 0:
            // selector k + 4 picks hi's byte k, k picks lo's
            d[i] = __builtin_amdgcn_perm(hi, lo, (((lo & tie[h]) | up[h]) << 2) | 0x03020100u);
        } else {
            if (__builtin_amdgcn_ballot_w64(lo != hi) != 0u) {         // wave-uniform
                const float* x = v + 4 * i;
                const float q0 = fp8_ro_quotient<FMI, CLAMP>(x[0], s[h], rs[h], rl[h]);
                lo = f8_pair<FMT>(q0, fp8_ro_quotient<FMI, CLAMP>(x[1], s[h], rs[h], rl[h]), __float_as_uint(q0), false);
                lo = f8_pair<FMT>(fp8_ro_quotient<FMI, CLAMP>(x[2], s[h], rs[h], rl[h]),
                                  fp8_ro_quotient<FMI, CLAMP>(x[3], s[h], rs[h], rl[h]), lo, true);
            }
            d[i] = lo;
        }
    }
}

// FP8 codes (E4M3 / E5M2): with an FP32 or FP16 scale the code of the exact
// quotient, from the bracket above or, in a wave where some lane's scale is
// below 2^-64, from the round-to-odd sequence for every code; with an E8M0
// scale x * 2^-e is exact, clamped to the format's largest magnitude and
// converted (RNE).
template <int FMT, int SC, int H, bool NARROW>
__device__ __forceinline__ void fp8_encode(const float (&v)[32], const EncScale (&sc)[H], uint32_t (&d)[8])
{
    constexpr float FM = (float)Fmt<FMT>::fmax;
    if constexpr (SC == kSE8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float m = sc[H == 2 ? i / 4 : 0].m;
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(v[4 * i + j] * m, -FM), FM);
            d[i] = f8_pair<FMT>(y[2], y[3], f8_pair<FMT>(y[0], y[1], __float_as_uint(y[0]), false), true);
        }
    } else {
        float s[H], dir[H];
        bool tiny = false;
#pragma unroll
        for (int h = 0; h < H; ++h) {
            s[h] = sc[h].zero ? 1.0f : sc[h].m;
            dir[h] = sc[h].m_lo;
            if constexpr (SC == kS32) tiny = tiny || (s[h] < 0x1p-64f);
        }
        // FP32 scale: s = RN32(absmax / fmax) is normal or the block is zero,
        // so |x| / s <= fmax / (1 - 2^-24), which rounds to fmax in both
        // formats (the next code point up lies far beyond); the round-to-odd
        // value stays below the first value that would overflow.  FP16
        // scales (subnormal or clamped at 65504) need the clamp.
        constexpr bool CL = SC != kS32;
        if (__builtin_amdgcn_ballot_w64(tiny) == 0u) {                  // wave-uniform
            fp8_bracket_codes<FMT, H, CL, NARROW>(v, s, dir, d);
        } else {                              // some scale below 2^-64: the exact sequence
            if (!tiny) {
                fp8_quotient_codes<FMT, H, CL>(v, s, 1.0f, d);
            } else {                          // tiny scale: x * 2^64 and s * 2^64 are exact
                float sk[H];
#pragma unroll
                for (int h = 0; h < H; ++h) sk[h] = s[h] * 0x1p64f;
                fp8_quotient_codes<FMT, H, CL>(v, sk, 0x1p64f, d);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] &= keep_mask(sc, i / 4);
    }
}

// acc[e] (+)= code_e * S.  FP32 scale: RN32(code * s) then RN32(acc + d);
// FP16 and E8M0 scales: code * S is exact, so one fma is the same -- unless
// it exceeds binary32 (E8M0 exponents the encoder never writes): ROUNDED
// then rounds each product as with FP32 scales.
template <int FMT, int SC, bool FIRST, int H, bool ROUNDED = false>
__device__ __forceinline__ void fp8_accumulate(const uint32_t (&D)[8], const float (&dm)[H], float (&acc)[32])
{
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        const float m = dm[H == 2 ? d / 4 : 0];
        const f2 lo = f8_dec<FMT>(D[d], false), hi = f8_dec<FMT>(D[d], true);
        const float c[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (SC == kS32 || ROUNDED) {
                const float dv = __fmul_rn(c[j], m);                 // RN32(code * s)
                if (FIRST) acc[4 * d + j] = dv;
                else acc[4 * d + j] = __fadd_rn(acc[4 * d + j], dv);  // RN32(acc + d)
            } else {
                if (FIRST) acc[4 * d + j] = c[j] * m;
                else acc[4 * d + j] = __builtin_fmaf(c[j], m, acc[4 * d + j]);
            }
        }
    }
}

// ---------------------------------------------------------------- MXFP4 ----
// Word d holds elements 8d..8d+7 (element 8d+j in nibble j), E2M1 codes.

template <int H>
__device__ __forceinline__ void mx_encode(const float (&v)[32], const EncScale (&sc)[H], uint32_t (&D)[4])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float p = sc[H == 2 ? d / 2 : 0].m;         // 2^e as the conversion's scale operand
        uint32_t w = __float_as_uint(v[8 * d]);   // all four bytes are overwritten
#pragma unroll
        for (int b = 0; b < 4; ++b) w = fp4_enc(w, v[8 * d + 2 * b], v[8 * d + 2 * b + 1], p, b);
        D[d] = w;
    }
}

// acc[e] (+)= code_e * 2^e (dm = 2^e).  ROUNDED: the conversion applies 2^e
// and rounds, so a product beyond binary32 is +-inf before the add.
template <bool FIRST, int H, bool ROUNDED = false>
__device__ __forceinline__ void mx_accumulate(const uint32_t (&D)[4], const float (&dm)[H], float (&acc)[32])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float p = dm[H == 2 ? d / 2 : 0];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (ROUNDED) {                         // the conversion applies 2^e and rounds
                const f2 v = fp4_dec(D[d], p, b);
                if (FIRST) { acc[8 * d + 2 * b] = v.x; acc[8 * d + 2 * b + 1] = v.y; }
                else {
                    acc[8 * d + 2 * b] = __fadd_rn(acc[8 * d + 2 * b], v.x);
                    acc[8 * d + 2 * b + 1] = __fadd_rn(acc[8 * d + 2 * b + 1], v.y);
                }
                continue;
            }
            const f2 c = fp4_dec(D[d], 1.0f, b);            // code value, exact
            if (FIRST) { acc[8 * d + 2 * b] = c.x * p; acc[8 * d + 2 * b + 1] = c.y * p; }
            else {                                            // c * 2^e is exact: one rounding
                acc[8 * d + 2 * b] = __builtin_fmaf(c.x, p, acc[8 * d + 2 * b]);
                acc[8 * d + 2 * b + 1] = __builtin_fmaf(c.y, p, acc[8 * d + 2 * b + 1]);
            }
        }
    }
}

// ------------------------------------------------------ decode scales ----

// E8M0 byte -> 2^(byte - 127 + k); the NaN byte makes every product NaN.
template <int K>
__device__ __forceinline__ float e8m0_mult(uint32_t b)
{
    return (b == 255u) ? __builtin_nanf("") : __builtin_ldexpf(1.0f, (int)b - 127 + K);
}

// Decode multiplier of one block from its stored scale bits: what the
// format's code value (as the conversion instructions return it) is
// multiplied by.  P: the sums are held at 2^-P of their value (INT with FP16
// scales in the reduce: P = 1 for INT3, 9 for INT4, where the multiplier is
// then the fp16 scale itself).
template <int FMT, int SC, int P = 0>
__device__ __forceinline__ float dec_mult(uint32_t bits)
{
    if constexpr (SC == kS16) {
        const float s = __half2float(__ushort_as_half((unsigned short)bits));
        if constexpr (FMT == 2) return P == 1 ? s : 2.0f * s;       // E2M1 value q/2
        else if constexpr (FMT == 1) return P == 9 ? s : 512.0f * s; // E4M3 subnormal q 2^-9
        else return s;
    } else if constexpr (SC == kS32) {
        return __uint_as_float(bits);
    } else {
        if constexpr (FMT == 2) return e8m0_mult<1>(bits);
        else return e8m0_mult<0>(bits);                   // INT4: codes decoded as q (scale operand 512)
    }
}

}  // namespace rc
