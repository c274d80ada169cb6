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
//     clear.  Quantize = E2M1 conversion of x * (r/2), r = fp32(1/s);
//     dequantize = E2M1 conversion back, times 2s.
//   * INT4 magnitudes 0..7 are the E4M3 subnormals m * 2^-9, so a sign /
//     magnitude INT4 code is an E4M3 byte with exponent 0.
// Both conversions round their binary32 input to nearest even, which is the
// INT rounding rule itself: magnitude = min(RNE(fp32(|x| * fp32(1/s))), qmax).
// Below the clamp the code's low bit is the parity of the integer, so ties
// go the same way.  For a normal, unsaturated fp16 scale |x| * r <= qmax +
// 0.004, so no clamp is needed; for a subnormal or saturated scale the clamp
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

__device__ __forceinline__ float absmax32(const float (&v)[32])
{
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; e += 2) a = fmaxf(fmaxf(fabsf(v[e]), fabsf(v[e + 1])), a);
    return a;
}

// ------------------------------------------------------- INT scale rule ----

struct IntScale {
    float s;          // fp16 scale as binary32 (exact)
    uint32_t bits;    // fp16 bit pattern
    float r;          // fp32(1/s) (IEEE division), 0 for a zero block
    bool zero;        // s == 0: the block is stored as zeros
    bool abnormal;    // subnormal fp16 or saturated: codes need the clamp
};

// Correctly rounded a / b for a constant b: q = a * RN(1/b), then one
// residual correction.  For b = 3, 7 and 448 this equals the IEEE quotient
// for every finite a >= 0 (448: wherever the quotient is normal), which an
// exhaustive run over all binary32 inputs confirms; an infinite a gives NaN.
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
    return r;
}

__device__ __forceinline__ uint32_t signbit_u(float x) { return __float_as_uint(x) >> 31; }

// ----------------------------------------------------------------- INT3 ----
// Group word g (g = 0..3) of a block holds in nibble j the code of element
// 4j + g: (sign << 3) | magnitude.  Plane words:
//   q2w word 0 = (N0 & 0x33333333) | ((N1 & 0x33333333) << 2)
//   q2w word 1 = (N2 & 0x33333333) | ((N3 & 0x33333333) << 2)
//   q1w word   = sign of element e at bit e.

struct Int3Words { uint32_t w0, w1, h, sbits; };

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

// E2M1 nibbles of the 32 elements, group g in word N[g] (nibble j = element
// 4j + g), of x * r2 with r2 = fp32(1/s) / 2.
__device__ __forceinline__ void int3_groups(const float (&v)[32], float r2, uint32_t (&N)[4])
{
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t w = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) w = fp4_enc(w, v[8 * b + g] * r2, v[8 * b + 4 + g] * r2, 1.0f, b);
        N[g] = w;
    }
}

// min(magnitude, 3) on E2M1 nibbles: a magnitude code with bit 2 set (an E2M1
// value of 2 or more, i.e. an INT3 magnitude of 4 or more) becomes 3.
__device__ __forceinline__ uint32_t int3_clamp_word(uint32_t w)
{
    const uint32_t big = (w >> 2) & 0x11111111u;
    return (w & 0x88888888u) | (w & 0x33333333u) | (big * 3u);
}

__device__ __forceinline__ Int3Words int3_encode_block(const float (&v)[32])
{
    const IntScale sc = int_scale<3>(absmax32(v));
    const float r2 = 0.5f * sc.r;                       // exact
    uint32_t N[4];
    int3_groups(v, r2, N);
    // Only a subnormal or saturated scale lets |x| * r exceed 3 + 1/2.
    if (sc.abnormal) {
#pragma unroll
        for (int g = 0; g < 4; ++g) N[g] = int3_clamp_word(N[g]);
    }
    const uint32_t keep = sc.zero ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int g = 0; g < 4; ++g) N[g] &= keep;
    Int3Words o = int3_planes(N);
    o.sbits = sc.zero ? 0u : sc.bits;
    return o;
}

// acc[e] (+)= q_e * s for the 32 elements of one INT3 block.
template <bool FIRST>
__device__ __forceinline__ void int3_accumulate(uint32_t w0, uint32_t w1, uint32_t h, uint32_t sbits,
                                                float (&acc)[32])
{
    const float s2 = 2.0f * __half2float(__ushort_as_half((unsigned short)sbits));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t Ng = int3_group(w0, w1, h, g);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f2 c = fp4_dec(Ng, 1.0f, b);
            if (FIRST) { acc[8 * b + g] = c.x * s2; acc[8 * b + 4 + g] = c.y * s2; }
            else {
                acc[8 * b + g] = __builtin_fmaf(c.x, s2, acc[8 * b + g]);
                acc[8 * b + 4 + g] = __builtin_fmaf(c.y, s2, acc[8 * b + 4 + g]);
            }
        }
    }
}

// ----------------------------------------------------------------- INT4 ----
// Word d (d = 0..3) of a block holds elements 8d..8d+7, element 8d+j in
// nibble j: (sign << 3) | magnitude.  E4M3 view: byte = (sign << 7) | m.

struct Int4Words { uint32_t d[4]; uint32_t sbits; };

// min(magnitude, 7) on four E4M3 bytes of INT4 codes: a byte with a nonzero
// exponent field (value 8 * 2^-9 or more) gets mantissa bits 111; only the
// mantissa and sign bits are packed afterwards.
__device__ __forceinline__ uint32_t int4_clamp_bytes(uint32_t x)
{
    const uint32_t big = (((x & 0x78787878u) + 0x78787878u) >> 7) & 0x01010101u;
    return x | big | (big << 1) | (big << 2);
}

__device__ __forceinline__ Int4Words int4_encode_block(const float (&v)[32])
{
    const IntScale sc = int_scale<7>(absmax32(v));
    const float r9 = sc.r * 0x1p-9f;                    // exact
    // E4M3 subnormal bytes of x * r9: word d's even elements 0,2,4,6 in the
    // bytes of xe[d], odd elements 1,3,5,7 in xo[d]
    uint32_t xe[4], xo[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float* y = v + 8 * d;
        xe[d] = fp8_pair(y[4] * r9, y[6] * r9, fp8_pair(y[0] * r9, y[2] * r9, 0u, false), true);
        xo[d] = fp8_pair(y[5] * r9, y[7] * r9, fp8_pair(y[1] * r9, y[3] * r9, 0u, false), true);
    }
    // Only a subnormal or saturated scale lets |x| * r exceed 7 + 1/2.
    if (sc.abnormal) {
#pragma unroll
        for (int d = 0; d < 4; ++d) { xe[d] = int4_clamp_bytes(xe[d]); xo[d] = int4_clamp_bytes(xo[d]); }
    }
    const uint32_t keep = sc.zero ? 0u : 0xFFFFFFFFu;
    Int4Words o;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        o.d[d] = ((xe[d] & 0x07070707u) | ((xe[d] >> 4) & 0x08080808u) | ((xo[d] << 4) & 0x70707070u) |
                  (xo[d] & 0x80808080u)) & keep;
    o.sbits = sc.zero ? 0u : sc.bits;
    return o;
}

template <bool FIRST>
__device__ __forceinline__ void int4_accumulate(const uint32_t (&D)[4], uint32_t sbits, float (&acc)[32])
{
    const float s9 = 512.0f * __half2float(__ushort_as_half((unsigned short)sbits));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t xe = (D[d] & 0x07070707u) | ((D[d] << 4) & 0x80808080u);
        const uint32_t xo = ((D[d] >> 4) & 0x07070707u) | (D[d] & 0x80808080u);
        const f2 e01 = fp8_dec(xe, false), e23 = fp8_dec(xe, true);
        const f2 o01 = fp8_dec(xo, false), o23 = fp8_dec(xo, true);
        const float cs[8] = {e01.x, o01.x, e01.y, o01.y, e23.x, o23.x, e23.y, o23.y};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (FIRST) acc[8 * d + j] = cs[j] * s9;
            else acc[8 * d + j] = __builtin_fmaf(cs[j], s9, acc[8 * d + j]);
        }
    }
}

// ------------------------------------------------------------------ FP8 ----
// Byte e of the block's 32 code bytes = E4M3 code of element e.

struct Fp8Words { uint32_t d[8]; float s; };

// Round-to-odd binary32 value of the exact quotient |x| / s, with the sign
// of x and clamped to 448; its round-to-nearest-even E4M3 conversion equals
// that of the exact quotient (binary32 carries more than 4 + 2 significant
// bits).  rs is the hardware reciprocal of s (within 1 ulp):
//   y0 = |x| * rs is within 3 ulp of the quotient q,
//   y1 = y0 + fma(-y0, s, |x|) * rs is within 1/2 ulp (plus 2^-20 ulp) of q,
//   and the sign of r = fma(-y1, s, |x|) (zero only when y1 = q) says on
//   which side of y1 the quotient lies.
// The residuals must not underflow: callers pass s >= 2^-64 (smaller block
// scales are handled by multiplying x and s by 2^64).
__device__ __forceinline__ float fp8_ro_quotient(float x, float s, float rs)
{
    const float ax = fabsf(x);
    const float y0 = ax * rs;
    const float y1 = __builtin_fmaf(__builtin_fmaf(-y0, s, ax), rs, y0);
    const float r = __builtin_fmaf(-y1, s, ax);
    uint32_t t = __float_as_uint(y1);
    t = (t - (r < 0.0f ? 1u : 0u)) | (r != 0.0f ? 1u : 0u);
    const float yo = fminf(__uint_as_float(t), 448.0f);
    return __uint_as_float(__float_as_uint(yo) | (__float_as_uint(x) & 0x80000000u));
}

__device__ __forceinline__ void fp8_codes(const float (&v)[32], float k, float sk, uint32_t (&d)[8])
{
    const float rs = __builtin_amdgcn_rcpf(sk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float* x = v + 4 * i;
        uint32_t w = fp8_pair(fp8_ro_quotient(x[0] * k, sk, rs), fp8_ro_quotient(x[1] * k, sk, rs), 0u, false);
        d[i] = fp8_pair(fp8_ro_quotient(x[2] * k, sk, rs), fp8_ro_quotient(x[3] * k, sk, rs), w, true);
    }
}

__device__ __forceinline__ Fp8Words fp8_encode_block(const float (&v)[32])
{
    Fp8Words o;
    const float a = absmax32(v);
    const float s = (a == __builtin_inff()) ? a : div_by<448>(a);   // inf / 448 = inf
    const bool zero = !(s >= 0x1p-126f);
    o.s = zero ? 0.0f : s;
    if (!(s < 0x1p-64f)) {
        fp8_codes(v, 1.0f, s, o.d);
    } else {                                  // tiny scale: x * 2^64 and s * 2^64 are exact
        fp8_codes(v, 0x1p64f, s * 0x1p64f, o.d);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) o.d[i] = zero ? 0u : o.d[i];
    return o;
}

template <bool FIRST>
__device__ __forceinline__ void fp8_accumulate(const uint32_t (&D)[8], float s, float (&acc)[32])
{
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        const f2 lo = fp8_dec(D[d], false), hi = fp8_dec(D[d], true);
        const float c[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float dv = __fmul_rn(c[j], s);                 // RN32(code * s)
            if (FIRST) acc[4 * d + j] = dv;
            else acc[4 * d + j] = __fadd_rn(acc[4 * d + j], dv);  // RN32(acc + d)
        }
    }
}

// ---------------------------------------------------------------- MXFP4 ----
// Word d holds elements 8d..8d+7 (element 8d+j in nibble j), E2M1 codes.

struct MxWords { uint32_t d[4]; uint32_t e8; };

// floor(log2 a) of a positive finite binary32, subnormals included.
__device__ __forceinline__ int ilog2f(float a)
{
    const uint32_t b = __float_as_uint(a);
    const int ef = (int)(b >> 23);
    return ef ? ef - 127 : (31 - (int)__builtin_clz(b)) - 149;
}

__device__ __forceinline__ MxWords mx_encode_block(const float (&v)[32])
{
    MxWords o;
    const float a = absmax32(v);
    int e = (a == 0.0f) ? -127 : ilog2f(a) - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    o.e8 = (uint32_t)(e + 127);
    const float p = __builtin_ldexpf(1.0f, e);          // 2^e, subnormal for e < -126
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t w = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) w = fp4_enc(w, v[8 * d + 2 * b], v[8 * d + 2 * b + 1], p, b);
        o.d[d] = w;
    }
    return o;
}

template <bool FIRST>
__device__ __forceinline__ void mx_accumulate(const uint32_t (&D)[4], uint32_t e8, float (&acc)[32])
{
    // 2^(e8-127) (subnormal below 2^-126); the E8M0 NaN byte makes every product NaN
    const float p = (e8 == 255u) ? __builtin_nanf("") : __builtin_ldexpf(1.0f, (int)e8 - 127);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f2 c = fp4_dec(D[d], 1.0f, b);            // code value, exact
            if (FIRST) { acc[8 * d + 2 * b] = c.x * p; acc[8 * d + 2 * b + 1] = c.y * p; }
            else {                                            // c * 2^e is exact: one rounding
                acc[8 * d + 2 * b] = __builtin_fmaf(c.x, p, acc[8 * d + 2 * b]);
                acc[8 * d + 2 * b + 1] = __builtin_fmaf(c.y, p, acc[8 * d + 2 * b + 1]);
            }
        }
    }
}

}  // namespace rc
