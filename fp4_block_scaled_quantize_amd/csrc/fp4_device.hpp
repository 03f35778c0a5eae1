// fp4_device.hpp -- device-side building blocks for the gfx950 kernels:
// bf16 unpacking, block-scale encode/decode, E2M1 element encode/decode,
// wave64 group reductions and the Philox4x32-10 counter-based generator.
//
// Formats (quant_prune_distill/486 "Метод"; gonzo_ML/3986 "Форматы FP4";
// ue5m3-fp4-pretraining "Что сделали"): E2M1 elements; block scales in an
// ExMy encoding (bias 2^(x-1)-1, subnormals, no infinity, the all-ones code
// is NaN) or E8M0 (2^(code-127)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bits_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __float_as_uint(f); }

// bf16 pair packed in a dword -> two fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// block-scale formats
// ---------------------------------------------------------------------------
struct ScaleFmt {
    int32_t ebits, mbits, bias, maxcode;   // ExMy parameters (unused for E8M0)
    float smax;                            // largest finite value
    int32_t is_e8m0;
};

// Nearest-even, saturating ExMy encode of u >= 0.  In the binade of u (or
// the subnormal range), t = u * 2^(mbits - e) is exact and its integer part
// indexes the code directly: code = ((e + bias - 1) << mbits) + floor(t),
// rounded up past the midpoint and, on an exact midpoint, to the even code.
__device__ __forceinline__ uint32_t scale_encode_exmy(float u, const ScaleFmt& f)
{
    if (!(u < f.smax)) return (u >= f.smax) ? (uint32_t)f.maxcode : 0u;
    uint32_t ub = f_bits(u);
    int eu = (int)((ub >> 23) & 0xFFu) - 127;          // floor(log2 u) for normal u
    int emin = 1 - f.bias;
    int e = eu > emin ? eu : emin;                      // fp32 subnormals fall below emin
    float t = __builtin_amdgcn_ldexpf(u, f.mbits - e);
    float fl = __builtin_floorf(t);
    float fr = t - fl;
    uint32_t lo = ((uint32_t)(e + f.bias - 1) << f.mbits) + (uint32_t)fl;
    uint32_t up = (fr > 0.5f) | ((fr == 0.5f) & (lo & 1u));
    uint32_t code = lo + up;
    return code < (uint32_t)f.maxcode ? code : (uint32_t)f.maxcode;
}

__device__ __forceinline__ float scale_decode_exmy(uint32_t code, const ScaleFmt& f)
{
    uint32_t e = code >> f.mbits;
    uint32_t m = code & ((1u << f.mbits) - 1u);
    float sig = (float)(e == 0 ? m : (m | (1u << f.mbits)));
    int ex = (e == 0 ? 1 : (int)e) - f.bias - f.mbits;
    return __builtin_amdgcn_ldexpf(sig, ex);
}

// Decode any scale byte: sign bit above ebits+mbits for signed formats, the
// all-ones magnitude is NaN; E8M0: 2^(code-127), 0xFF is NaN.
__device__ __forceinline__ float scale_decode_any(uint32_t code, const ScaleFmt& f)
{
    if (f.is_e8m0) {
        if (code == 0xFFu) return __uint_as_float(0x7FC00000u);
        return bits_f(code ? code << 23 : 0x00400000u);
    }
    const int nb = f.ebits + f.mbits;
    const uint32_t magmask = (1u << nb) - 1u;
    const uint32_t mag = code & magmask;
    if (mag == magmask) return __uint_as_float(0x7FC00000u);
    float v = scale_decode_exmy(mag, f);
    return (nb == 7 && (code & 0x80u)) ? -v : v;
}

// E8M0 block code: floor(log2 amax_b) - 2 + 127, clamped to [0, 254]; for a
// normal amax_b this is its biased exponent minus 2.
__device__ __forceinline__ uint32_t scale_code_e8m0(float amax_b)
{
    int ex = (int)((f_bits(amax_b) >> 23) & 0xFFu);
    return (uint32_t)(ex > 2 ? ex - 2 : 0);
}

// As scale_code_e8m0 with the element grid's offset EMAX (the block maximum
// lands in [2^EMAX, 2^(EMAX+1)) after scaling): 8 for FP8 E4M3 elements, 6
// for INT8.
template <int EMAX>
__device__ __forceinline__ uint32_t scale_code_e8m0_emax(float amax_b)
{
    int ex = (int)((f_bits(amax_b) >> 23) & 0xFFu);
    return (uint32_t)(ex > EMAX ? ex - EMAX : 0);
}

// 2^(127 - code): exact reciprocal of an E8M0 scale, code in [0, 252].
__device__ __forceinline__ float e8m0_inv(uint32_t code) { return bits_f((254u - code) << 23); }

// ---------------------------------------------------------------------------
// E2M1 elements
// ---------------------------------------------------------------------------
// Hardware pack: two fp32 -> two E2M1 codes (round to nearest even,
// saturating, sign kept) into byte `sel` of `old`, scale 1.
#define FP4_CVT_PK(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// Software E2M1 nearest-even magnitude code of |v| (saturating at 6): in each
// binade of the grid the spacing is a power of two, so a scaled rint with an
// offset gives the code: [0,2) step 0.5, [2,4) step 1, [4,8) step 2.
__device__ __forceinline__ uint32_t e2m1_rtn_sw(float v)
{
    float a = __builtin_fabsf(v);
    float sp = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
    float off = a < 2.0f ? 0.0f : (a < 4.0f ? 2.0f : 4.0f);
    float c = __builtin_fminf(__builtin_rintf(a * sp) + off, 7.0f);
    return (uint32_t)c | ((f_bits(v) >> 28) & 8u);
}

// Stochastic E2M1 codes through the gfx950 scaled SR conversion.  The
// reading: the magnitude rounds up from its lower grid neighbour lo iff
// r16 / 2^16 < frac, frac = (|v| - lo) / (hi - lo).  Measured behaviour of
// v_cvt_scalef32_sr_pk_fp4_f32 on its first element: with the scale's power
// of two 2^k it takes w = v / 2^k and rounds up iff
// floor(frac(w) * 2^32) + seed >= 2^32 (the second element derives its
// random bits from the seed differently, so it is always given 0 here).
// Two exact steps make that rule the reading's:
//  - w is |v| rounded up to a multiple of 2^-17 (sign kept), passed as
//    ceil(|v| 2^17) with scale 2^17.  Every grid spacing is at least 1/2, so
//    frac(w) * 2^16 rounds frac(v) * 2^16 up to the next multiple of
//    2^-1, 2^-2 or 2^-3 (never past the next integer: the comparison with
//    the integer r16 is unchanged), and frac(w) * 2^32 is an integer.
//  - seed = 2^32 - 1 - r16 * 2^16 = (~r16 << 16) | 0xFFFF, so the rule reads
//    r16 * 2^16 < frac(w) * 2^32.
// |v| >= 6 (and infinities) saturate to 6 as in the reading; the sign of v,
// zero included, is kept.  Checked against the reading on every binary32
// within 3000 ulps of each grid point and midpoint, 300000 random values
// below 7 (subnormals included) and values next to multiples of 2^-17, at
// the boundary variates of each and random ones.
__device__ __forceinline__ float e2m1_sr_operand(float v)
{
    return __builtin_copysignf(__builtin_ceilf(__builtin_fabsf(v) * 0x1p17f), v);
}

typedef float fp4_f2 __attribute__((ext_vector_type(2)));

// The conversion writes byte J of its destination and keeps the other three
// (checked on the device).  The compiler's builtin for it does not tie the
// destination to the value passed as the old one, so the instruction is
// written here with the destination as an in/out operand.
template <int J>
__device__ __forceinline__ uint32_t e2m1_sr_byte(uint32_t old, float v, uint32_t seed)
{
    const fp4_f2 pr = {e2m1_sr_operand(v), 0.0f};
    const float scale = 0x1p17f;
    if constexpr (J == 0)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(old) : "v"(pr), "v"(seed), "s"(scale));
    else if constexpr (J == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(old) : "v"(pr), "v"(seed), "s"(scale));
    else if constexpr (J == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(old) : "v"(pr), "v"(seed), "s"(scale));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(old) : "v"(pr), "v"(seed), "s"(scale));
    return old;
}

// Four stochastic E2M1 codes, element k in nibble k, from the 16-bit halves
// of two random words (element 2j takes the low half of w[j], 2j + 1 the
// high half).
__device__ __forceinline__ uint32_t e2m1_sr_pack4(float v0, float v1, float v2, float v3, uint32_t w0, uint32_t w1)
{
    const uint32_t n0 = ~w0, n1 = ~w1;
    uint32_t even = e2m1_sr_byte<0>(0u, v0, (n0 << 16) | 0xFFFFu);
    uint32_t odd = e2m1_sr_byte<0>(0u, v1, n0 | 0xFFFFu);
    even = e2m1_sr_byte<1>(even, v2, (n1 << 16) | 0xFFFFu);
    odd = e2m1_sr_byte<1>(odd, v3, n1 | 0xFFFFu);
    return even | (odd << 4);
}

// Eight stochastic E2M1 codes, element k in nibble k (the units' layout).
__device__ __forceinline__ uint32_t e2m1_sr_pack8(const float v[8], uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3)
{
    const uint32_t n0 = ~w0, n1 = ~w1, n2 = ~w2, n3 = ~w3;
    uint32_t even = e2m1_sr_byte<0>(0u, v[0], (n0 << 16) | 0xFFFFu);
    uint32_t odd = e2m1_sr_byte<0>(0u, v[1], n0 | 0xFFFFu);
    even = e2m1_sr_byte<1>(even, v[2], (n1 << 16) | 0xFFFFu);
    odd = e2m1_sr_byte<1>(odd, v[3], n1 | 0xFFFFu);
    even = e2m1_sr_byte<2>(even, v[4], (n2 << 16) | 0xFFFFu);
    odd = e2m1_sr_byte<2>(odd, v[5], n2 | 0xFFFFu);
    even = e2m1_sr_byte<3>(even, v[6], (n3 << 16) | 0xFFFFu);
    odd = e2m1_sr_byte<3>(odd, v[7], n3 | 0xFFFFu);
    return even | (odd << 4);
}

// E2M1 magnitude code -> value (exact): code 0..7 -> 0,.5,1,1.5,2,3,4,6.
__device__ __forceinline__ float e2m1_value(uint32_t nib)
{
    uint32_t e = (nib >> 1) & 3u, m = nib & 1u;
    // normal: (1 + m/2) * 2^(e-1) = bits (e + 126) << 23 | m << 22 ; subnormal: m * 0.5
    float mag = e ? bits_f(((e + 126u) << 23) | (m << 22)) : (m ? 0.5f : 0.0f);
    return (nib & 8u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// INT4 elements (quant_prune_distill/574 "Метод": the NV and MX block/scale
// schemes paired with an integer grid, NVINT4 / MXINT4).  Reading: the
// symmetric grid -7..7 as two's-complement nibbles (zero has no sign),
// nearest with ties to the even integer, saturating at 7; stochastic
// rounding with grid spacing 1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t int4_nibble(float v, float mag)
{
    const uint32_t m = (uint32_t)mag;
    return (f_bits(v) >> 31) ? ((16u - m) & 15u) : m;
}

// Clamping to the integer bounds commutes with the nearest-even rounding, so
// the signed integer of RN(clamp(v, -7, 7)), masked to 4 bits, is the
// two's-complement code (rint(-0.4) = -0 converts to 0: zero has no sign).
__device__ __forceinline__ uint32_t int4_rtn_code(float v)
{
    return (uint32_t)(int32_t)__builtin_rintf(__builtin_amdgcn_fmed3f(v, -7.0f, 7.0f)) & 15u;
}

__device__ __forceinline__ uint32_t int4_sr_code(float v, uint32_t r16)
{
    const float a = __builtin_fabsf(v);
    const float fl = __builtin_floorf(a);
    const float frac = a - fl;                                     // exact
    const float up = ((float)r16 < frac * 65536.0f) ? 1.0f : 0.0f;
    return int4_nibble(v, a >= 7.0f ? 7.0f : fl + up);
}

__device__ __forceinline__ float int4_value(uint32_t nib) { return (float)((int32_t)(nib << 28) >> 28); }

// ---------------------------------------------------------------------------
// 8-bit MX elements (quant_prune_distill/574 "Метод": MXFP8 / MXINT8).
// Reading: FP8 E4M3 elements, nearest-even and saturating at 448, the sign
// bit kept (also for zero); INT8 on the symmetric grid -127..127 (two's
// complement, zero unsigned).  One byte per element.
// ---------------------------------------------------------------------------
constexpr ScaleFmt kFp8E4M3{4, 3, 7, 0x7E, 448.0f, 0};

// Four RTN codes, element k in byte k: clamp to the largest finite value,
// then the hardware OCP E4M3 conversion (nearest-even, subnormals, sign of
// zero kept): on every finite input the nearest-even E4M3 encoding that
// saturates at 448.
__device__ __forceinline__ uint32_t fp8_rtn_pack4(float v0, float v1, float v2, float v3)
{
    const float c0 = __builtin_amdgcn_fmed3f(v0, -448.0f, 448.0f), c1 = __builtin_amdgcn_fmed3f(v1, -448.0f, 448.0f);
    const float c2 = __builtin_amdgcn_fmed3f(v2, -448.0f, 448.0f), c3 = __builtin_amdgcn_fmed3f(v3, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
    return (uint32_t)w;
}

// Stochastic: in the binade e of |v| (e >= -6; below 2^-6 the subnormal
// spacing 2^-9) t = |v| 2^(3-e) is exact, floor(t) indexes the lower grid
// neighbour and the code ((e + 7) << 3) + m - 8 also covers the carry into
// the next binade and the subnormals.
__device__ __forceinline__ uint32_t fp8_sr_code(float v, uint32_t r16)
{
    const float a = __builtin_fabsf(v);
    const uint32_t sign = (f_bits(v) >> 24) & 0x80u;
    if (!(a < 448.0f)) return 0x7Eu | sign;
    const int eu = (int)((f_bits(a) >> 23) & 0xFFu) - 127;
    const int e = eu > -6 ? eu : -6;
    const float t = __builtin_amdgcn_ldexpf(a, 3 - e);
    const float fl = __builtin_floorf(t);
    const float frac = t - fl;
    const uint32_t m = (uint32_t)fl + (((float)r16 < frac * 65536.0f) ? 1u : 0u);
    const uint32_t code = (uint32_t)((e + 7) << 3) + m - 8u;
    return (code < 0x7Eu ? code : 0x7Eu) | sign;
}

__device__ __forceinline__ uint32_t int8_rtn_code(float v)
{
    return (uint32_t)(int32_t)__builtin_rintf(__builtin_amdgcn_fmed3f(v, -127.0f, 127.0f)) & 0xFFu;
}

__device__ __forceinline__ uint32_t int8_sr_code(float v, uint32_t r16)
{
    const float a = __builtin_fabsf(v);
    const float fl = __builtin_floorf(a);
    const float frac = a - fl;                                      // exact
    const float up = ((float)r16 < frac * 65536.0f) ? 1.0f : 0.0f;
    const uint32_t m = (uint32_t)(a >= 127.0f ? 127.0f : fl + up);
    return (f_bits(v) >> 31) ? ((256u - m) & 0xFFu) : m;
}

__device__ __forceinline__ float int8_value(uint32_t b) { return (float)(int32_t)(int8_t)(b & 0xFFu); }

// ---------------------------------------------------------------------------
// 6-bit MX elements (quant_prune_distill/574 "Метод": MXFP6 / MXINT6).
// Reading: the OCP FP6 element formats E2M3 (bias 1, largest 7.5) and E3M2
// (bias 3, largest 28), sign bit 5, subnormals, every code finite; INT6 on
// the symmetric grid -31..31 (six-bit two's complement).  Element c of a
// row sits at bits 6c .. 6c + 5 of the row (a little-endian bit stream).
// ---------------------------------------------------------------------------
constexpr ScaleFmt kFp6E2M3{2, 3, 1, 0x1F, 7.5f, 0};
constexpr ScaleFmt kFp6E3M2{3, 2, 3, 0x1F, 28.0f, 0};

__device__ __forceinline__ uint32_t fp6_rtn_code(float v, const ScaleFmt& f)
{
    return scale_encode_exmy(__builtin_fabsf(v), f) | ((f_bits(v) >> 26) & 0x20u);
}

// Stochastic, as fp8_sr_code: in the binade e of |v| (at least the
// subnormal exponent 1 - BIAS) t = |v| 2^(MB - e) is exact, floor(t) is the
// lower neighbour's significand and ((e + BIAS) << MB) + m - 2^MB its code.
template <int MB, int BIAS>
__device__ __forceinline__ uint32_t fp6_sr_code(float v, uint32_t r16, float smax)
{
    const float a = __builtin_fabsf(v);
    const uint32_t sign = (f_bits(v) >> 26) & 0x20u;
    if (!(a < smax)) return 0x1Fu | sign;
    const int eu = (int)((f_bits(a) >> 23) & 0xFFu) - 127;
    const int e = eu > 1 - BIAS ? eu : 1 - BIAS;
    const float t = __builtin_amdgcn_ldexpf(a, MB - e);
    const float fl = __builtin_floorf(t);
    const float frac = t - fl;
    const uint32_t m = (uint32_t)fl + (((float)r16 < frac * 65536.0f) ? 1u : 0u);
    const uint32_t code = (uint32_t)((e + BIAS) << MB) + m - (1u << MB);
    return (code < 0x1Fu ? code : 0x1Fu) | sign;
}

__device__ __forceinline__ float fp6_value(uint32_t c, const ScaleFmt& f)
{
    const float v = scale_decode_exmy(c & 0x1Fu, f);
    return (c & 0x20u) ? -v : v;
}

__device__ __forceinline__ uint32_t int6_rtn_code(float v)
{
    return (uint32_t)(int32_t)__builtin_rintf(__builtin_amdgcn_fmed3f(v, -31.0f, 31.0f)) & 0x3Fu;
}

__device__ __forceinline__ uint32_t int6_sr_code(float v, uint32_t r16)
{
    const float a = __builtin_fabsf(v);
    const float fl = __builtin_floorf(a);
    const float frac = a - fl;
    const float up = ((float)r16 < frac * 65536.0f) ? 1.0f : 0.0f;
    const uint32_t m = (uint32_t)(a >= 31.0f ? 31.0f : fl + up);
    return (f_bits(v) >> 31) ? ((64u - m) & 0x3Fu) : m;
}

__device__ __forceinline__ float int6_value(uint32_t c) { return (float)(((int32_t)(c << 26)) >> 26); }

// Four FP6 RTN codes packed at bits 0, 6, 12, 18.  FP6 E2M3 is FP8 E4M3
// scaled by 2^-6 (the E4M3 minimum normal 2^-6 and subnormal spacing 2^-9
// are E2M3's 1 and 2^-3 times 2^-6, both with 3 mantissa bits), and FP6 E3M2
// is FP8 E5M2 scaled by 2^-12 (2^-14 and 2^-16 against 2^-2 and 2^-4, 2
// mantissa bits).  So after the saturating clamp and the exact power-of-two
// scaling the hardware OCP FP8 / BF8 conversion (nearest-even) yields the
// FP6 magnitude in its low 5 bits; the sign moves from bit 7 to bit 5.
template <int ELEM>
__device__ __forceinline__ uint32_t fp6_rtn_pack4_hw(float v0, float v1, float v2, float v3)
{
    constexpr float kMax = ELEM == 4 ? 7.5f : 28.0f;
    constexpr float kShift = ELEM == 4 ? 0x1p-6f : 0x1p-12f;
    const float c0 = __builtin_amdgcn_fmed3f(v0, -kMax, kMax) * kShift;
    const float c1 = __builtin_amdgcn_fmed3f(v1, -kMax, kMax) * kShift;
    const float c2 = __builtin_amdgcn_fmed3f(v2, -kMax, kMax) * kShift;
    const float c3 = __builtin_amdgcn_fmed3f(v3, -kMax, kMax) * kShift;
    int w;
    if constexpr (ELEM == 4) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c0, c1, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c2, c3, w, true);
    }
    const uint32_t b = ((uint32_t)w & 0x1F1F1F1Fu) | (((uint32_t)w >> 2) & 0x20202020u);   // 6-bit codes per byte
    return (b & 0x3Fu) | ((b >> 2) & (0x3Fu << 6)) | ((b >> 4) & (0x3Fu << 12)) | ((b >> 6) & (0x3Fu << 18));
}

// One element grid's code of v (ELEM 4 FP6 E2M3, 5 FP6 E3M2, 6 INT6).
template <int ELEM>
__device__ __forceinline__ uint32_t w6_rtn_code(float v)
{
    if constexpr (ELEM == 6) return int6_rtn_code(v);
    else return fp6_rtn_code(v, ELEM == 4 ? kFp6E2M3 : kFp6E3M2);
}

template <int ELEM>
__device__ __forceinline__ uint32_t w6_sr_code(float v, uint32_t r16)
{
    if constexpr (ELEM == 6) return int6_sr_code(v, r16);
    else if constexpr (ELEM == 4) return fp6_sr_code<3, 1>(v, r16, 7.5f);
    else return fp6_sr_code<2, 3>(v, r16, 28.0f);
}

template <int ELEM>
__device__ __forceinline__ float w6_value(uint32_t c)
{
    if constexpr (ELEM == 6) return int6_value(c);
    else return fp6_value(c, ELEM == 4 ? kFp6E2M3 : kFp6E3M2);
}

// ---------------------------------------------------------------------------
// wave64 helpers
// ---------------------------------------------------------------------------
// Max of non-negative binary32 bit patterns across lane pairs / quads.
__device__ __forceinline__ uint32_t dpp_umax_xor1(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    return v > o ? v : o;
}
__device__ __forceinline__ uint32_t dpp_umax_xor2(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    return v > o ? v : o;
}

// Max across lane pairs / quads with DPP quad permutations.
__device__ __forceinline__ float dpp_max_xor1(float v)
{
    int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    return __builtin_fmaxf(v, __int_as_float(o));
}
__device__ __forceinline__ float dpp_max_xor2(float v)
{
    int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    return __builtin_fmaxf(v, __int_as_float(o));
}

// ---------------------------------------------------------------------------
// Blockwise randomized Hadamard transform, applied before quantization
// (ue5m3-fp4-pretraining "Что сделали": a randomized Hadamard transform
// spreads outliers over the block before quantization; quant_prune_distill/
// 574 "Метод": Hadamard rotations bring distributions closer to Gaussian).
// A block of 8*G elements lives in G adjacent lanes, lane `sub` holding
// elements 8*sub .. 8*sub+7.  Forward: y = c * H * D * v, D negating element
// j where bit j of `signs` is set, H the Sylvester Hadamard matrix by
// butterfly stages h = 1, 2, 4 inside the lane and h = 8 (lane pairs), 16
// (lane quads) across lanes, each pair (i, i + h) becoming (a + b, a - b) in
// binary32; c = 1/sqrt(8 G) in binary32.  Inverse: v = D * (c * (H * y)).
// ---------------------------------------------------------------------------
constexpr float kRhtNorm16 = 0.25f;
constexpr float kRhtNorm32 = 0x1.6a09e6p-3f;     // 1/sqrt(32), nearest binary32

template <int G>
__device__ __forceinline__ void fwht_block(float v[8], uint32_t sub)
{
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i & h) continue;
            const float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
    // h = 8: the partner lane is sub ^ 1; the lower lane keeps a + b, the
    // upper one a - b with a the lower lane's element
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[k]), 0xB1, 0xF, 0xF, false));
        v[k] = (sub & 1u) ? o - v[k] : v[k] + o;
    }
    if (G == 4) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {                                   // h = 16: partner sub ^ 2
            const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[k]), 0x4E, 0xF, 0xF, false));
            v[k] = (sub & 2u) ? o - v[k] : v[k] + o;
        }
    }
}

template <int G>
__device__ __forceinline__ void rht_forward(float v[8], uint32_t sub, uint32_t signs)
{
    static_assert(G == 2 || G == 4, "blocks of 16 or 32");
    const uint32_t m = signs >> (8 * sub);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ((m >> k) & 1u) ? -v[k] : v[k];
    fwht_block<G>(v, sub);
    const float c = G == 2 ? kRhtNorm16 : kRhtNorm32;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = v[k] * c;
}

template <int G>
__device__ __forceinline__ void rht_inverse(float v[8], uint32_t sub, uint32_t signs)
{
    static_assert(G == 2 || G == 4, "blocks of 16 or 32");
    fwht_block<G>(v, sub);
    const uint32_t m = signs >> (8 * sub);
    const float c = G == 2 ? kRhtNorm16 : kRhtNorm32;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float t = v[k] * c;
        v[k] = ((m >> k) & 1u) ? -t : t;
    }
}

// The same transform on a block held whole by one lane (column-wise
// quantization): v[0 .. B-1], stages h = 1, 2, ..., B/2 in order.
template <int B>
__device__ __forceinline__ void rht_forward_lane(float v[B], uint32_t signs)
{
    static_assert(B == 16 || B == 32, "blocks of 16 or 32");
#pragma unroll
    for (int k = 0; k < B; ++k) v[k] = ((signs >> k) & 1u) ? -v[k] : v[k];
#pragma unroll
    for (int h = 1; h < B; h <<= 1) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            if (i & h) continue;
            const float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
    const float c = B == 16 ? kRhtNorm16 : kRhtNorm32;
#pragma unroll
    for (int k = 0; k < B; ++k) v[k] = v[k] * c;
}

// max |v| of N binary32 values as bits (non-negative floats order like
// their bit patterns)
template <int N>
__device__ __forceinline__ uint32_t absmax_bits_n(const float v[N])
{
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const uint32_t u = __float_as_uint(v[k]) & 0x7FFFFFFFu;
        m = m > u ? m : u;
    }
    return m;
}
__device__ __forceinline__ uint32_t absmax_bits8(const float v[8]) { return absmax_bits_n<8>(v); }

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): ten rounds, multipliers
// 0xD2511F53 / 0xCD9E8D57, Weyl key increments 0x9E3779B9 / 0xBB67AE85.
// ---------------------------------------------------------------------------
struct U4 { uint32_t x, y, z, w; };

// a ^ b ^ c in one gfx950 three-input bit operation (truth table 0x96); the
// compiler otherwise emits two xors when c is a scalar
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ U4 philox10(U4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)c.x * 0xD2511F53u;
        uint64_t p1 = (uint64_t)c.z * 0xCD9E8D57u;
        U4 n;
        n.x = xor3((uint32_t)(p1 >> 32), c.y, k0);
        n.y = (uint32_t)p1;
        n.z = xor3((uint32_t)(p0 >> 32), c.w, k1);
        n.w = (uint32_t)p0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

}  // namespace fp4
