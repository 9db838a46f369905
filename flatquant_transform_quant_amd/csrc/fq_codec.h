// Device-side element codecs of libfq: 16-bit loads, rounding of the intermediate to
// the input dtype, the int4 and E2M1 encoders and the e8m0 scale rules.
//
// Operator page "aclnnFlatQuantV2 算子拆解" ([FQV2]), section 拆开算: 第3步 (per-token
// int4 scale and per-group power-of-two scale), 第4步 (V2 ceil-exponent scale).  The
// E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} are those of the E2M1 table of the
// ModelOpt Conv3D page (section 6.1).  Rounding is half-to-even throughout.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fq_internal.h"

namespace fq {

template <int DT>
__device__ __forceinline__ float load16(uint16_t bits) {
  if constexpr (DT == kBF16) {
    return __uint_as_float(static_cast<uint32_t>(bits) << 16);
  } else {
    _Float16 h = __builtin_bit_cast(_Float16, bits);
    return static_cast<float>(h);
  }
}

// fp32 -> dtype, round to nearest even (hardware conversions).
template <int DT>
__device__ __forceinline__ uint16_t round16(float v) {
  if constexpr (DT == kBF16) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
}

// Two fp32 values -> two dtype values packed in one dword (low half = a), one
// v_cvt_pk_{bf16,f16}_f32 (round to nearest even).
template <int DT>
__device__ __forceinline__ uint32_t round16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  if constexpr (DT == kBF16) {
    typedef __attribute__((ext_vector_type(2))) __bf16 b16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, b16x2));
  } else {
    typedef __attribute__((ext_vector_type(2))) _Float16 h16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, h16x2));
  }
}

// int4 code of q = y / scale: round half to even, clamp to [-8, 7]; returns the 4-bit
// two's-complement nibble.
__device__ __forceinline__ uint32_t int4_nibble(float q) {
  float r = __builtin_rintf(q);
  r = fminf(fmaxf(r, -8.0f), 7.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFu;
}

// Per-token 8-bit codes (the dequant_swiglu_quant page, section 3.4: dynamic per-row
// quantization, clamp(round(q), -max_val, max_val) with max_val 127 for INT8, 448 for FP8
// E4M3FN and 57344 for FP8 E5M2; round half to even, section 6.1).
//
// INT8: clamp(RNE(q), -127, 127) in the low byte of a dword.  q is clamped first, then
// 1.5 * 2^23 is added: fp32 numbers of that size are spaced 1 apart, so the sum is q rounded
// to the nearest integer, ties to even (1.5 * 2^23 is even), and its bit pattern is that of
// 1.5 * 2^23 (low byte 0) plus the integer, whose two's-complement byte is therefore the low
// byte.  (Clamping before rounding gives the same integer: the bounds are integers.)
__device__ __forceinline__ uint32_t int8_bits(float q) {
  return __float_as_uint(__builtin_amdgcn_fmed3f(q, -127.0f, 127.0f) + 12582912.0f);
}
__device__ __forceinline__ uint32_t int8_code(float q) { return int8_bits(q) & 0xFFu; }

// Low bytes of a, b -> bytes 0, 1 (bytes 2, 3 zero).
__device__ __forceinline__ uint32_t low_bytes2(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
}

// FP8 (OCP encodings: E4M3FN = sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities; E5M2 = sign, 5 exponent bits with bias 15, 2 mantissa bits): the value nearest
// clamp(q, -max_val, max_val), a tie to the even code, with q's sign bit.  gfx950's packed
// conversions to the OCP formats round to nearest even; with the clamp applied first they
// never overflow (the GPU tests check the codes bit-exact at every FP8 value, every tie and
// its neighbours, both signs).
// Two codes per call; `old` keeps the other word (HI = false: codes in bytes 0, 1; HI =
// true: bytes 2, 3).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2(float a, float b, uint32_t old) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f), cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, static_cast<int>(old), HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t e5m2x2(float a, float b, uint32_t old) {
  const float ca = __builtin_amdgcn_fmed3f(a, -57344.0f, 57344.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -57344.0f, 57344.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, static_cast<int>(old), HI));
}
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) { return e4m3x2<false>(a, b, 0u); }
__device__ __forceinline__ uint32_t e5m2x2(float a, float b) { return e5m2x2<false>(a, b, 0u); }

// Two bytes of a per-token 8-bit mode (byte 0 = a) for q = y / scale (y * (1 / scale) in the
// MFMA kernels).
template <int MODE>
__device__ __forceinline__ uint32_t code8x2(float a, float b) {
  if constexpr (MODE == kPerTokenInt8)
    return low_bytes2(int8_bits(a), int8_bits(b));
  else if constexpr (MODE == kPerTokenE4M3)
    return e4m3x2(a, b);
  else
    return e5m2x2(a, b);
}

// INT8 without the clamp, for q = y * inv where |y * inv| stays below 127.5 (the scale is
// max|y| / (127 / clipRatio), so this holds while 127 / clipRatio, with the few ulp the scale
// and its reciprocal add, stays below 127.5): one fused multiply-add rounds y * inv to the
// nearest integer as int8_bits does (one rounding of the exact product instead of rounding
// the product to fp32 first; either integer is within the product's rounding interval).
__device__ __forceinline__ uint32_t int8_bits_fma(float y, float inv) {
  return __float_as_uint(__builtin_fmaf(y, inv, 12582912.0f));
}

// Four bytes (byte 0 = a).
template <int MODE>
__device__ __forceinline__ uint32_t code8x4(float a, float b, float c, float d) {
  if constexpr (MODE == kPerTokenInt8) {
    const uint32_t lo = low_bytes2(int8_bits(a), int8_bits(b)), hi = low_bytes2(int8_bits(c), int8_bits(d));
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);  // [lo.b0, lo.b1, hi.b0, hi.b1]
  } else if constexpr (MODE == kPerTokenE4M3) {
    return e4m3x2<true>(c, d, e4m3x2<false>(a, b, 0u));
  } else {
    return e5m2x2<true>(c, d, e5m2x2<false>(a, b, 0u));
  }
}

// The same four codes of y0..y3 * inv; CLAMP = false: the INT8 clamp is known not to bite.
template <int MODE, bool CLAMP>
__device__ __forceinline__ uint32_t code8x4(float y0, float y1, float y2, float y3, float inv) {
  if constexpr (MODE == kPerTokenInt8 && !CLAMP) {
    const uint32_t lo = low_bytes2(int8_bits_fma(y0, inv), int8_bits_fma(y1, inv));
    const uint32_t hi = low_bytes2(int8_bits_fma(y2, inv), int8_bits_fma(y3, inv));
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  } else {
    return code8x4<MODE>(y0 * inv, y1 * inv, y2 * inv, y3 * inv);
  }
}

// E2M1 code (sign << 3 | magnitude index) by counting the decision points passed.
// At a decision point the even index wins: the points in front of an even index
// (0.75, 1.75, 3.5) are passed at equality, the others (0.25, 1.25, 2.5, 5) only when
// exceeded.  Above 6 the index stays 7 (saturation).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t i = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return ((__float_as_uint(v) >> 28) & 0x8u) | i;
}

// e8m0 code of a group's max |y|.
//  V1 (dmax == 0): floor(log2 amax) - 2 + 127 in [0, 254] -- for a normal amax that is
//    its biased exponent field minus 2; a subnormal or zero amax gives 0.
//  V2: S = amax / dmax (IEEE fp32); biased exponent E of S, plus one when S is normal,
//    E < 254 and S's mantissa is non-zero.
__device__ __forceinline__ uint32_t e8m0_code(float amax, float dmax) {
  if (dmax == 0.0f) {
    const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu) - 2;
    return static_cast<uint32_t>(e < 0 ? 0 : (e > 254 ? 254 : e));
  }
  const uint32_t s = __float_as_uint(amax / dmax);
  uint32_t E = (s >> 23) & 0xFFu;
  if (E >= 1u && E < 254u && (s & 0x7FFFFFu) != 0u) E += 1u;
  return E;
}

// The e8m0 rule as a compile-time variant, so a kernel's epilogue has no branch on it:
//   kE8V1     dmax == 0: the V1 rule;
//   kE8V2Pow2 dmax a power of two, dinv = 1/dmax: amax * dinv is exactly the IEEE
//             quotient amax / dmax, so the division is skipped;
//   kE8V2Div  any other dmax: the quotient by division.
enum E8Variant : int { kE8V1 = 0, kE8V2Pow2 = 1, kE8V2Div = 2 };

template <int SV>
__device__ __forceinline__ uint32_t e8m0_code_v(float amax, float dmax, float dinv) {
  if constexpr (SV == kE8V1) {
    const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu) - 2;
    return static_cast<uint32_t>(e < 0 ? 0 : (e > 254 ? 254 : e));
  } else {
    const uint32_t s = __float_as_uint(SV == kE8V2Pow2 ? amax * dinv : amax / dmax);
    uint32_t E = (s >> 23) & 0xFFu;
    if (E >= 1u && E < 254u && (s & 0x7FFFFFu) != 0u) E += 1u;
    return E;
  }
}

// y * 2^(127 - code): exact (v_ldexp), the reciprocal of the e8m0 scale.
__device__ __forceinline__ float apply_e8m0(float y, uint32_t code) {
  return __builtin_amdgcn_ldexpf(y, 127 - static_cast<int>(code));
}

}  // namespace fq
