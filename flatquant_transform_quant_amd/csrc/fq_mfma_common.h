// Shared device helpers of the MFMA kernels: operand types, the 16x16x32 MFMA for either
// dtype, wave-level reductions and the packed int4 / E2M1 encoders.
//
// gfx950 v_mfma_f32_16x16x32_{bf16,f16} lane layout (wave64, l = lane):
//   A (16 x 32):  lane l holds row l%16, k = 8*(l/16) .. 8*(l/16)+7
//   B (32 x 16):  lane l holds column l%16, k = 8*(l/16) .. 8*(l/16)+7
//   C (16 x 16):  lane l holds column l%16, rows 4*(l/16) .. 4*(l/16)+3
// The contraction index k may be relabelled freely as long as A and B agree; the
// kernels use that to feed one product's accumulators into the next product without
// moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fq_codec.h"
#include "fq_internal.h"

namespace fq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Word 3 of a raw buffer resource on gfx9-class devices (32-bit data format, no swizzle).
constexpr int32_t kBufferWord3 = 0x00020000;

// Workgroup barrier that orders LDS accesses only.  The workgroup-scope fence of
// __syncthreads also waits for every earlier global store, and since loads and stores
// share one in-order memory counter, for every load issued before them: a barrier after
// a slice's output stores would drain all the input prefetched behind them.  Nothing in
// these kernels passes data between waves through global memory.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// f(std::integral_constant<int, I>{}) for I = B .. E-1, in order (compile-time indices).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// The same product with its accumulator kept in ordinary VGPRs.  A kernel that keeps a
// large accumulator block in the accumulation registers (all 256 of them) needs a second,
// short-lived accumulator elsewhere; the compiler picks one register form for every MFMA
// of a function, so these are written out.  The compiler does not see these as MFMAs, so
// they carry their own hazard handling:
//   * a chain on one accumulator uses the same registers as destination and C operand,
//     which the hardware forwards without wait states;
//   * the operands come from LDS/memory loads (ordered by the compiler's s_waitcnt) or
//     from long-lived registers; mfma_v_begin() adds the wait states a VALU-written
//     operand needs;
//   * mfma_v_drain() must follow the last product before anything reads an accumulator:
//     it holds every accumulator as an operand, so no consumer can be scheduled ahead of
//     its wait states (16, twice what a 4-pass product needs before a VALU read).
// None of the statements is volatile: data dependences alone order them, so the compiler
// stays free to issue LDS reads and other work ahead of and between the products.
template <int DT>
__device__ __forceinline__ f32x4_t mfma_v_first(u32x4_t a, u32x4_t b) {
  f32x4_t d;
  if constexpr (DT == kBF16)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}

template <int DT>
__device__ __forceinline__ void mfma_v_acc(f32x4_t& d, u32x4_t a, u32x4_t b) {
  if constexpr (DT == kBF16)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// Accumulation in the accumulation registers, destination tied to the C operand.  For the
// 16x16 shapes the compiler has no tied form and, with every accumulation register live,
// rotates tiles through spare registers instead of accumulating in place; the tie rules
// that out.  Hazards as above: C is written by other products of the same chain or by
// fenced VALU writes (agpr_fence after zeroing), and every read of the results must
// follow an agpr_fence<16>.
template <int DT>
__device__ __forceinline__ void mfma_a_acc(f32x4_t& d, u32x4_t a, u32x4_t b) {
  if constexpr (DT == kBF16)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

// The first product of such a chain: C = 0, so the block needs no zeroing.
template <int DT>
__device__ __forceinline__ void mfma_a_first(f32x4_t& d, u32x4_t a, u32x4_t b) {
  if constexpr (DT == kBF16)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(d) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(d) : "v"(a), "v"(b));
}

// Marks 4 accumulation-register tiles as read from here on.  Placed after at least four
// further products have been issued behind the tiles' last product (the products run in
// order, so by then it has written its results), this orders VALU reads of the tiles
// without wait states of its own.
__device__ __forceinline__ void agpr_tiles_done(f32x4_t (&t)[4]) {
  asm("" : "+a"(t[0]), "+a"(t[1]), "+a"(t[2]), "+a"(t[3]));
}

// Wait states on 4 ordinary registers (a VALU result about to feed an inline-asm product).
__device__ __forceinline__ void vgpr_fence2(u32x4_t (&v)[4]) {
  asm("s_nop 1" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

#define FQ_A4(y, i) "+a"(y[i][0]), "+a"(y[i][1]), "+a"(y[i][2]), "+a"(y[i][3])
// Wait states held on a 16 x 4 block of accumulation-register tiles: WS = 2 after VALU
// writes that products will read, WS = 16 after products whose results VALU will read.
template <int WS>
__device__ __forceinline__ void agpr_fence(f32x4_t (&y)[16][4]) {
  if constexpr (WS == 2)
    asm("s_nop 1"
        : FQ_A4(y, 0), FQ_A4(y, 1), FQ_A4(y, 2), FQ_A4(y, 3), FQ_A4(y, 4), FQ_A4(y, 5), FQ_A4(y, 6), FQ_A4(y, 7),
          FQ_A4(y, 8), FQ_A4(y, 9), FQ_A4(y, 10), FQ_A4(y, 11), FQ_A4(y, 12), FQ_A4(y, 13), FQ_A4(y, 14), FQ_A4(y, 15));
  else
    asm("s_nop 7\n\ts_nop 7"
        : FQ_A4(y, 0), FQ_A4(y, 1), FQ_A4(y, 2), FQ_A4(y, 3), FQ_A4(y, 4), FQ_A4(y, 5), FQ_A4(y, 6), FQ_A4(y, 7),
          FQ_A4(y, 8), FQ_A4(y, 9), FQ_A4(y, 10), FQ_A4(y, 11), FQ_A4(y, 12), FQ_A4(y, 13), FQ_A4(y, 14), FQ_A4(y, 15));
}
// Ends a pass over the block that produced `r`: every read of that pass happens before
// this point (r passes through it), and copies read before it are dead after it (the block
// is redefined), so a second pass reads the registers again instead of keeping 256 copies.
__device__ __forceinline__ void agpr_pass_end(f32x4_t (&y)[16][4], float& r) {
  asm(""
      : FQ_A4(y, 0), FQ_A4(y, 1), FQ_A4(y, 2), FQ_A4(y, 3), FQ_A4(y, 4), FQ_A4(y, 5), FQ_A4(y, 6), FQ_A4(y, 7),
        FQ_A4(y, 8), FQ_A4(y, 9), FQ_A4(y, 10), FQ_A4(y, 11), FQ_A4(y, 12), FQ_A4(y, 13), FQ_A4(y, 14), FQ_A4(y, 15),
        "+v"(r));
}
#undef FQ_A4

template <int N>
__device__ __forceinline__ void mfma_v_drain(f32x4_t (&d)[N]) {
  static_assert(N == 4 || N == 8, "drain of 4 or 8 accumulators");
  if constexpr (N == 4)
    asm("s_nop 7\n\ts_nop 7" : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
  else
    asm("s_nop 7\n\ts_nop 7"
        : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]), "+v"(d[4]), "+v"(d[5]), "+v"(d[6]), "+v"(d[7]));
}

// DPP lane moves inside 16-lane rows.
enum : int {
  kDppQuadXor1 = 0xB1,    // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,    // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
  kDppRowRor4 = 0x124,    // rotate by 4 / 8 / 12 lanes within the row
  kDppRowRor8 = 0x128,
  kDppRowRor12 = 0x12C,
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Max over aligned groups of SPAN consecutive lanes of a 16-lane row (SPAN = 1, 2, 4, 8, 16).
template <int SPAN>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (SPAN >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  if constexpr (SPAN >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  if constexpr (SPAN >= 8) v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  if constexpr (SPAN >= 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return v;
}

// Max over the whole wave; every lane gets the result.
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

// ---- per-token int4 ------------------------------------------------------------------
// RNE(y * inv) with the round-to-integer done by the fp32 adder: fma(y, inv, 1.5*2^23 + 8)
// rounds the exact product once at unit spacing (ties to even, as 1.5*2^23 + 8 is even),
// leaving code + 8 in the low mantissa bits.  The clamp to [-8, 7] is a clamp of the bit
// pattern as a SIGNED integer (needed only when 7/clipRatio can reach 7.5): over positive
// floats the bit order is the value order, and a sum that went negative (y * inv below
// -12582920, possible when clipRatio is below about 5.6e-7) has its sign bit set, so it
// sorts below every positive pattern and clamps to -8.  Result: low nibble = code + 8,
// bits 4..7 zero, bits above are the constant's (ignored by the packers).
constexpr float kInt4Magic = 12582920.0f;  // 1.5 * 2^23 + 8
constexpr int32_t kInt4MagicLo = 0x4B400000;  // bits of 1.5 * 2^23 (code -8)
constexpr int32_t kInt4MagicHi = 0x4B40000F;  // code +7

template <bool CLAMP>
__device__ __forceinline__ uint32_t int4_biased(float y, float inv) {
  int32_t b = __float_as_int(__builtin_fmaf(y, inv, kInt4Magic));
  if constexpr (CLAMP) b = min(max(b, kInt4MagicLo), kInt4MagicHi);
  return static_cast<uint32_t>(b);
}

// The reciprocal of a per-token scale as a pair (pre, inv) with y * scale^-1 = (y * pre) * inv.
// For a scale below 2^-126 the reciprocal itself can overflow (1 / scale is +inf below
// 2^-128); there both factors are taken with 2^64 moved into y: pre = 2^64 (exact: y is at
// most max|y| = scale * d, far from overflow) and inv = 1 / (scale * 2^64) (scale * 2^64 is
// exact).  A zero scale (all-zero slice) gives inv = 0 and so codes of 0.
struct TokenRecip {
  float pre, inv;
  bool tiny;
};
__device__ __forceinline__ TokenRecip token_recip(float scale) {
  TokenRecip r;
  r.tiny = scale > 0.0f && scale < 0x1p-126f;
  r.pre = r.tiny ? 0x1p64f : 1.0f;
  r.inv = scale > 0.0f ? 1.0f / (scale * r.pre) : 0.0f;
  return r;
}

// Two biased codes -> one byte (low nibble = first), in the low byte of the result.
__device__ __forceinline__ uint32_t pair_byte(uint32_t lo, uint32_t hi) { return lo | (hi << 4); }

// Low bytes of four dwords -> one dword (byte i from d_i).
__device__ __forceinline__ uint32_t gather4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
  const uint32_t a = __builtin_amdgcn_perm(d1, d0, 0x0C0C0400u);  // [d0.b0, d1.b0, 0, 0]
  const uint32_t b = __builtin_amdgcn_perm(d3, d2, 0x0C0C0400u);  // [d2.b0, d3.b0, 0, 0]
  return __builtin_amdgcn_perm(b, a, 0x05040100u);               // [a.b0, a.b1, b.b0, b.b1]
}

// Biased nibbles (code + 8) -> two's complement nibbles.
__device__ __forceinline__ uint32_t unbias(uint32_t packed) { return packed ^ 0x88888888u; }

// ---- per-group E2M1 ----------------------------------------------------------------------
// The e8m0 scale 2^(code - 127) as an fp32 value (code 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_float(uint32_t code) {
  return code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);
}

// v_cvt_scalef32_pk_fp4_f32: two values divided by the power-of-two scale, rounded to
// E2M1 (nearest, ties to even, saturating at 6, sign kept), packed into byte SEL of
// `old` with the first value in the low nibble.  The GPU tests check it bit-exact against
// the encoder of the page's magnitudes at every decision point, the values next to it,
// saturation above 6, and the extreme e8m0 codes 0 and 254.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

}  // namespace fq
