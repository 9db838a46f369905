// Dequantization of the quantizer's outputs: codes + scales -> values in x's dtype, the
// second half of a quantize -> dequantize ("fake-quant") round trip.
//
//   per token:  value = q * quantScale[k]                   (APT-LLM page, section 2.1:
//               q the two's-complement int4 code              the symmetric integer format
//                                                             dequantizes as q * scale)
//   per group:  value = E2M1(code) * 2^(e8m0 - 127)          ([FQV2] 第3步 pergroup: the
//               E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6     scale is a power of two;
//               with the sign bit on top                       ModelOpt page, section 6.1)
//
// The product is formed in IEEE fp32 (per group it is exact or overflows to inf; an e8m0
// byte 0xFF, NaN in the MX encoding, makes its group NaN) and rounded once, to nearest
// even, to the output dtype.  Codes are read in the packed layouts the quantizer writes:
// K * M*N/2 bytes, low nibble = lower flattened index; e8m0 [K, 2*ceil(M*N/64)] bytes.
//
// 8-bit per-token codes (INT8, FP8 E4M3FN, FP8 E5M2; the quantizer writes them from the
// dynamic per-row rule of the dequant_swiglu_quant page, section 3.4): value = q * scale_k in
// IEEE fp32, rounded once to the dtype, q the INT8 integer or the FP8 value (gfx950's exact
// fp8 -> fp32 conversion).  Codes the quantizer never writes (INT8 -128, the FP8 NaN and
// infinity encodings) are outside the domain.
//
// HBM-bound streaming (0.5 byte in, 2 bytes out per element; 1 byte in for 8-bit codes).  Slices whose element
// count is a multiple of 32 take the fast path (8 codes -> 16 bytes per lane and step, each
// instruction of a wave one contiguous run); other shapes take a thread per code byte.
#include <hip/hip_runtime.h>

#include "fq_codec.h"
#include "fq_internal.h"
#include "fq_mfma_common.h"

namespace fq {
namespace {

constexpr int kDqThreads = 256;
// Steps of 64 runs per wave on the fast paths (a run = 8 codes -> 16 output bytes); eight
// measured 4-5% slower than four on the 4096- and 65536-element slices.
constexpr int kDqSteps = 4;

// fp32 value of an E2M1 code (bit 3 the sign, bits 0-2 the magnitude index)
__device__ __forceinline__ float e2m1_float(uint32_t code) {
  const uint32_t c = code & 7u;
  const uint32_t mag = c < 2u ? (c ? 0x3F000000u : 0u)                       // 0, 0.5
                               : (((126u + (c >> 1)) << 23) | ((c & 1u) << 22));  // 1 .. 6
  return __uint_as_float(mag | ((code & 8u) << 28));
}

// value of a code: per token with the slice's fp32 scale, per group with the group's e8m0 byte
template <bool PG>
__device__ __forceinline__ float dq_value(uint32_t code, float scale, uint32_t e8) {
  if constexpr (!PG) {
    const int q = static_cast<int>(code << 28) >> 28;  // sign-extend the nibble
    return static_cast<float>(q) * scale;
  } else {
    const float v = __builtin_amdgcn_ldexpf(e2m1_float(code), static_cast<int>(e8) - 127);
    return e8 == 255u ? __uint_as_float(0x7FC00000u) : v;
  }
}

// Code loads of a wave's four steps, all issued before the first is used: a buffer resource
// that ends at the last run (or covers nothing for a wave past it) turns the loads beyond the
// end into zeros without a memory access, so the wave has its four loads in flight at once
// instead of one round trip per step.  BYTES = bytes of codes per run.
template <int BYTES>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dq_codes_rsrc(const uint8_t* codes, uint32_t wave_run,
                                                                uint32_t runs) {
  const uint32_t left = wave_run < runs ? min(runs - wave_run, 64u * kDqSteps) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes) + static_cast<uint64_t>(wave_run) * BYTES,
                                           static_cast<int16_t>(0), static_cast<int32_t>(left * BYTES), kBufferWord3);
}

// Fast path: a wave covers 2048 consecutive elements of the flattened [K, M*N] tensor in
// four steps; at step w lane l turns the 8 codes of elements base + 512w + 8l .. +7 (one
// dword) into 16 output bytes, so every load and store instruction of the wave touches one
// contiguous run (256 B of codes, 1 KB of values).  An 8-element run never leaves its slice
// or its 32-group (M*N is a multiple of 32).
template <int DT, bool PG>
__global__ __launch_bounds__(kDqThreads) void dequant32_kernel(const uint8_t* __restrict__ codes,
                                                                const void* __restrict__ scale,
                                                                uint16_t* __restrict__ out, uint32_t runs,
                                                                uint32_t runs_per_slice, uint32_t e8_per_slice) {
  const uint32_t lane = threadIdx.x & 63;
  // first 8-element run of the wave (wave-uniform)
  const uint32_t wave_run = __builtin_amdgcn_readfirstlane((blockIdx.x * kDqThreads + (threadIdx.x & ~63u)) * kDqSteps);
  const auto rs = dq_codes_rsrc<4>(codes, wave_run, runs);
  uint32_t c[kDqSteps], e8[kDqSteps] = {};
  float sc[kDqSteps] = {};
#pragma unroll
  for (int w = 0; w < kDqSteps; ++w) c[w] = __builtin_amdgcn_raw_buffer_load_b32(rs, (64 * w + lane) * 4, 0, 0);
#pragma unroll
  for (int w = 0; w < kDqSteps; ++w) {
    // a run past the end reads the last run's scale (its values are not stored)
    const uint32_t r = min(wave_run + 64 * w + lane, runs - 1);
    const uint32_t k = r / runs_per_slice;
    if constexpr (!PG)
      sc[w] = static_cast<const float*>(scale)[k];
    else
      e8[w] = static_cast<const uint8_t*>(scale)[static_cast<uint64_t>(k) * e8_per_slice + (r - k * runs_per_slice) / 4];
  }
#pragma unroll
  for (int w = 0; w < kDqSteps; ++w) {
    const uint32_t r = wave_run + 64 * w + lane;  // this lane's run: elements 8r .. 8r+7
    u32x4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      o[p] = round16x2<DT>(dq_value<PG>((c[w] >> (8 * p)) & 15u, sc[w], e8[w]),
                           dq_value<PG>((c[w] >> (8 * p + 4)) & 15u, sc[w], e8[w]));
    if (r < runs) __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out) + r);  // written once
  }
}

// Any shape: a thread per code byte (elements 2b and 2b+1; M*N is even, so a byte never
// spans two slices).
template <int DT, bool PG>
__global__ __launch_bounds__(kDqThreads) void dequant_bytes_kernel(const uint8_t* __restrict__ codes,
                                                                    const void* __restrict__ scale,
                                                                    uint16_t* __restrict__ out, uint64_t bytes,
                                                                    uint64_t mn, uint32_t e8_per_slice) {
  const uint64_t bi = static_cast<uint64_t>(blockIdx.x) * kDqThreads + threadIdx.x;
  if (bi >= bytes) return;
  const uint64_t e = 2 * bi, k = e / mn, f = e - k * mn;
  const uint32_t byte = codes[bi];
  float sc = 0.0f;
  uint32_t e8 = 0;
  if constexpr (!PG)
    sc = static_cast<const float*>(scale)[k];
  else
    e8 = static_cast<const uint8_t*>(scale)[k * e8_per_slice + f / 32];
  reinterpret_cast<uint32_t*>(out)[bi] = round16x2<DT>(dq_value<PG>(byte & 15u, sc, e8), dq_value<PG>(byte >> 4, sc, e8));
}

// 8-bit codes, fast path: a wave covers 2048 consecutive codes in four steps; at step w lane
// l turns the 8 codes base + 512 w + 8 l .. +7 (8 bytes) into 16 output bytes, so every load
// and store instruction of the wave is one contiguous run (512 B of codes, 1 KB of values).
// An 8-code run never leaves its slice (M*N is a multiple of 8).
// values of bytes 0, 1 (HI = false) or 2, 3 (HI = true) of w
template <int MODE, bool HI>
__device__ __forceinline__ float2 q8x2(uint32_t w) {
  if constexpr (MODE == kPerTokenInt8) {
    const uint32_t h = HI ? w >> 16 : w;
    return float2{static_cast<float>(static_cast<int8_t>(h & 0xFFu)), static_cast<float>(static_cast<int8_t>((h >> 8) & 0xFFu))};
  } else {
    typedef __attribute__((ext_vector_type(2))) float f2;
    const f2 v = MODE == kPerTokenE4M3 ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI)
                                       : __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), HI);
    return float2{v[0], v[1]};
  }
}

template <int DT, int MODE>
__global__ __launch_bounds__(kDqThreads) void dequant8_kernel(const uint8_t* __restrict__ codes,
                                                               const float* __restrict__ scale,
                                                               uint16_t* __restrict__ out, uint32_t runs,
                                                               uint32_t runs_per_slice) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
  const uint32_t lane = threadIdx.x & 63;
  // first 8-code run of the wave (wave-uniform); the four steps' loads go out together
  const uint32_t wave_run = __builtin_amdgcn_readfirstlane((blockIdx.x * kDqThreads + (threadIdx.x & ~63u)) * kDqSteps);
  const auto rs = dq_codes_rsrc<8>(codes, wave_run, runs);
  u32x2_t c[kDqSteps];
  float sc[kDqSteps];
#pragma unroll
  for (int w = 0; w < kDqSteps; ++w) c[w] = __builtin_amdgcn_raw_buffer_load_b64(rs, (64 * w + lane) * 8, 0, 0);
#pragma unroll
  for (int w = 0; w < kDqSteps; ++w) sc[w] = scale[min(wave_run + 64 * w + lane, runs - 1) / runs_per_slice];
#pragma unroll
  for (int w = 0; w < kDqSteps; ++w) {
    const uint32_t r = wave_run + 64 * w + lane;  // this lane's run: codes 8r .. 8r+7
    const float2 q0 = q8x2<MODE, false>(c[w][0]), q1 = q8x2<MODE, true>(c[w][0]);
    const float2 q2 = q8x2<MODE, false>(c[w][1]), q3 = q8x2<MODE, true>(c[w][1]);
    const float s = sc[w];
    if (r < runs)
      __builtin_nontemporal_store(u32x4_t{round16x2<DT>(q0.x * s, q0.y * s), round16x2<DT>(q1.x * s, q1.y * s),
                                          round16x2<DT>(q2.x * s, q2.y * s), round16x2<DT>(q3.x * s, q3.y * s)},
                                  reinterpret_cast<u32x4_t*>(out) + r);  // written once
  }
}

// 8-bit codes, any shape: a thread per code.
template <int DT, int MODE>
__global__ __launch_bounds__(kDqThreads) void dequant8_each_kernel(const uint8_t* __restrict__ codes,
                                                                    const float* __restrict__ scale,
                                                                    uint16_t* __restrict__ out, uint64_t count,
                                                                    uint64_t mn) {
  const uint64_t e = static_cast<uint64_t>(blockIdx.x) * kDqThreads + threadIdx.x;
  if (e >= count) return;
  float v = q8x2<MODE, false>(codes[e]).x * scale[e / mn];
  // the fp32 product is rounded to the dtype on its own: without the register barrier the
  // compiler fuses product and conversion into one mixed-precision FMA with a +0 addend,
  // which rounds once (not twice) and turns a -0 product into +0
  asm volatile("" : "+v"(v));
  out[e] = static_cast<uint16_t>(round16x2<DT>(v, 0.0f));
}

template <int DT, int MODE>
hipError_t launch_dq8(int64_t K, int64_t MN, const uint8_t* codes, const float* scale, uint16_t* out, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(codes) % 8 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0);
  if (MN % 8 == 0 && aligned) {
    const uint64_t runs = static_cast<uint64_t>(K) * (MN / 8);  // < 2^32
    const uint64_t per_block = kDqSteps * kDqThreads;
    const uint32_t grid = static_cast<uint32_t>((runs + per_block - 1) / per_block);
    dequant8_kernel<DT, MODE><<<grid, kDqThreads, 0, s>>>(codes, scale, out, static_cast<uint32_t>(runs),
                                                          static_cast<uint32_t>(MN / 8));
  } else {
    const uint64_t count = static_cast<uint64_t>(K) * MN;
    const uint64_t grid = (count + kDqThreads - 1) / kDqThreads;
    dequant8_each_kernel<DT, MODE><<<static_cast<uint32_t>(grid), kDqThreads, 0, s>>>(codes, scale, out, count,
                                                                                    static_cast<uint64_t>(MN));
  }
  return hipGetLastError();
}

template <int DT, bool PG>
hipError_t launch_dq(int64_t K, int64_t MN, const uint8_t* codes, const void* scale, uint16_t* out,
                     hipStream_t s) {
  const uint32_t e8_per_slice = static_cast<uint32_t>(e8m0_bytes_per_slice(MN));
  const bool aligned = (reinterpret_cast<uintptr_t>(codes) % 16 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0);
  if (MN % 32 == 0 && aligned) {
    const uint64_t runs = static_cast<uint64_t>(K) * (MN / 8);  // <= 2^31
    const uint64_t per_block = kDqSteps * kDqThreads;                   // runs a workgroup covers
    const uint32_t grid = static_cast<uint32_t>((runs + per_block - 1) / per_block);
    dequant32_kernel<DT, PG><<<grid, kDqThreads, 0, s>>>(codes, scale, out, static_cast<uint32_t>(runs),
                                                          static_cast<uint32_t>(MN / 8), e8_per_slice);
  } else {
    const uint64_t bytes = static_cast<uint64_t>(K) * (MN / 2);
    const uint64_t grid = (bytes + kDqThreads - 1) / kDqThreads;
    dequant_bytes_kernel<DT, PG><<<static_cast<uint32_t>(grid), kDqThreads, 0, s>>>(
        codes, scale, out, bytes, static_cast<uint64_t>(MN), e8_per_slice);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant8(int32_t dtype, int32_t mode, int64_t K, int64_t M, int64_t N, const uint8_t* codes,
                           const float* scale, uint16_t* out, hipStream_t s) {
  const int64_t MN = M * N;
  if (dtype == kBF16) {
    if (mode == kPerTokenInt8) return launch_dq8<kBF16, kPerTokenInt8>(K, MN, codes, scale, out, s);
    if (mode == kPerTokenE4M3) return launch_dq8<kBF16, kPerTokenE4M3>(K, MN, codes, scale, out, s);
    return launch_dq8<kBF16, kPerTokenE5M2>(K, MN, codes, scale, out, s);
  }
  if (mode == kPerTokenInt8) return launch_dq8<kF16, kPerTokenInt8>(K, MN, codes, scale, out, s);
  if (mode == kPerTokenE4M3) return launch_dq8<kF16, kPerTokenE4M3>(K, MN, codes, scale, out, s);
  return launch_dq8<kF16, kPerTokenE5M2>(K, MN, codes, scale, out, s);
}

hipError_t launch_dequant(int32_t dtype, bool per_group, int64_t K, int64_t M, int64_t N, const uint8_t* codes,
                          const void* scale, uint16_t* out, hipStream_t s) {
  const int64_t MN = M * N;
  if (dtype == kBF16)
    return per_group ? launch_dq<kBF16, true>(K, MN, codes, scale, out, s)
                     : launch_dq<kBF16, false>(K, MN, codes, scale, out, s);
  return per_group ? launch_dq<kF16, true>(K, MN, codes, scale, out, s)
                   : launch_dq<kF16, false>(K, MN, codes, scale, out, s);
}

}  // namespace fq
