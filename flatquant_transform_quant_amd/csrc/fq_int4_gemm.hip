// int4 consumer GEMM: C[T, O] = sa[t] * sw[o] * sum_h qa[t, h] qw[o, h] with A the
// quantizer's per-token int4 codes ([FQV2] 第3步 pertoken: two's-complement int4, two a
// byte, low nibble first; the INT32 [K, M, N/8] and INT4 [K, M, N] outputs are the same bytes)
// and its fp32 per-token scales, W int4 weights with one fp32 scale per output channel.  The
// symmetric integer format dequantizes as q * scale (the APT-LLM page, section 2.1), so the
// product of two such values is qa qw sa sw.
//
// gfx950 has no int4 matrix instruction: each lane widens its 16-byte chunk of 32 codes to two
// 16-byte int8 operands of v_mfma_i32_16x16x64_i8.  The integer dot product is exact in int32
// (|acc| <= 64 H), so C = fl32(fl32(acc) * fl32(sa * sw)) is one defined value, rounded once
// more to a bf16 C.  The widening only relabels the contraction index, the same way for both
// operands, so it does not change the sums.
//
// Tiling as in the MXFP4 GEMM: a workgroup of 8 waves computes a 256 x 256 tile, each wave
// 128 (t) x 64 (o) as 8 x 4 tiles per 128-deep half-stage (two products each); stages of 256 of
// the contraction (256 rows of A and of W, 128 bytes each, 64 KB) are copied by LDS-DMA loads
// into one of two buffers while the other feeds the products, one barrier per stage; chunk c
// of row r sits at LDS position c ^ (r & 7); W is the first operand, so a lane's four results
// are four consecutive columns of one row; tiles are numbered XCD by XCD in groups of four
// row bands.  Operand rows past T or O read zeros through bounded buffer resources.
#include <hip/hip_runtime.h>

#include "fq_mfma_common.h"

namespace fq {
namespace {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

constexpr int kThreads = 512;               // 8 waves: 2 (t) x 4 (o)
constexpr int kBT = 256, kBO = 256;         // C tile of a workgroup
constexpr int kKT = 256;                    // contraction elements per stage
constexpr int kRowB = kKT / 2;              // 128 code bytes of a row per stage
constexpr int kCodeB = kBT * kRowB;         // 32 KB of codes per operand and stage
constexpr int kStageB = 2 * kCodeB;         // 64 KB
constexpr int kGroup = 4;                   // row bands walked together

__device__ __forceinline__ int swz(int r) { return r & 7; }

// 32 int4 codes (16 bytes) -> two int8 operands.  Dword p holds codes 8p .. 8p+7 (byte j: codes
// 2j, 2j+1); its low nibbles go to one dword, its high nibbles to another, each nibble
// sign-extended to its byte: u | 0xF0 when bit 3 is set ((u & 8) * 0x1E = 0xF0 never carries
// into the next byte).
__device__ __forceinline__ void widen(const u32x4_t raw, i32x4_t& lo, i32x4_t& hi) {
  uint32_t v[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t l = raw[p] & 0x0F0F0F0Fu, h = (raw[p] >> 4) & 0x0F0F0F0Fu;
    l |= (l & 0x08080808u) * 0x1Eu;
    h |= (h & 0x08080808u) * 0x1Eu;
    v[2 * p] = l;
    v[2 * p + 1] = h;
  }
  lo = i32x4_t{static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]), static_cast<int>(v[3])};
  hi = i32x4_t{static_cast<int>(v[4]), static_cast<int>(v[5]), static_cast<int>(v[6]), static_cast<int>(v[7])};
}

// 32 int4 codes -> two operands of their values plus 8 (0 .. 15: the nibble with bit 3 flipped,
// no sign extension), in the byte order of widen().
__device__ __forceinline__ void widen_biased(const u32x4_t raw, i32x4_t& lo, i32x4_t& hi) {
  uint32_t v[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t x = raw[p] ^ 0x88888888u;
    v[2 * p] = x & 0x0F0F0F0Fu;
    v[2 * p + 1] = (x >> 4) & 0x0F0F0F0Fu;
  }
  lo = i32x4_t{static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]), static_cast<int>(v[3])};
  hi = i32x4_t{static_cast<int>(v[4]), static_cast<int>(v[5]), static_cast<int>(v[6]), static_cast<int>(v[7])};
}

template <bool F32OUT>
__global__ __launch_bounds__(kThreads) void int4_gemm_kernel(const uint8_t* __restrict__ a, const float* __restrict__ sa,
                                                              const uint8_t* __restrict__ w, const float* __restrict__ sw,
                                                              void* __restrict__ c, int32_t T, int32_t O, int32_t H,
                                                              int32_t nT, int32_t nO, int32_t vec_out) {
  __shared__ __align__(16) uint8_t lds0[kStageB];  // stages of even / odd index
  __shared__ __align__(16) uint8_t lds1[kStageB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  // this workgroup's tile
  int b = blockIdx.x;
  const int n = nT * nO;
  if ((n & 7) == 0) b = (b & 7) * (n >> 3) + (b >> 3);  // dispatch goes round-robin over the 8 XCDs
  const int grp = b / (kGroup * nO), gfirst = grp * kGroup, gsz = min(nT - gfirst, kGroup);
  const int rem = b - grp * kGroup * nO;
  const int t0 = (gfirst + rem % gsz) * kBT, o0 = (rem / gsz) * kBO;

  const int row_bytes = H >> 1;
  const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a), static_cast<int16_t>(0), T * row_bytes, kBufferWord3);
  const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w), static_cast<int16_t>(0), O * row_bytes, kBufferWord3);

  // Copy into a stage with LDS-DMA loads: load j of wave wv fills tile rows 64 j + 8 wv .. +7,
  // lane l row 64 j + tid/8 at position l%8, so it loads chunk (l%8) ^ swz(row) of that row.
  const int crow = tid >> 3, cchunk = (tid & 7) ^ swz(crow);
  int aoff[4], woff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    aoff[j] = (t0 + 64 * j + crow) * row_bytes + 16 * cchunk;
    woff[j] = (o0 + 64 * j + crow) * row_bytes + 16 * cchunk;
  }
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto dma = [&](uint8_t* st, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(st + (64 * j + 8 * wv) * kRowB), 16, aoff[j] + kRowB * kt, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(st + kCodeB + (64 * j + 8 * wv) * kRowB), 16,
                                               woff[j] + kRowB * kt, 0, 0, 0);
    }
  };
  auto dma_wait = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // products: this wave's rows of A are 128 wm + 16 i + lane%16, of W 64 wn + 16 j + lane%16
  const int wm = wv >> 2, wn = wv & 3;
  const int r16 = lane & 15, kb = lane >> 4, sw8 = swz(r16);
  // A's codes enter the products as qa + 8 (widening without sign extension, half the work of
  // W's), so acc[i][j] sums (qa + 8) qw; wsum[j] accumulates sum_h qw for the same rows o of W
  // (products with an all-ones operand), and the exact sum is acc - 8 wsum.
  i32x4_t acc[8][4], wsum[4];
  const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
  for (int j = 0; j < 4; ++j) wsum[j] = i32x4_t{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4_t{0, 0, 0, 0};

  // one 128-deep half of a stage: the W fragments widened once, then 8 A fragments, each
  // read while the products of the one before run
  auto half_step = [&](const uint8_t* st, int h) __attribute__((always_inline)) {
    const int pos = 16 * ((4 * h + kb) ^ sw8);
    i32x4_t wlo[4], whi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      widen(*reinterpret_cast<const u32x4_t*>(st + kCodeB + (64 * wn + 16 * j + r16) * kRowB + pos), wlo[j], whi[j]);
      wsum[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo[j], ones, wsum[j], 0, 0, 0);
      wsum[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi[j], ones, wsum[j], 0, 0, 0);
    }
    auto read_a = [&](int i) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4_t*>(st + (128 * wm + 16 * i + r16) * kRowB + pos);
    };
    u32x4_t af = read_a(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t afn = af;
      if (i < 7) afn = read_a(i + 1);
      __builtin_amdgcn_sched_barrier(0);
      i32x4_t alo, ahi;
      widen_biased(af, alo, ahi);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo[j], alo, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi[j], ahi, acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      af = afn;
    }
  };

  const int nkt = (H + kKT - 1) / kKT;  // H is a multiple of 128: the last stage may hold one half
  dma(lds0, 0);
  dma_wait();
  __syncthreads();
  for (int kt = 0; kt < nkt; kt += 2) {
    if (kt + 1 < nkt) dma(lds1, kt + 1);
    half_step(lds0, 0);
    if ((kt + 1) * kKT <= H) half_step(lds0, 1);
    dma_wait();
    __syncthreads();
    if (kt + 1 >= nkt) break;
    if (kt + 2 < nkt) dma(lds0, kt + 2);
    half_step(lds1, 0);
    if ((kt + 2) * kKT <= H) half_step(lds1, 1);
    dma_wait();
    __syncthreads();
  }

  // lane l holds C[t][o .. o+3] with t = t0 + 128 wm + 16 i + l%16, o = o0 + 64 wn + 16 j + 4 (l/16)
  const auto rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sa), static_cast<int16_t>(0), T * 4, kBufferWord3);
  const auto rsw = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sw), static_cast<int16_t>(0), O * 4, kBufferWord3);
  float swv[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      swv[j][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsw, 4 * (o0 + 64 * wn + 16 * j + 4 * kb + e), 0, 0));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + 128 * wm + 16 * i + r16;
    const float sat = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsa, 4 * t, 0, 0));
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = o0 + 64 * wn + 16 * j + 4 * kb;
      const int64_t idx = static_cast<int64_t>(t) * O + o;
      f32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(acc[i][j][e] - 8 * wsum[j][e]) * (sat * swv[j][e]);
      if (vec_out && o + 4 <= O) {
        if constexpr (F32OUT)
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(c) + idx) = v;
        else
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(c) + idx) =
              u32x2_t{round16x2<kBF16>(v[0], v[1]), round16x2<kBF16>(v[2], v[3])};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (o + e >= O) break;
          if constexpr (F32OUT)
            static_cast<float*>(c)[idx + e] = v[e];
          else
            static_cast<uint16_t*>(c)[idx + e] = static_cast<uint16_t>(round16x2<kBF16>(v[e], 0.0f));
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_int4_gemm(int64_t T, int64_t O, int64_t H, const uint8_t* a, const float* sa, const uint8_t* w,
                            const float* sw, void* c, bool f32_out, hipStream_t s) {
  const int32_t nT = static_cast<int32_t>((T + kBT - 1) / kBT), nO = static_cast<int32_t>((O + kBO - 1) / kBO);
  const uintptr_t al = f32_out ? 16 : 8;
  const int32_t vec = (O % 4 == 0) && (reinterpret_cast<uintptr_t>(c) % al == 0);
  const dim3 grid(static_cast<uint32_t>(nT) * static_cast<uint32_t>(nO));
  if (f32_out)
    int4_gemm_kernel<true><<<grid, kThreads, 0, s>>>(a, sa, w, sw, c, static_cast<int32_t>(T), static_cast<int32_t>(O),
                                                      static_cast<int32_t>(H), nT, nO, vec);
  else
    int4_gemm_kernel<false><<<grid, kThreads, 0, s>>>(a, sa, w, sw, c, static_cast<int32_t>(T), static_cast<int32_t>(O),
                                                       static_cast<int32_t>(H), nT, nO, vec);
  return hipGetLastError();
}

}  // namespace fq
