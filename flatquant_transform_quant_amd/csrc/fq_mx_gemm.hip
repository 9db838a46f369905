// MXFP4 consumer GEMM: C[T, O] = A[T, H] . W[O, H]^T with both operands in the quantizer's
// per-group format -- E2M1 codes (two per byte, low nibble first) and one e8m0 power of two
// per 32 consecutive elements of a row ([FQV2] 第3步 pergroup / 第4步; E2M1 magnitudes from
// the ModelOpt page, section 6.1) -- so the quantizer's FLOAT4_E2M1 output [K, M*N] and
// FLOAT8_E8M0 scales feed it directly as A (T = K tokens, H = M*N).
//
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in fp4 takes the block scales
// as they are stored: lane l of an A fragment holds row l%16, k = 32*(l/16) .. +31 (16 bytes of
// codes) and that 32-block's e8m0 byte in its scale operand; B the same with columns; the
// 16x16 fp32 result is laid out as for the other 16x16 products (lane l: column l%16, rows
// 4*(l/16) .. +3).  Products are accumulated in fp32 (any order: the result lies within
// gamma(H) * sum|terms| of the exact sum) and rounded once to C's dtype.
//
// Tiling: a workgroup of 4 waves (2 x 2) computes a 128 x 128 tile of C, a wave 64 x 64 as
// 4 x 4 products per 128-deep k-step.  Fragments come straight from memory (a wave's rows
// are shared with one other wave of the workgroup and with the other workgroups of its
// row band, served by L1/L2), through buffer resources bounded to the operand, so rows past
// T or O read zeros; the next k-step's fragments are loaded while the current one's products
// run.
#include <hip/hip_runtime.h>

#include "fq_codec.h"
#include "fq_internal.h"

namespace fq {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kGemmThreads = 256;
constexpr int kTile = 128;  // C rows and columns per workgroup
constexpr int kWT = 4;      // 16 x 16 products per wave and dimension (64 / 16)
constexpr int32_t kBufWord3 = 0x00020000;

struct Frags {
  u32x4_t a[kWT], b[kWT];
  uint32_t sa[kWT], sb[kWT];
};

template <bool F32OUT>
__global__ __launch_bounds__(kGemmThreads) void mx_gemm_kernel(const uint8_t* __restrict__ a,
                                                                const uint8_t* __restrict__ a_e8,
                                                                const uint8_t* __restrict__ w,
                                                                const uint8_t* __restrict__ w_e8, void* __restrict__ c,
                                                                int32_t T, int32_t O, int32_t H, int32_t gs) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, kb = lane >> 4;
  const int t0 = blockIdx.y * kTile + (wv >> 1) * 64, o0 = blockIdx.x * kTile + (wv & 1) * 64;
  const int row_bytes = H / 2;
  const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a), static_cast<int16_t>(0), T * row_bytes, kBufWord3);
  const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w), static_cast<int16_t>(0), O * row_bytes, kBufWord3);
  const auto rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a_e8), static_cast<int16_t>(0), T * gs, kBufWord3);
  const auto rsw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w_e8), static_cast<int16_t>(0), O * gs, kBufWord3);
  // this lane's row of each fragment; rows past T / O read zeros (their offsets lie beyond
  // the resource's size)
  int arow[kWT], wrow[kWT];
#pragma unroll
  for (int i = 0; i < kWT; ++i) {
    arow[i] = t0 + 16 * i + r16;
    wrow[i] = o0 + 16 * i + r16;
  }
  auto load = [&](Frags& f, int ks) {  // k-step ks: elements 128 ks .. +127 of every row
#pragma unroll
    for (int i = 0; i < kWT; ++i) {
      f.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, arow[i] * row_bytes + 64 * ks + 16 * kb, 0, 0);
      f.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, wrow[i] * row_bytes + 64 * ks + 16 * kb, 0, 0);
      f.sa[i] = __builtin_amdgcn_raw_buffer_load_b8(rsa, arow[i] * gs + 4 * ks + kb, 0, 0);
      f.sb[i] = __builtin_amdgcn_raw_buffer_load_b8(rsw, wrow[i] * gs + 4 * ks + kb, 0, 0);
    }
  };

  f32x4_t acc[kWT][kWT];
#pragma unroll
  for (int i = 0; i < kWT; ++i)
#pragma unroll
    for (int j = 0; j < kWT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nks = H / 128;
  Frags cur, nxt;
  load(cur, 0);
  for (int ks = 0; ks < nks; ++ks) {
    load(nxt, ks + 1 < nks ? ks + 1 : ks);  // the last step reloads its own data (no branch)
#pragma unroll
    for (int i = 0; i < kWT; ++i) {
      const i32x8_t av = {static_cast<int>(cur.a[i][0]), static_cast<int>(cur.a[i][1]), static_cast<int>(cur.a[i][2]),
                          static_cast<int>(cur.a[i][3]), 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < kWT; ++j) {
        const i32x8_t bv = {static_cast<int>(cur.b[j][0]), static_cast<int>(cur.b[j][1]), static_cast<int>(cur.b[j][2]),
                            static_cast<int>(cur.b[j][3]), 0, 0, 0, 0};
        // format 4 = fp4 (E2M1) for both operands; scale byte 0 of each lane's scale operand
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0,
                                                                       static_cast<int>(cur.sa[i]), 0,
                                                                       static_cast<int>(cur.sb[j]));
      }
    }
    cur = nxt;
  }

  // lane l holds C[t0 + 16 i + 4 (l/16) + e][o0 + 16 j + l%16]
#pragma unroll
  for (int i = 0; i < kWT; ++i)
#pragma unroll
    for (int j = 0; j < kWT; ++j) {
      const int col = o0 + 16 * j + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = t0 + 16 * i + 4 * kb + e;
        if (row < T && col < O) {
          const int64_t idx = static_cast<int64_t>(row) * O + col;
          if constexpr (F32OUT)
            static_cast<float*>(c)[idx] = acc[i][j][e];
          else
            static_cast<uint16_t*>(c)[idx] = static_cast<uint16_t>(round16x2<kBF16>(acc[i][j][e], 0.0f));
        }
      }
    }
}

}  // namespace

hipError_t launch_mx_gemm(int64_t T, int64_t O, int64_t H, const uint8_t* a, const uint8_t* a_e8, const uint8_t* w,
                          const uint8_t* w_e8, void* c, bool f32_out, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>((O + kTile - 1) / kTile), static_cast<uint32_t>((T + kTile - 1) / kTile));
  const int32_t gs = static_cast<int32_t>(e8m0_bytes_per_slice(H));
  if (f32_out)
    mx_gemm_kernel<true><<<grid, kGemmThreads, 0, s>>>(a, a_e8, w, w_e8, c, static_cast<int32_t>(T),
                                                       static_cast<int32_t>(O), static_cast<int32_t>(H), gs);
  else
    mx_gemm_kernel<false><<<grid, kGemmThreads, 0, s>>>(a, a_e8, w, w_e8, c, static_cast<int32_t>(T),
                                                        static_cast<int32_t>(O), static_cast<int32_t>(H), gs);
  return hipGetLastError();
}

}  // namespace fq
