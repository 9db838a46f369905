// MXFP4 consumer GEMM: C[T, O] = A[T, H] . W[O, H]^T with both operands in the quantizer's
// per-group format -- E2M1 codes (two per byte, low nibble first) and one e8m0 power of two
// per 32 consecutive elements of a row ([FQV2] 第3步 pergroup / 第4步; E2M1 magnitudes from
// the ModelOpt page, section 6.1) -- so the quantizer's FLOAT4_E2M1 output [K, M*N] and
// FLOAT8_E8M0 scales feed it directly as A (T = K tokens, H = M*N).
//
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in fp4 takes the block scales
// as they are stored: lane l of the first operand holds row l%16, k = 32*(l/16) .. +31 (16
// bytes of codes) and that 32-block's e8m0 byte in its scale operand; the second operand the
// same with columns; the 16x16 fp32 result is laid out as for the other 16x16 products (lane
// l: column l%16, rows 4*(l/16) .. +3).  W is passed as the first operand and A as the
// second, so a lane's four results are four consecutive columns o of one row t of C.
// Products are accumulated in fp32 (any order: the result lies within gamma(H) * sum|terms|
// of the exact sum) and rounded once to C's dtype.
//
// Tiling: a workgroup of 8 waves computes a 256 x 256 tile of C, each wave 128 (t) x 64 (o)
// as 8 x 4 products per 128-deep half of a stage.  A stage is 256 elements of the contraction:
// the workgroup's 256 rows of A and 256 rows of W (128 code bytes and 8 scale bytes a row,
// 68 KB) are copied from memory into one of two LDS buffers while the other one feeds the
// products, one barrier per stage.  In LDS a row's eight 16-byte chunks are stored XOR-
// permuted (chunk c at position c ^ (r & 7) ^ (r >> 3 & 1)), so that the 16 rows a fragment
// read touches at one chunk land in 16 distinct bank groups.  Operand rows past T or O read
// zeros through buffer resources bounded to the operand.  Workgroups are numbered so that
// the ones dispatched to one XCD (its own L2) cover a contiguous range of tiles, walked in
// groups of four row bands so that concurrently running tiles share operand rows.
#include <hip/hip_runtime.h>

#include "fq_codec.h"
#include "fq_internal.h"

namespace fq {
namespace {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kThreads = 512;               // 8 waves: 2 (t) x 4 (o)
constexpr int kBT = 256, kBO = 256;         // C tile of a workgroup
constexpr int kKT = 256;                    // contraction elements per stage
constexpr int kRowB = kKT / 2;              // 128 code bytes of a row per stage
constexpr int kScB = kKT / 32;              // 8 e8m0 bytes of a row per stage
constexpr int kCodeB = kBT * kRowB;         // 32 KB of codes per operand and stage
constexpr int kScOff = 2 * kCodeB;          // scales: [256 rows of A][256 rows of W] x 8 bytes
constexpr int kStageB = kScOff + (kBT + kBO) * kScB;  // 69632
constexpr int kGroup = 4;                   // row bands walked together
constexpr int32_t kBufWord3 = 0x00020000;

// LDS position of 16-byte chunk c of tile row r is c ^ swz(r)
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <bool F32OUT>
__global__ __launch_bounds__(kThreads) void mx_gemm_kernel(const uint8_t* __restrict__ a,
                                                            const uint8_t* __restrict__ a_e8,
                                                            const uint8_t* __restrict__ w,
                                                            const uint8_t* __restrict__ w_e8, void* __restrict__ c,
                                                            int32_t T, int32_t O, int32_t H, int32_t gs, int32_t nT,
                                                            int32_t nO, int32_t vec_out) {
  __shared__ __align__(16) uint8_t lds[2 * kStageB];
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
  const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a), static_cast<int16_t>(0), T * row_bytes, kBufWord3);
  const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w), static_cast<int16_t>(0), O * row_bytes, kBufWord3);
  // waves 0-3 copy the scales of A's rows, waves 4-7 those of W's rows
  const bool sc_a = wv < 4;
  const auto rs = sc_a ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a_e8), static_cast<int16_t>(0), T * gs, kBufWord3)
                       : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w_e8), static_cast<int16_t>(0), O * gs, kBufWord3);

  // copy mapping: load j takes tile row 64 j + tid/8, LDS position tid%8 (so 8 threads move
  // one row's 128 bytes); swz(64 j + r) == swz(r)
  const int crow = tid >> 3, cpos = tid & 7, cchunk = cpos ^ swz(crow);
  int aoff[4], woff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    aoff[j] = (t0 + 64 * j + crow) * row_bytes + 16 * cchunk;
    woff[j] = (o0 + 64 * j + crow) * row_bytes + 16 * cchunk;
  }
  const int soff = ((sc_a ? t0 : o0) + (tid & 255)) * gs;

  struct Pref {
    u32x4_t a[4], w[4];
    uint32_t s0, s1;
  };
  auto gload = [&](Pref& p, int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p.a[j] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[j] + kRowB * kt, 0, 0);
      p.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff[j] + kRowB * kt, 0, 0);
    }
    p.s0 = __builtin_amdgcn_raw_buffer_load_b32(rs, soff + kScB * kt, 0, 0);
    p.s1 = __builtin_amdgcn_raw_buffer_load_b32(rs, soff + kScB * kt + 4, 0, 0);
  };
  auto lstore = [&](const Pref& p, int s) {
    uint8_t* st = lds + s * kStageB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4_t*>(st + (64 * j + crow) * kRowB + 16 * cpos) = p.a[j];
      *reinterpret_cast<u32x4_t*>(st + kCodeB + (64 * j + crow) * kRowB + 16 * cpos) = p.w[j];
    }
    *reinterpret_cast<u32x2_t*>(st + kScOff + kScB * tid) = u32x2_t{p.s0, p.s1};
  };

  // products: this wave's rows of A are 128 wm + 16 i + lane%16, of W 64 wn + 16 j + lane%16
  const int wm = wv >> 2, wn = wv & 3;
  const int r16 = lane & 15, kb = lane >> 4, sw = swz(r16);
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto half_step = [&](const uint8_t* st, int h) {
    const int pos = 16 * ((4 * h + kb) ^ sw);
    u32x4_t wf[4];
    int wsc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 64 * wn + 16 * j + r16;
      wf[j] = *reinterpret_cast<const u32x4_t*>(st + kCodeB + r * kRowB + pos);
      wsc[j] = st[kScOff + kScB * (kBT + r) + 4 * h + kb];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 128 * wm + 16 * i + r16;
      const u32x4_t af = *reinterpret_cast<const u32x4_t*>(st + r * kRowB + pos);
      const int asc = st[kScOff + kScB * r + 4 * h + kb];
      const i32x8_t bv = {static_cast<int>(af[0]), static_cast<int>(af[1]), static_cast<int>(af[2]),
                          static_cast<int>(af[3]), 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x8_t av = {static_cast<int>(wf[j][0]), static_cast<int>(wf[j][1]), static_cast<int>(wf[j][2]),
                            static_cast<int>(wf[j][3]), 0, 0, 0, 0};
        // format 4 = fp4 (E2M1) for both operands; scale byte 0 of each lane's scale operand
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0, wsc[j], 0, asc);
      }
    }
  };

  const int nkt = (H + kKT - 1) / kKT;  // H is a multiple of 128: the last stage may hold one half
  Pref p;
  gload(p, 0);
  lstore(p, 0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) gload(p, kt + 1);
    const uint8_t* st = lds + (kt & 1) * kStageB;
    half_step(st, 0);
    if ((kt + 1) * kKT <= H) half_step(st, 1);
    if (more) lstore(p, (kt + 1) & 1);
    __syncthreads();
  }

  // lane l holds C[t][o .. o+3] with t = t0 + 128 wm + 16 i + l%16, o = o0 + 64 wn + 16 j + 4 (l/16)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + 128 * wm + 16 * i + r16;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = o0 + 64 * wn + 16 * j + 4 * kb;
      const int64_t idx = static_cast<int64_t>(t) * O + o;
      const f32x4_t v = acc[i][j];
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

hipError_t launch_mx_gemm(int64_t T, int64_t O, int64_t H, const uint8_t* a, const uint8_t* a_e8, const uint8_t* w,
                          const uint8_t* w_e8, void* c, bool f32_out, hipStream_t s) {
  const int32_t nT = static_cast<int32_t>((T + kBT - 1) / kBT), nO = static_cast<int32_t>((O + kBO - 1) / kBO);
  const int32_t gs = static_cast<int32_t>(e8m0_bytes_per_slice(H));
  // four results of a lane are stored at once when every row of C starts suitably aligned
  const uintptr_t al = f32_out ? 16 : 8;
  const int32_t vec = (O % 4 == 0) && (reinterpret_cast<uintptr_t>(c) % al == 0);
  const dim3 grid(static_cast<uint32_t>(nT) * static_cast<uint32_t>(nO));
  if (f32_out)
    mx_gemm_kernel<true><<<grid, kThreads, 0, s>>>(a, a_e8, w, w_e8, c, static_cast<int32_t>(T), static_cast<int32_t>(O),
                                                   static_cast<int32_t>(H), gs, nT, nO, vec);
  else
    mx_gemm_kernel<false><<<grid, kThreads, 0, s>>>(a, a_e8, w, w_e8, c, static_cast<int32_t>(T), static_cast<int32_t>(O),
                                                    static_cast<int32_t>(H), gs, nT, nO, vec);
  return hipGetLastError();
}

}  // namespace fq
