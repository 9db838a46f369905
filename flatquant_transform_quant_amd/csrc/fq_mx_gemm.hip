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
// 68 KB) are copied from memory into one of two LDS buffers by LDS-DMA loads while the other
// buffer feeds the products, one barrier per stage.  In LDS a row's eight 16-byte chunks are
// stored XOR-permuted (chunk c at position c ^ (r & 7)), which the LDS bank-conflict counter
// reads as zero for the fragment reads.  Operand rows past T or O read zeros through buffer
// resources bounded to the operand.  Workgroups are numbered so that the ones dispatched to
// one XCD (its own L2) cover a contiguous range of tiles, walked in groups of four row bands
// so that concurrently running tiles share operand rows.
#include <hip/hip_runtime.h>

#include "fq_mfma_common.h"

namespace fq {
namespace {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

constexpr int kThreads = 512;               // 8 waves: 2 (t) x 4 (o)
constexpr int kBT = 256, kBO = 256;         // C tile of a workgroup
constexpr int kKT = 256;                    // contraction elements per stage
constexpr int kRowB = kKT / 2;              // 128 code bytes of a row per stage
constexpr int kScB = kKT / 32;              // 8 e8m0 bytes of a row per stage
constexpr int kCodeB = kBT * kRowB;         // 32 KB of codes per operand and stage
constexpr int kScOff = 2 * kCodeB;          // scales: [256 rows of A][256 rows of W] x 8 bytes
constexpr int kStageB = kScOff + (kBT + kBO) * kScB;  // 69632
constexpr int kGroup = 4;                   // row bands walked together

// LDS position of 16-byte chunk c of tile row r is c ^ swz(r)
__device__ __forceinline__ int swz(int r) { return r & 7; }

template <bool F32OUT>
__global__ __launch_bounds__(kThreads) void mx_gemm_kernel(const uint8_t* __restrict__ a,
                                                            const uint8_t* __restrict__ a_e8,
                                                            const uint8_t* __restrict__ w,
                                                            const uint8_t* __restrict__ w_e8, void* __restrict__ c,
                                                            int32_t T, int32_t O, int32_t H, int32_t gs, int32_t nT,
                                                            int32_t nO, int32_t vec_out) {
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
  // waves 0-3 copy the scales of A's rows, waves 4-7 those of W's rows
  const bool sc_a = wv < 4;
  const auto rs = sc_a ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a_e8), static_cast<int16_t>(0), T * gs, kBufferWord3)
                       : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w_e8), static_cast<int16_t>(0), O * gs, kBufferWord3);

  // Copy into a stage with LDS-DMA loads (buffer_load ... lds): lane l of a wave writes the 16
  // (or 4) bytes it loads to LDS at the wave's base + 16 l (4 l).  Codes: load j of wave wv
  // fills tile rows 64 j + 8 wv .. +7, lane l row 64 j + tid/8 at position l%8, so it loads
  // chunk (l%8) ^ swz(row) of that row (swz(64 j + r) == swz(r)).  Scales: the stage's 512
  // rows x 8 bytes (A's rows, then W's) in 16 runs of 32 rows; wave wv fills runs 2 wv and
  // 2 wv + 1, lane l row 32 q + l/2, dword l%2.
  const int crow = tid >> 3, cchunk = (tid & 7) ^ swz(crow);
  int aoff[4], woff[4], soff[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    aoff[j] = (t0 + 64 * j + crow) * row_bytes + 16 * cchunk;
    woff[j] = (o0 + 64 * j + crow) * row_bytes + 16 * cchunk;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) soff[q] = ((sc_a ? t0 : o0) + ((32 * (2 * wv + q) + (lane >> 1)) & 255)) * gs + 4 * (lane & 1);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto dma = [&](uint8_t* st, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(st + (64 * j + 8 * wv) * kRowB), 16, aoff[j] + kRowB * kt, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(st + kCodeB + (64 * j + 8 * wv) * kRowB), 16,
                                               woff[j] + kRowB * kt, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(st + kScOff + 256 * (2 * wv + q)), 4, soff[q] + kScB * kt, 0, 0, 0);
  };
  // every load of this wave has landed in LDS; the barrier after it publishes the stage
  auto dma_wait = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // products: this wave's rows of A are 128 wm + 16 i + lane%16, of W 64 wn + 16 j + lane%16
  const int wm = wv >> 2, wn = wv & 3;
  const int r16 = lane & 15, kb = lane >> 4, sw = swz(r16);
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One stage's products: NH halves of 128, each 8 A fragments x 4 W fragments.  The reads
  // run one fragment ahead of the products: A fragment i + 1 (or, after the last one, the
  // next half's W fragments and first A fragment) is read while the products of fragment i run.
  // Per-lane LDS offsets of this wave's fragments in a stage (half h: code chunk 4 h + kb, so
  // the XOR-permuted position of half 1 is that of half 0 ^ 4); fragment i / j adds a
  // constant (2048 i for codes, 128 i for scales).  Kept opaque so that the compiler holds
  // these few offsets instead of one address per stage, half and fragment.
  int oa[2], ow[2], osa, osw;
  oa[0] = (128 * wm + r16) * kRowB + 16 * (kb ^ sw);
  oa[1] = oa[0] ^ 64;
  ow[0] = kCodeB + (64 * wn + r16) * kRowB + 16 * (kb ^ sw);
  ow[1] = ow[0] ^ 64;
  osa = kScOff + kScB * (128 * wm + r16) + kb;
  osw = kScOff + kScB * (kBT + 64 * wn + r16) + kb;
  asm volatile("" : "+v"(oa[0]), "+v"(oa[1]), "+v"(ow[0]), "+v"(ow[1]), "+v"(osa), "+v"(osw));
  auto read_a = [&](const uint8_t* st, int h, int i, u32x4_t& f, int& sc) __attribute__((always_inline)) {
    f = *reinterpret_cast<const u32x4_t*>(st + oa[h] + 16 * kRowB * i);
    sc = st[osa + 16 * kScB * i + 4 * h];
  };
  auto read_w = [&](const uint8_t* st, int h, u32x4_t (&f)[4], int (&sc)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = *reinterpret_cast<const u32x4_t*>(st + ow[h] + 16 * kRowB * j);
      sc[j] = st[osw + 16 * kScB * j + 4 * h];
    }
  };
  // One stage's products: one or two halves of 128, each 8 A fragments x 4 W fragments.  The
  // reads run one fragment ahead of the products: A fragment i + 1 (after the last one, the
  // next half's W fragments and first A fragment) is read while the products of i run.
  auto half = [&](const uint8_t* st, int h, u32x4_t (&wf)[4], int (&wsc)[4], u32x4_t& af, int& asc,
                  u32x4_t (&wfn)[4], int (&wscn)[4], bool next) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t afn;
      int ascn = 0;
      if (i < 7) {
        read_a(st, h, i + 1, afn, ascn);
      } else if (next) {
        read_w(st, h + 1, wfn, wscn);
        read_a(st, h + 1, 0, afn, ascn);
      }
      __builtin_amdgcn_sched_barrier(0);
      const i32x8_t bv = {static_cast<int>(af[0]), static_cast<int>(af[1]), static_cast<int>(af[2]),
                          static_cast<int>(af[3]), 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x8_t av = {static_cast<int>(wf[j][0]), static_cast<int>(wf[j][1]), static_cast<int>(wf[j][2]),
                            static_cast<int>(wf[j][3]), 0, 0, 0, 0};
        // format 4 = fp4 (E2M1) for both operands; scale byte 0 of each lane's scale operand
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0, wsc[j], 0, asc);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i < 7 || next) {
        af = afn;
        asc = ascn;
      }
    }
  };
  auto stage_products = [&](const uint8_t* st, bool full) __attribute__((always_inline)) {
    u32x4_t w0[4], w1[4], af;
    int s0[4], s1[4], asc;
    read_w(st, 0, w0, s0);
    read_a(st, 0, 0, af, asc);
    half(st, 0, w0, s0, af, asc, w1, s1, full);
    if (full) half(st, 1, w1, s1, af, asc, w0, s0, false);
  };

  const int nkt = (H + kKT - 1) / kKT;  // H is a multiple of 128: the last stage may hold one half
  // stage kt lives in lds0 for even kt, lds1 for odd kt; the loads of stage kt + 1 run while
  // stage kt feeds the products
  dma(lds0, 0);
  dma_wait();
  __syncthreads();
  for (int kt = 0; kt < nkt; kt += 2) {
    if (kt + 1 < nkt) dma(lds1, kt + 1);
    stage_products(lds0, (kt + 1) * kKT <= H);
    dma_wait();
    __syncthreads();
    if (kt + 1 >= nkt) break;
    if (kt + 2 < nkt) dma(lds0, kt + 2);
    stage_products(lds1, (kt + 2) * kKT <= H);
    dma_wait();
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
