// Pipelined whole-workgroup MFMA kernel for 256 x 256 slices with both transforms and
// per-token int4 codes (INT32 / INT4 out).
//
// [FQV2] 拆开算 第1步/第2步 fused with 第3步 (pertoken) for M = N = 256.  The layout is that of
// the 256-class two-sided kernel: one 4-wave workgroup per CU (one wave per SIMD), P1
// staged once in LDS as GEMM2 A fragments (128 KB), wave w owning the 64 output columns
// 64w .. 64w+63 with its strip of P2 as GEMM1 B fragments, x streaming through two 16 KB LDS
// buffers in chunks of 32 rows, two chunks ahead in registers.  What differs is the order
// of the work, which keeps the per-token epilogue off the matrix cores' critical path:
//   * GEMM1 (T_c = RNE(x_c . P2)) runs two chunks ahead of GEMM2 (y += P1[:, c] . T_c), so
//     the rounding of T never waits for the products that feed it;
//   * at a slice boundary the next slice's first two GEMM1 blocks (128 products a wave) run
//     back to back, and the finished slice's int4 codes are formed in between -- VALU work
//     the SIMD issues while its matrix core runs the products;
//   * the wave's P2 strip sits in accumulation registers (MFMA operands may come from them)
//     and y's row tiles 8..15 in ordinary registers, so the max and codes passes read those
//     tiles without register-file moves (tiles 0..7 stay in accumulation registers).
// Per slice and wave the order of the 16 blocks of 16 stages (4 products sharing one A
// fragment) is
//   G2(0) G1(2) G2(1) G1(3) ... G2(5) G1(7) G2(6) G2(7) | reduce max | G1'(0) G1'(1)
// where G1'(c) is chunk c of the wave's next slice and the codes of this slice run during
// G1'(0) and G1'(1).  The slice's max|y| is taken tile by tile during G2(7) and reduced
// across the 4 waves through an LDS buffer that is free at that point.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fq_mfma_common.h"

namespace fq {
namespace {

constexpr int kW = 256;       // M = N
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kNT = 4;        // n-tiles per wave (64 columns)
constexpr int kChunk = 32;    // rows of x per chunk
constexpr int kNChunk = kW / kChunk;
constexpr int kIT = kW / 16;  // 16-row tiles of y
constexpr int kYA = 8;        // y tiles 0 .. kYA-1 in accumulation registers, the rest in ordinary ones

// GEMM1 products with the B operand (P2) in accumulation registers and the accumulator in
// ordinary ones.  Hazards as for the other inline-asm products (fq_mfma_common.h): chains
// on one accumulator forward without wait states, mfma_v_drain() precedes VALU reads.
template <int DT>
__device__ __forceinline__ f32x4_t g1_first(u32x4_t a, u32x4_t b) {
  f32x4_t d;
  if constexpr (DT == kBF16)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  else
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  return d;
}
template <int DT>
__device__ __forceinline__ void g1_acc(f32x4_t& d, u32x4_t a, u32x4_t b) {
  if constexpr (DT == kBF16)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  else
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// Marks the 4 n-tiles of one y tile as read from here on (placed at least four products
// after the tile's last product; the products run in order, so it has written its result).
__device__ __forceinline__ void tile_done_a(f32x4_t (&t)[kNT]) {
  asm("" : "+a"(t[0]), "+a"(t[1]), "+a"(t[2]), "+a"(t[3]));
}
__device__ __forceinline__ void tile_done_v(f32x4_t (&t)[kNT]) {
  asm("" : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]));
}

// Wait states between the writes of the P2 fragments into accumulation registers (VALU
// moves) and the first products that read them: the products are inline asm, so the
// compiler adds none of its own.  Every fragment passes through the statement.
#define FQ_P4(p, i) "+a"(p[i][0]), "+a"(p[i][1]), "+a"(p[i][2]), "+a"(p[i][3])
__device__ __forceinline__ void p2f_fence(u32x4_t (&p)[kW / 32][kNT]) {
  asm volatile("s_nop 7\n\ts_nop 7" : FQ_P4(p, 0), FQ_P4(p, 1), FQ_P4(p, 2), FQ_P4(p, 3), FQ_P4(p, 4), FQ_P4(p, 5),
               FQ_P4(p, 6), FQ_P4(p, 7));
}
#undef FQ_P4

// Redefines y's tiles in accumulation registers after the max pass: the codes pass then
// reads them again instead of keeping the max pass's 128 register copies alive.
#define FQ_T4(y, i) "+a"(y[i][0]), "+a"(y[i][1]), "+a"(y[i][2]), "+a"(y[i][3])
__device__ __forceinline__ void redefine_a_tiles(f32x4_t (&y)[kIT][kNT]) {
  static_assert(kYA == 8, "eight tiles in accumulation registers");
  asm("" : FQ_T4(y, 0), FQ_T4(y, 1), FQ_T4(y, 2), FQ_T4(y, 3), FQ_T4(y, 4), FQ_T4(y, 5), FQ_T4(y, 6), FQ_T4(y, 7));
}
#undef FQ_T4

template <int DT, bool CLAMP>
__global__ __launch_bounds__(kThreads, 1) void mfma_wide2t_kernel(Problem pb, Buffers b) {
  __shared__ u32x4_t frag1[kIT * kNChunk * 64];  // 128 KB: P1 A fragments
  // 2 x 16 KB: x chunks in GEMM1 A-fragment order (the 16-byte slot q = 4ks + g of chunk
  // row r = 16h + c at (2ks + h)*64 + 16g + (c ^ 4g): conflict-free reads and stores)
  __shared__ u32x4_t xs[2][kChunk * 32];
  constexpr int D = 2;                                     // chunks ahead in registers
  constexpr int XR = kChunk * kW * 2 / 16 / kThreads;     // 16-byte pieces per thread per chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t stride = gridDim.x;

  // ---- P1 -> LDS fragments: P1[i, m] -> frag1[(it*8 + ch)*64 + 16*gg + i%16] element t,
  // m = 32ch + (t < 4 ? 4gg + t : 16 + 4gg + t - 4): GEMM1's accumulator rows are GEMM2's
  // k-slots as they stand ----
  {
    uint16_t* f1 = reinterpret_cast<uint16_t*>(frag1);
    for (int base = 0; base < kW * kW / 8; base += kThreads * 4) {
      u32x4_t r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = reinterpret_cast<const u32x4_t*>(b.p1)[base + q * kThreads + tid];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch16 = base + q * kThreads + tid;
        const int i = ch16 >> 5, m0 = (ch16 & 31) * 8;
        const int it = i >> 4, rr = i & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = m0 + e, ch = m >> 5, wv = m & 31;
          const int gg = wv < 16 ? (wv >> 2) : ((wv - 16) >> 2);
          const int t = wv < 16 ? (wv & 3) : 4 + ((wv - 16) & 3);
          f1[((it * kNChunk + ch) * 64 + 16 * gg + rr) * 8 + t] = static_cast<uint16_t>(r[q][e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
  // ---- this wave's P2 strip as GEMM1 B fragments: p2f[ks][nt] element t =
  // P2[32ks + 8g + t, 64w + 4c + nt] (column label c of n-tile nt is column 64w + 4c + nt,
  // so after GEMM2 a lane holds 4 neighbouring columns) ----
  u32x4_t p2f[kW / 32][kNT];
#pragma unroll
  for (int ks = 0; ks < kW / 32; ++ks)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const uint16_t* col = b.p2 + (32 * ks + 8 * g) * kW + 64 * w + 4 * c + nt;
      uint32_t v[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) v[p] = uint32_t(col[(2 * p) * kW]) | (uint32_t(col[(2 * p + 1) * kW]) << 16);
      p2f[ks][nt] = u32x4_t{v[0], v[1], v[2], v[3]};
    }
  p2f_fence(p2f);

  // Chunk j of the workgroup: slice blockIdx.x + (j / 8) * gridDim.x, x rows 32 * (j % 8) ..
  // Load h of wave w covers chunk rows 8h + 4(w/2) .. +3, slots 16(w%2) .. +15: lane l takes
  // row + (l % 4), slot + l / 4.  Bounded buffer loads (zeros past K, no memory access):
  // unconditional, so the compiler's memory-counter waits cover exactly the chunk consumed.
  u32x4_t xr[D][XR];
  const int ld_off = ((4 * (w >> 1) + (lane & 3)) * 32 + 16 * (w & 1) + (lane >> 2)) * 16;
  auto load_chunk = [&](int64_t j, u32x4_t* r) {
    const int64_t slice = blockIdx.x + (j >> 3) * stride;
    const bool in = slice < pb.K;
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(b.x + (in ? slice : 0) * (kW * kW) + (j & 7) * (kChunk * kW)),
        static_cast<int16_t>(0), in ? kChunk * kW * 2 : 0, kBufferWord3);
#pragma unroll
    for (int h = 0; h < XR; ++h) r[h] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ld_off, h * 8 * kW * 2, 0);
  };
  const int sg = (lane >> 2) & 3;
  const int st_even = (4 * (w & 1) + (lane >> 4)) * 2 * 64 + 16 * sg + ((4 * (w >> 1) + (lane & 3)) ^ (4 * sg));
  const int st_odd = st_even ^ 8;
  auto store_chunk = [&](const u32x4_t* r, u32x4_t* dst) {
#pragma unroll
    for (int h = 0; h < XR; ++h) dst[((h & 1) ? st_odd : st_even) + (h >> 1) * 64] = r[h];
  };
  // LDS read bases (opaque: every fragment read is a base plus an immediate offset)
  int rd_base = 16 * g + (c ^ (4 * g));
  int f1_lo = lane, f1_hi = lane + kIT / 2 * kNChunk * 64;
  asm volatile("" : "+v"(rd_base), "+v"(f1_lo), "+v"(f1_hi));

  int64_t s = blockIdx.x;
  if (s >= pb.K) return;

  f32x4_t y[kIT][kNT];
  f32x4_t acc[2 * kNT];
  u32x4_t tb[2][kNT];      // T of the two chunks GEMM1 is ahead by (chunk c in tb[c & 1])
  constexpr int P = 3;     // A fragments are read P stages ahead
  u32x4_t ring[P + 1];

  // ---- fragment reads ----
  // G1 stage k of chunk c: row half k & 1, k-step k >> 1 of the x chunk in xs[c & 1]
  auto read_g1 = [&](int buf, int k, int slot) { ring[slot] = xs[buf][rd_base + (2 * (k >> 1) + (k & 1)) * 64]; };
  // G2 stage t of chunk c: P1 rows 16t .. 16t+15, columns 32c .. 32c+31
  auto read_g2 = [&](int ch, int t, int slot) {
    ring[slot] = t < kIT / 2 ? frag1[f1_lo + (t * kNChunk + ch) * 64] : frag1[f1_hi + ((t - kIT / 2) * kNChunk + ch) * 64];
  };

  // One GEMM1 block for chunk j of the workgroup (chunk cj = j % 8 of its slice).  At its
  // start chunk j + 1 goes from registers to LDS and chunk j + 1 + D is requested into the
  // registers it frees; at its end T is rounded into tb[cj & 1] and a barrier makes chunk
  // j + 1 visible and releases the buffer this block read.  VIS(k) runs VALU work at stage
  // k (the codes pass).  NEXT_G2 / NEXT_CH: the block after this one (its first P fragments
  // are read during this block's last stages, unless it is the GEMM1 block of chunk j + 1,
  // whose chunk is visible only after this block's barrier).
  auto g1_block = [&](int64_t j, auto cjv, auto carry_inv, auto next_g2v, auto next_chv, auto&& vis) {
    constexpr int cj = decltype(cjv)::value;
    constexpr bool carry_in = decltype(carry_inv)::value;
    constexpr bool next_g2 = decltype(next_g2v)::value;
    constexpr int next_ch = decltype(next_chv)::value;
    constexpr int buf = cj & 1;
    if constexpr (!carry_in) {
      read_g1(buf, 0, 0);
      read_g1(buf, 1, 1);
      read_g1(buf, 2, 2);
    }
    store_chunk(xr[(cj + 1) % D], xs[(cj + 1) & 1]);
    load_chunk(j + 1 + D, xr[(cj + 1) % D]);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 16>([&](auto kv) {
      constexpr int k = decltype(kv)::value;
      if constexpr (k + P < 16)
        read_g1(buf, k + P, (k + P) % (P + 1));
      else if constexpr (next_g2)
        read_g2(next_ch, k + P - 16, (k + P) % (P + 1));
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t a = ring[k % (P + 1)];
      constexpr int h = k & 1, ks = k >> 1;
      static_for<0, kNT>([&](auto ntv) {
        constexpr int nt = decltype(ntv)::value;
        if constexpr (ks == 0)
          acc[h * kNT + nt] = g1_first<DT>(a, p2f[ks][nt]);
        else
          g1_acc<DT>(acc[h * kNT + nt], a, p2f[ks][nt]);
        // VALU work issued while this product runs (a few instructions per product: the
        // wave issues in order, so work placed after several products overlaps only the
        // last of them)
        __builtin_amdgcn_sched_barrier(0);
        vis(kv, ntv);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    mfma_v_drain(acc);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
      tb[cj & 1][nt] = u32x4_t{round16x2<DT>(acc[nt][0], acc[nt][1]), round16x2<DT>(acc[nt][2], acc[nt][3]),
                               round16x2<DT>(acc[kNT + nt][0], acc[kNT + nt][1]),
                               round16x2<DT>(acc[kNT + nt][2], acc[kNT + nt][3])};
    vgpr_fence2(tb[cj & 1]);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // One GEMM2 block for chunk CH of the current slice (T in tb[CH & 1]).  FIRST: the
  // slice's first chunk (the products start from 0).  AMAX: the slice's last chunk -- the
  // max of tile t is taken during stage t + 1 (the last tile's after the block).  NEXT_*:
  // as for g1_block (the next block's first fragments are always valid here).
  float amax_run = 0.0f;
  auto g2_block = [&](auto chv, auto next_g1v, auto next_bufv, auto next_chv) {
    constexpr int ch = decltype(chv)::value;
    constexpr bool first = ch == 0;
    constexpr bool amax_pass = ch == kNChunk - 1;
    constexpr bool next_g1 = decltype(next_g1v)::value;
    constexpr int next_buf = decltype(next_bufv)::value;
    constexpr int next_ch = decltype(next_chv)::value;
    static_for<0, 16>([&](auto tv) {
      constexpr int t = decltype(tv)::value;
      if constexpr (t + P < 16)
        read_g2(ch, t + P, (t + P) % (P + 1));
      else if constexpr (next_g1)
        read_g1(next_buf, t + P - 16, (t + P) % (P + 1));
      else
        read_g2(next_ch, t + P - 16, (t + P) % (P + 1));
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t a = ring[t % (P + 1)];
      constexpr int tp = t - 1;  // the tile the previous stage finished
      if constexpr (amax_pass && t >= 1) {
        if constexpr (tp < kYA)
          tile_done_a(y[tp]);
        else
          tile_done_v(y[tp]);
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        if constexpr (t < kYA) {
          if constexpr (first)
            mfma_a_first<DT>(y[t][nt], a, tb[ch & 1][nt]);
          else
            mfma_a_acc<DT>(y[t][nt], a, tb[ch & 1][nt]);
        } else {
          if constexpr (first)
            y[t][nt] = mfma_v_first<DT>(a, tb[ch & 1][nt]);
          else
            mfma_v_acc<DT>(y[t][nt], a, tb[ch & 1][nt]);
        }
        if constexpr (amax_pass && t >= 1) {
          // max|y| of the finished tile, a quarter after each product
          __builtin_amdgcn_sched_barrier(0);
          amax_run = fmaxf(amax_run, fmaxf(fmaxf(__builtin_fabsf(y[tp][nt][0]), __builtin_fabsf(y[tp][nt][1])),
                                           fmaxf(__builtin_fabsf(y[tp][nt][2]), __builtin_fabsf(y[tp][nt][3]))));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (amax_pass) {
      // the last tile: wait states before its VALU reads
      mfma_v_drain(y[kIT - 1]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        amax_run = fmaxf(amax_run, fmaxf(fmaxf(__builtin_fabsf(y[kIT - 1][nt][0]), __builtin_fabsf(y[kIT - 1][nt][1])),
                                         fmaxf(__builtin_fabsf(y[kIT - 1][nt][2]), __builtin_fabsf(y[kIT - 1][nt][3]))));
    }
  };

  // ---- the codes of a finished slice (sp), formed during the next slice's first two GEMM1
  // blocks, two elements per product (128 products, 256 elements a lane) as a software
  // pipeline over product slots m: slot m reads elements 2m+2, 2m+3 from accumulation
  // registers, forms the biased codes of elements 2m, 2m+1 (read in slot m-1), joins the
  // pair formed in slot m-1 into a byte, and stores the code row whose two bytes were both
  // ready before this slot.  The instructions of a slot depend only on earlier slots, so
  // they issue back to back while the slot's product runs.  Element e is y[t][j][i] with
  // t = e / 16 (16-row tile), i = (e / 4) % 4 (row in the lane's 4-row group), j = e % 4
  // (column); a row's two bytes are the pairs j = 0, 1 and j = 2, 3. ----
  int64_t sp = 0;   // the slice whose codes are pending
  float inv = 0.0f;
  float rr[2][2];      // elements read ahead (slot parity)
  uint32_t ff[2][2];   // biased codes formed (slot parity)
  uint32_t ll[4];      // the bytes of pairs q (q % 4)
  constexpr int kEl = kIT * 16;  // elements a lane
  auto yel = [&](auto ev) -> float {
    constexpr int e = decltype(ev)::value;
    return y[e >> 4][e & 3][(e >> 2) & 3];
  };
  auto read_el = [&](auto ev, float& dst) {
    constexpr int e = decltype(ev)::value;
    if constexpr (e < kEl) {
      if constexpr ((e >> 4) < kYA) dst = yel(ev);  // a v_accvgpr_read
    }
  };
  auto code_el = [&](auto ev, float ra) -> uint32_t {
    constexpr int e = decltype(ev)::value;
    return int4_biased<CLAMP>((e >> 4) < kYA ? ra : yel(ev), inv);
  };
  auto encode_slot = [&](auto mv, const auto& rs_codes, int code_off) {
    constexpr int m = decltype(mv)::value;
    // store the row whose pairs (2r, 2r+1) were joined in slots <= m-1: pair 2r+1 = m-2
    if constexpr (m >= 2 && ((m - 2) & 1) == 1) {
      constexpr int q = m - 2, r = q >> 1, t = r >> 2, i = r & 3;
      __builtin_amdgcn_raw_buffer_store_b16(
          static_cast<uint16_t>(unbias(__builtin_amdgcn_perm(ll[q & 3], ll[(q - 1) & 3], 0x0C0C0400u))), rs_codes,
          code_off, (16 * t + i) * (kW / 2), 2 /* non-temporal */);
    }
    // join pair m-1 (its codes were formed in slot m-1)
    if constexpr (m >= 1 && m - 1 < kEl / 2) ll[(m - 1) & 3] = pair_byte(ff[(m - 1) & 1][0], ff[(m - 1) & 1][1]);
    // form the codes of elements 2m, 2m+1 (read in slot m-1)
    if constexpr (2 * m < kEl) {
      ff[m & 1][0] = code_el(std::integral_constant<int, 2 * m>{}, rr[m & 1][0]);
      ff[m & 1][1] = code_el(std::integral_constant<int, 2 * m + 1>{}, rr[m & 1][1]);
    }
    // read elements 2m+2, 2m+3
    read_el(std::integral_constant<int, 2 * m + 2>{}, rr[(m + 1) & 1][0]);
    read_el(std::integral_constant<int, 2 * m + 3>{}, rr[(m + 1) & 1][1]);
  };
  using F = std::false_type;
  using T = std::true_type;
  auto nothing = [](auto, auto) {};
  int64_t j0 = 0;  // chunk index of the current slice's chunk 0

  // prologue: chunk 0 in LDS, chunks 1 .. D in registers (chunk k in xr[k % D])
  load_chunk(0, xr[0]);
  store_chunk(xr[0], xs[0]);
#pragma unroll
  for (int k = 1; k <= D; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(k, xr[k % D]);
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  // the first slice's GEMM1 of chunks 0 and 1 (nothing to encode yet)
  g1_block(j0 + 0, std::integral_constant<int, 0>{}, F{}, F{}, std::integral_constant<int, 0>{}, nothing);
  g1_block(j0 + 1, std::integral_constant<int, 1>{}, F{}, T{}, std::integral_constant<int, 0>{}, nothing);

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  while (true) {
    // ---- slice s: G2(0) G1(2) G2(1) G1(3) ... G1(7) G2(6) G2(7) ----
    g2_block(std::integral_constant<int, 0>{}, T{}, I0{}, I0{});   // next: G1(2), buffer 0
    g1_block(j0 + 2, std::integral_constant<int, 2>{}, T{}, T{}, std::integral_constant<int, 1>{}, nothing);
    g2_block(std::integral_constant<int, 1>{}, T{}, I1{}, I0{});   // next: G1(3), buffer 1
    g1_block(j0 + 3, std::integral_constant<int, 3>{}, T{}, T{}, std::integral_constant<int, 2>{}, nothing);
    g2_block(std::integral_constant<int, 2>{}, T{}, I0{}, I0{});
    g1_block(j0 + 4, std::integral_constant<int, 4>{}, T{}, T{}, std::integral_constant<int, 3>{}, nothing);
    g2_block(std::integral_constant<int, 3>{}, T{}, I1{}, I0{});
    g1_block(j0 + 5, std::integral_constant<int, 5>{}, T{}, T{}, std::integral_constant<int, 4>{}, nothing);
    g2_block(std::integral_constant<int, 4>{}, T{}, I0{}, I0{});
    g1_block(j0 + 6, std::integral_constant<int, 6>{}, T{}, T{}, std::integral_constant<int, 5>{}, nothing);
    g2_block(std::integral_constant<int, 5>{}, T{}, I1{}, I0{});
    g1_block(j0 + 7, std::integral_constant<int, 7>{}, T{}, T{}, std::integral_constant<int, 6>{}, nothing);
    g2_block(std::integral_constant<int, 6>{}, F{}, I0{}, std::integral_constant<int, 7>{});  // next: G2(7)
    amax_run = 0.0f;
    g2_block(std::integral_constant<int, 7>{}, T{}, I0{}, I0{});   // next: G1'(0), buffer 0

    // ---- [FQV2] 第3步 pertoken: max|y| over the slice (4 waves), scale.  The partial maxima
    // pass through xs[1]: its last reader, GEMM1 of chunk 7, is behind the barrier of that
    // block, and its next writer, G1'(0), starts after the second barrier below. ----
    {
      float* red = reinterpret_cast<float*>(xs[1]);
      float amax = wave_max(amax_run);
      red[w] = amax;  // every lane writes the same value
      lds_barrier();
      amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      lds_barrier();
      const float scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(amax / pb.d)));
      // (a scale below 2^-126, whose reciprocal can overflow, is re-encoded by division after
      // this kernel)
      inv = scale > 0.0f ? 1.0f / scale : 0.0f;
      const auto rs_scale = __builtin_amdgcn_make_buffer_rsrc(static_cast<float*>(b.scale) + s, static_cast<int16_t>(0),
                                                              4, kBufferWord3);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(scale), rs_scale, 0, 0, 0);  // every lane, same bytes
    }
    sp = s;
    s += stride;
    j0 += kNChunk;

    // ---- the next slice's GEMM1 of chunks 0 and 1 (zeros past K), with slice sp's codes ----
    {
      redefine_a_tiles(y);
      const auto rs_codes = __builtin_amdgcn_make_buffer_rsrc(b.codes + sp * (kW * kW / 2), static_cast<int16_t>(0),
                                                              kW * kW / 2, kBufferWord3);
      int code_off = 4 * g * (kW / 2) + 32 * w + 2 * c;  // the lane's 4 codes of a row: columns 64w + 4c ..
      asm volatile("" : "+v"(code_off));
      read_el(std::integral_constant<int, 0>{}, rr[0][0]);  // slot 0's elements
      read_el(std::integral_constant<int, 1>{}, rr[0][1]);
      g1_block(j0 + 0, I0{}, T{}, F{}, I0{}, [&](auto kv, auto ntv) {
        encode_slot(std::integral_constant<int, 4 * decltype(kv)::value + decltype(ntv)::value>{}, rs_codes, code_off);
      });
      g1_block(j0 + 1, I1{}, F{}, T{}, I0{}, [&](auto kv, auto ntv) {
        encode_slot(std::integral_constant<int, 64 + 4 * decltype(kv)::value + decltype(ntv)::value>{}, rs_codes,
                    code_off);
      });
      // the pipeline's last two slots (the last pair's byte, the last row's store)
      encode_slot(std::integral_constant<int, kEl / 2>{}, rs_codes, code_off);
      encode_slot(std::integral_constant<int, kEl / 2 + 1>{}, rs_codes, code_off);
    }
    if (s >= pb.K) break;
  }
}

}  // namespace

bool mfma_wide2t_supports(const Problem& pb) {
  return pb.M == kW && pb.N == kW && pb.two_sided && (pb.mode == kPerTokenInt32 || pb.mode == kPerTokenInt4);
}

hipError_t launch_mfma_wide2t(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (!mfma_wide2t_supports(pb)) return hipErrorNotSupported;
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  const int grid = static_cast<int>(pb.K < cus ? pb.K : cus);
  // the int4 clamp can only bite when (7/clipRatio) * (1 + 4 ulp) reaches 7.5
  const bool clamp = pb.d >= 7.4999f;
  if (pb.dtype == kBF16) {
    if (clamp)
      mfma_wide2t_kernel<kBF16, true><<<grid, kThreads, 0, s>>>(pb, b);
    else
      mfma_wide2t_kernel<kBF16, false><<<grid, kThreads, 0, s>>>(pb, b);
  } else {
    if (clamp)
      mfma_wide2t_kernel<kF16, true><<<grid, kThreads, 0, s>>>(pb, b);
    else
      mfma_wide2t_kernel<kF16, false><<<grid, kThreads, 0, s>>>(pb, b);
  }
  return hipGetLastError();
}

}  // namespace fq
