// Pipelined whole-workgroup MFMA kernel for 256 x 256 slices with both transforms and
// per-token int4 codes (INT32 / INT4 out).
//
// [FQV2] 拆开算 第1步/第2步 fused with 第3步 (pertoken) for M = N = 256.  The layout is that of
// the 256-class two-sided kernel: one 4-wave workgroup per CU (one wave per SIMD), P1
// staged once in LDS as GEMM2 A fragments (128 KB), wave w owning the 64 output columns
// 64w .. 64w+63 with its strip of P2 as GEMM1 B fragments, x streaming through two 16 KB LDS
// buffers in chunks of 32 rows, two chunks ahead in registers.  What differs is the order
// of the work, which spreads the per-token epilogue over as many products as the registers
// allow.  With one wave per SIMD a wave issues its own VALU work between its products, and a
// product leaves room for about two VALU instructions or one accumulation-register read
// before further ones delay the next product; so the epilogue is cut into a few instructions
// after each product, over every product the data dependences leave:
//   * GEMM1 (T_c = RNE(x_c . P2)) runs two chunks ahead of GEMM2 (y += P1[:, c] . T_c); the
//     GEMM2 block after a GEMM1 block rounds that block's T (two conversions a product) and
//     passes its barrier mid-block, and a GEMM1 block moves its next x chunk from registers
//     to LDS a quarter at a time;
//   * GEMM2 of chunks 6 and 7 is one block, tile by tile, so that max|y| is taken as tiles
//     become final (at most two accumulation-register reads a product);
//   * a slice's int4 codes are formed during the next slice's first two GEMM1 blocks and
//     its first GEMM2 block, each tile before the product that overwrites it;
//   * the wave's P2 strip sits in accumulation registers (MFMA operands may come from them)
//     and y's row tiles 8..15 in ordinary registers, so the max and codes passes read those
//     tiles without register-file moves (tiles 0..7 stay in accumulation registers).
// Per slice and wave the order of the blocks of 16 stages (4 products sharing one A
// fragment) is
//   G2(0) G1(2) G2(1) G1(3) ... G2(5) G1(7) G2(6+7) | reduce max | G1'(0) G1'(1)
// where G1'(c) is chunk c of the wave's next slice; the codes of this slice run during
// G1'(0), G1'(1) and the next slice's G2(0).  The slice's max|y| is reduced across the 4
// waves through an LDS buffer that is free at that point.
//
// Slices are handed out at run time: a counter in device memory (zeroed before the launch)
// gives each workgroup its next slice, one atomic increment per slice, taken two slices ahead
// (the next slice's first x chunk is requested halfway through the current one) and passed
// to the workgroup's waves with the max reduction.  The XCDs of the device run at clocks a
// few percent apart under this load, and with a fixed share of the slices per workgroup
// the launch ended with the slowest (every workgroup takes the same cycle count).
#include <hip/hip_runtime.h>

#include <atomic>

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
constexpr int kEl = kIT * 16;  // y elements a lane
constexpr int kBarStage = 8;   // the stage of a GEMM2 block that passes the barrier of the GEMM1 block before it

// A ticket of the slice counter: the counter's value before adding one.  An increment that
// wraps at 2^32 - 1 (the same as adding one for every reachable value) rather than an add: the
// compiler rewrites a single-address add into a wave-combined form that reads the reply
// straight away, with a wait for every memory access in flight, where this form leaves the
// wait at the reply's first use.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* ctr) {
  return __builtin_amdgcn_atomic_inc32(ctr, 0xFFFFFFFFu, __ATOMIC_RELAXED, "agent");
}

// GEMM2 of chunks 6 and 7 as one 32-stage block: stage s -> (tile, chunk).  Chunk 7 starts
// at stage 3 (its T is rounded during stages 1 and 2) and the accumulation-register tiles
// 0 .. 7 come first, so that their max pass (register-file reads, the costly part) can
// stream over most of the block.
constexpr int kM67[32][2] = {{0, 6},  {1, 6},  {2, 6},  {0, 7},  {3, 6},  {1, 7},  {4, 6},  {2, 7},
                             {5, 6},  {3, 7},  {6, 6},  {4, 7},  {7, 6},  {5, 7},  {6, 7},  {7, 7},
                             {8, 6},  {9, 6},  {8, 7},  {10, 6}, {9, 7},  {11, 6}, {10, 7}, {12, 6},
                             {11, 7}, {13, 6}, {12, 7}, {14, 6}, {13, 7}, {15, 6}, {14, 7}, {15, 7}};
constexpr int m67_tile(int s) { return kM67[s][0]; }
constexpr int m67_ch(int s) { return kM67[s][1]; }
constexpr int m67_done(int t) {
  for (int s = 0; s < 32; ++s)
    if (kM67[s][0] == t && kM67[s][1] == 7) return s;
  return -1;
}
// max pass of the merged block, counted in products (4 per stage); a tile is read from two
// stages after its last product, and the merged block passes its barrier at stage kM67Bar.
// Accumulation-register tiles: read r (0 .. 127; tile r / 16, element r % 16) after product
// amax_rd(r), the max of pair k after product amax_rd(2k+1) + 1 (at most two register-file
// reads a product).  Ordinary-register tiles 8 .. 13: pair j (0 .. 7) after product
// 4 * (m67_done(t) + 2) + j; tiles 14 and 15 after the block.
constexpr int kM67Bar = 4;
constexpr int amax_rd(int r) { return 4 * (kM67Bar + 1) + (r * 104) / 127; }
constexpr bool amax_ok() {
  for (int r = 0; r < 128; ++r) {
    if (amax_rd(r) < 4 * (m67_done(r / 16) + 2)) return false;  // read before the tile is final
    if (r > 1 && amax_rd(r) == amax_rd(r - 2)) return false;    // at most two reads a product
  }
  return amax_rd(127) + 1 < 128 && 4 * (m67_done(13) + 2) + 7 < 128 && m67_done(14) + 2 > 31;
}
static_assert(amax_ok(), "max pass schedule of the merged block");
// lookups by product: the first read after it (-1: none) and how many; the pair whose max
// follows it (-1: none); the ordinary-register tile whose pair it takes (-1: none); the tile
// fenced before stage s (-1: none)
constexpr int amax_rd_first(int pos) {
  for (int r = 0; r < 128; ++r)
    if (amax_rd(r) == pos) return r;
  return -1;
}
constexpr int amax_rd_count(int pos) {
  int n = 0;
  for (int r = 0; r < 128; ++r) n += amax_rd(r) == pos;
  return n;
}
constexpr int amax_pair_at(int pos) {
  for (int k = 0; k < 64; ++k)
    if (amax_rd(2 * k + 1) + 1 == pos) return k;
  return -1;
}
constexpr int amax_vtile_at(int pos) {
  for (int t = 8; t < 14; ++t)
    if (pos >= 4 * (m67_done(t) + 2) && pos < 4 * (m67_done(t) + 2) + 8) return t;
  return -1;
}
constexpr int m67_fence_at(int s) {
  for (int t = 0; t < 14; ++t)
    if (m67_done(t) + 2 == s) return t;
  return -1;
}

// Code step m (0 .. kEl/2 + 1) runs after product enc_pos(m) of the 192 products of the next
// slice's G1(0), G1(1) and G2(0); enc_step_at inverts it (-1: no step at that product).
constexpr int kEncOff = 8;
constexpr int enc_pos(int m) { return kEncOff + (27 * m) / 20; }
constexpr int enc_step_at(int pos) {
  if (pos < kEncOff) return -1;
  const int m = ((pos - kEncOff) * 20 + 26) / 27;
  return (m <= kEl / 2 + 1 && enc_pos(m) == pos) ? m : -1;
}
// the last read of tile t (its element 16t+15: by step 8t+6 in accumulation registers, at
// step 8t+7 in ordinary ones) precedes stage t of G2(0), product 128 + 4t
constexpr bool enc_schedule_ok() {
  for (int t = 0; t < kIT; ++t)
    if (enc_pos(t < kYA ? 8 * t + 6 : 8 * t + 7) >= 128 + 4 * t) return false;
  for (int m = 0; m <= kEl / 2 + 1; ++m)
    if (enc_step_at(enc_pos(m)) != m || enc_pos(m) >= 192) return false;
  return true;
}
static_assert(enc_schedule_ok(), "code steps overlap the GEMM2 products that overwrite their tiles");
// every stage of the merged block is one (tile, chunk) pair, each pair once, chunk 7 of a
// tile after its chunk 6
constexpr bool m67_ok() {
  int seen[2][16] = {};
  for (int s = 0; s < 32; ++s) {
    const int t = m67_tile(s), c = m67_ch(s);
    if (t < 0 || t > 15 || (c != 6 && c != 7)) return false;
    if (seen[c - 6][t]++) return false;
    if (c == 7 && (s < 3 || !seen[0][t])) return false;  // tb of chunk 7 is rounded during stages 1 and 2
  }
  return true;
}
static_assert(m67_ok(), "merged GEMM2 order");

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
  // The workgroup's first two slices (tickets of the slice counter; one thread takes them and
  // they reach every wave through xs[1], which is free until the first GEMM1 block)
  uint32_t tk0 = 0, tk1 = 0;
  if (tid == 0) {
    tk0 = take_ticket(b.ctr);
    tk1 = take_ticket(b.ctr);
  }

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

  // Chunk cc of a slice: x rows 32cc .. 32cc+31.
  // Load h of wave w covers chunk rows 8h + 4(w/2) .. +3, slots 16(w%2) .. +15: lane l takes
  // row + (l % 4), slot + l / 4.  Bounded buffer loads (zeros past K, no memory access):
  // unconditional, so the compiler's memory-counter waits cover exactly the chunk consumed.
  u32x4_t xr[D][XR];
  const int ld_off = ((4 * (w >> 1) + (lane & 3)) * 32 + 16 * (w & 1) + (lane >> 2)) * 16;
  auto chunk_rsrc = [&](int64_t slice, int cc) {
    const bool in = slice < pb.K;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(b.x + (in ? slice : 0) * (kW * kW) + cc * (kChunk * kW)),
        static_cast<int16_t>(0), in ? kChunk * kW * 2 : 0, kBufferWord3);
  };
  auto load_chunk = [&](int64_t slice, int cc, u32x4_t* r) {
    const auto rsrc = chunk_rsrc(slice, cc);
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
  auto load_piece = [&](const auto& rsrc, int h, u32x4_t& r) {
    r = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ld_off, h * 8 * kW * 2, 0);
  };
  auto store_piece = [&](const u32x4_t& r, int h, u32x4_t* dst) { dst[((h & 1) ? st_odd : st_even) + (h >> 1) * 64] = r; };
  // LDS read bases (opaque: every fragment read is a base plus an immediate offset)
  int rd_base = 16 * g + (c ^ (4 * g));
  int f1_lo = lane, f1_hi = lane + kIT / 2 * kNChunk * 64;
  asm volatile("" : "+v"(rd_base), "+v"(f1_lo), "+v"(f1_hi));

  // the current and the next slice (wave-uniform)
  int64_t s = 0, s_nx = 0;
  {
    uint32_t* slot = reinterpret_cast<uint32_t*>(xs[1]);
    if (tid == 0) {
      slot[0] = tk0;
      slot[1] = tk1;
    }
    lds_barrier();
    s = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(slot[0]));
    s_nx = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(slot[1]));
  }
  if (s >= pb.K) return;
  uint32_t tk2 = 0;  // the ticket of the slice after the next one (thread 0)

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

  // GEMM1 of chunk j rounded into tb[out] (the chunk's T as GEMM2 B fragments)
  auto round_part = [&](auto outv, auto qv) {  // half q & 1 of n-tile q >> 1
    constexpr int out = decltype(outv)::value, q = decltype(qv)::value, nt = q >> 1;
    if constexpr ((q & 1) == 0) {
      tb[out][nt][0] = round16x2<DT>(acc[nt][0], acc[nt][1]);
      tb[out][nt][1] = round16x2<DT>(acc[nt][2], acc[nt][3]);
    } else {
      tb[out][nt][2] = round16x2<DT>(acc[kNT + nt][0], acc[kNT + nt][1]);
      tb[out][nt][3] = round16x2<DT>(acc[kNT + nt][2], acc[kNT + nt][3]);
    }
  };

  // One GEMM1 block for chunk cj of the current slice.  During stages 2, 5, 8 and 11 chunk
  // cj + 1 goes from registers to LDS, a quarter at a time, and the registers each quarter
  // frees are refilled with chunk cj + 1 + D (of the next slice from 8 on).  TAIL: T is rounded
  // into tb[cj & 1] and a barrier ends the block (the next block is GEMM1 too and needs the
  // accumulators); otherwise the GEMM2 block after it does both (g2_tail).  The barrier makes
  // chunk j + 1 visible and releases the buffer this block read.  VIS(k, nt) runs VALU work
  // after each product.  NEXT_G2 / NEXT_CH: the block after this one (its first P fragments
  // are read during this block's last stages, unless it is the GEMM1 block of chunk j + 1,
  // whose chunk is visible only after this block's barrier).
  auto g1_block = [&](auto cjv, auto carry_inv, auto tailv, auto next_g2v, auto next_chv, auto&& vis) {
    constexpr int cj = decltype(cjv)::value;
    constexpr bool carry_in = decltype(carry_inv)::value;
    constexpr bool tail = decltype(tailv)::value;
    constexpr bool next_g2 = decltype(next_g2v)::value;
    constexpr int next_ch = decltype(next_chv)::value;
    constexpr int buf = cj & 1;
    if constexpr (!carry_in) {
      read_g1(buf, 0, 0);
      read_g1(buf, 1, 1);
      read_g1(buf, 2, 2);
    }
    constexpr int ld_ch = cj + 1 + D;
    const auto rs_x = chunk_rsrc(ld_ch < kNChunk ? s : s_nx, ld_ch % kNChunk);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 16>([&](auto kv) {
      constexpr int k = decltype(kv)::value;
      if constexpr (k + P < 16)
        read_g1(buf, k + P, (k + P) % (P + 1));
      else if constexpr (next_g2)
        read_g2(next_ch, k + P - 16, (k + P) % (P + 1));
      if constexpr (k % 3 == 2 && k / 3 < XR) {
        constexpr int h = k / 3;
        store_piece(xr[(cj + 1) % D][h], h, xs[(cj + 1) & 1]);
        load_piece(rs_x, h, xr[(cj + 1) % D][h]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t a = ring[k % (P + 1)];
      constexpr int h = k & 1, ks = k >> 1;
      static_for<0, kNT>([&](auto ntv) {
        constexpr int nt = decltype(ntv)::value;
        if constexpr (ks == 0)
          acc[h * kNT + nt] = g1_first<DT>(a, p2f[ks][nt]);
        else
          g1_acc<DT>(acc[h * kNT + nt], a, p2f[ks][nt]);
        // VALU work issued while this product runs
        __builtin_amdgcn_sched_barrier(0);
        vis(kv, ntv);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    if constexpr (tail) {
      mfma_v_drain(acc);
      static_for<0, 2 * kNT>([&](auto qv) { round_part(std::integral_constant<int, cj & 1>{}, qv); });
      vgpr_fence2(tb[cj & 1]);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The deferred end of a GEMM1 block, run by the GEMM2 block after it: the accumulators are
  // read from stage 1 on (four products behind the last GEMM1 product), rounded into tb[OUT]
  // two conversions per product over stages 1 and 2, and the barrier is passed at stage BAR
  // (before the stages that read the next GEMM1 block's first fragments).
  auto g2_tail_pre = [&](auto tv, auto outv, auto barv) {
    constexpr int t = decltype(tv)::value, out = decltype(outv)::value, bar = decltype(barv)::value;
    if constexpr (t == 1) asm("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                                   "+v"(acc[6]), "+v"(acc[7]));
    if constexpr (t == 3) vgpr_fence2(tb[out]);
    if constexpr (t == bar) lds_barrier();
  };
  auto g2_tail_post = [&](auto tv, auto ntv, auto outv) {
    constexpr int t = decltype(tv)::value, nt = decltype(ntv)::value;
    if constexpr (t == 1 || t == 2) round_part(outv, std::integral_constant<int, (t - 1) * kNT + nt>{});
  };

  // One GEMM2 block for chunk CH of the current slice (T in tb[CH & 1]).  FIRST: the slice's
  // first chunk (the products start from 0).  PRE(t) runs before stage t's products, POST(t,
  // nt) after each.  NEXT_G1 / NEXT_BUF / NEXT_CH: as for g1_block.
  auto g2_block = [&](auto chv, auto next_g1v, auto next_bufv, auto next_chv, auto&& pre, auto&& post) {
    constexpr int ch = decltype(chv)::value;
    constexpr bool first = ch == 0;
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
      pre(tv);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t a = ring[t % (P + 1)];
      static_for<0, kNT>([&](auto ntv) {
        constexpr int nt = decltype(ntv)::value;
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
        __builtin_amdgcn_sched_barrier(0);
        post(tv, ntv);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };

  // ---- GEMM2 of chunks 6 and 7 in one block of 32 stages, tile by tile, chunk 7 three
  // stages behind chunk 6: tile t is final after its chunk-7 stage m67_done(t), and max|y|
  // of the slice is taken tile by tile from two stages later on (accumulation-register tiles
  // two values per product with their reads one product ahead, the others two or four values
  // per product); tiles 14 and 15 are finished after the block. ----
  float am[2] = {0.0f, 0.0f};
  // am[i] = max(am[i], |u|, |v|) in one instruction.  As inline asm it skips the compiler's
  // quieting of possibly signalling NaN inputs (two more instructions a pair): the inputs are
  // product results, never signalling, and the instruction ignores quiet NaN inputs as fmaxf
  // does.  Its register inputs are products' results behind their tile fences (at least four
  // products back) or LDS loads the compiler waits for.
  auto amax_pair = [&](int i, float u, float v) { asm("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(am[i]) : "v"(u), "v"(v)); };
  float ar[4];  // accumulation-register values read ahead of their max (read r in ar[r % 4])
  auto m67_block = [&]() {
    static_for<0, 32>([&](auto sv) {
      constexpr int st = decltype(sv)::value;
      constexpr int t = m67_tile(st), ch = m67_ch(st);
      if constexpr (st + P < 32)
        read_g2(m67_ch(st + P), m67_tile(st + P), (st + P) % (P + 1));
      else
        read_g1(0, st + P - 32, (st + P) % (P + 1));  // G1'(0): chunk 0 of the next slice in xs[0]
      __builtin_amdgcn_sched_barrier(0);
      g2_tail_pre(sv, std::integral_constant<int, 1>{}, std::integral_constant<int, kM67Bar>{});
      // tile fences: a tile is read from two stages after its last product on
      constexpr int tf = m67_fence_at(st);
      if constexpr (tf >= 0 && tf < kYA) tile_done_a(y[tf]);
      if constexpr (tf >= kYA) tile_done_v(y[tf]);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t a = ring[st % (P + 1)];
      static_for<0, kNT>([&](auto ntv) {
        constexpr int nt = decltype(ntv)::value;
        if constexpr (t < kYA)
          mfma_a_acc<DT>(y[t][nt], a, tb[ch & 1][nt]);
        else
          mfma_v_acc<DT>(y[t][nt], a, tb[ch & 1][nt]);
        __builtin_amdgcn_sched_barrier(0);
        g2_tail_post(sv, ntv, std::integral_constant<int, 1>{});
        constexpr int pos = 4 * st + nt;
        // accumulation-register tiles: the max of the pair whose second read came one product
        // ago, then this product's reads
        constexpr int k = amax_pair_at(pos);
        if constexpr (k >= 0) amax_pair(k & 1, ar[(2 * k) & 3], ar[(2 * k + 1) & 3]);
        constexpr int r0 = amax_rd_first(pos), nr = amax_rd_count(pos);
        if constexpr (nr >= 1) ar[r0 & 3] = y[r0 >> 4][(r0 >> 2) & 3][r0 & 3];
        if constexpr (nr >= 2) ar[(r0 + 1) & 3] = y[(r0 + 1) >> 4][((r0 + 1) >> 2) & 3][(r0 + 1) & 3];
        // ordinary-register tiles 8 .. 13
        constexpr int tv = amax_vtile_at(pos);
        if constexpr (tv >= 0) {
          constexpr int j = pos - 4 * (m67_done(tv) + 2);
          amax_pair(j & 1, y[tv][j >> 1][2 * (j & 1)], y[tv][j >> 1][2 * (j & 1) + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    tile_done_v(y[14]);
    mfma_v_drain(y[kIT - 1]);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      amax_pair(0, y[14][nt][0], y[14][nt][1]);
      amax_pair(1, y[14][nt][2], y[14][nt][3]);
      amax_pair(0, y[15][nt][0], y[15][nt][1]);
      amax_pair(1, y[15][nt][2], y[15][nt][3]);
    }
  };

  // ---- the codes of a finished slice (sp), formed during the next slice's first two GEMM1
  // blocks and its first GEMM2 block, two elements per step (130 steps, 256 elements a lane)
  // as a software pipeline: step m reads elements 2m+2, 2m+3 from accumulation registers,
  // forms the biased codes of elements 2m, 2m+1 (read in step m-1), joins the pair formed in
  // step m-1 into a byte, and stores the code row whose two bytes were both ready before this
  // step.  Element e is y[t][j][i] with t = e / 16 (16-row tile), i = (e / 4) % 4 (row in the
  // lane's 4-row group), j = e % 4 (column); a row's two bytes are the pairs j = 0, 1 and
  // j = 2, 3.  Step m runs after product enc_pos(m) of the 192 in G1'(0) G1'(1) G2'(0): the
  // steps are spread so that the last read of tile t precedes the first GEMM2 product that
  // overwrites it (stage t of G2'(0)). ----
  int64_t sp = 0;    // the slice whose codes are pending
  float inv = 0.0f, amax = 0.0f, scale = 0.0f;
  float rr[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};  // elements read ahead (step parity)
  uint32_t ff[2][2] = {{0u, 0u}, {0u, 0u}};       // biased codes formed (step parity)
  uint32_t ll[4] = {0u, 0u, 0u, 0u};               // the bytes of pairs q (q % 4)
  // no codes are pending before the first slice: stores through an empty range are dropped
  auto rs_codes = __builtin_amdgcn_make_buffer_rsrc(b.codes, static_cast<int16_t>(0), 0, kBufferWord3);
  const int code_off = 4 * g * (kW / 2) + 32 * w + 2 * c;  // the lane's 4 codes of a row: columns 64w + 4c ..
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
  auto encode_step = [&](auto mv) {
    constexpr int m = decltype(mv)::value;
    // store the row whose pairs (2r, 2r+1) were joined in steps <= m-1: pair 2r+1 = m-2
    if constexpr (m >= 2 && ((m - 2) & 1) == 1) {
      constexpr int q = m - 2, r = q >> 1, t = r >> 2, i = r & 3;
      __builtin_amdgcn_raw_buffer_store_b16(
          static_cast<uint16_t>(unbias(__builtin_amdgcn_perm(ll[q & 3], ll[(q - 1) & 3], 0x0C0C0400u))), rs_codes,
          code_off, (16 * t + i) * (kW / 2), 2 /* non-temporal */);
    }
    // join pair m-1 (its codes were formed in step m-1)
    if constexpr (m >= 1 && m - 1 < kEl / 2) ll[(m - 1) & 3] = pair_byte(ff[(m - 1) & 1][0], ff[(m - 1) & 1][1]);
    // form the codes of elements 2m, 2m+1 (read in step m-1)
    if constexpr (2 * m < kEl) {
      ff[m & 1][0] = code_el(std::integral_constant<int, 2 * m>{}, rr[m & 1][0]);
      ff[m & 1][1] = code_el(std::integral_constant<int, 2 * m + 1>{}, rr[m & 1][1]);
    }
    // read elements 2m+2, 2m+3
    read_el(std::integral_constant<int, 2 * m + 2>{}, rr[(m + 1) & 1][0]);
    read_el(std::integral_constant<int, 2 * m + 3>{}, rr[(m + 1) & 1][1]);
  };
  // VALU work after product POS of G1'(0) (0 .. 63), G1'(1) (64 .. 127) and G2'(0) (128 ..):
  // the slice's scale and reciprocal first, then the code steps
  auto enc_at = [&](auto posv) {
    constexpr int pos = decltype(posv)::value;
    if constexpr (pos == 0) scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(amax / pb.d)));
    // (a scale below 2^-126, whose reciprocal can overflow, is re-encoded by division after
    // this kernel)
    if constexpr (pos == 2) inv = scale > 0.0f ? 1.0f / scale : 0.0f;
    if constexpr (pos == 3) {
      const auto rs_scale = __builtin_amdgcn_make_buffer_rsrc(static_cast<float*>(b.scale) + sp, static_cast<int16_t>(0),
                                                              4, kBufferWord3);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(scale), rs_scale, 0, 0, 0);  // every lane, same bytes
      rs_codes = __builtin_amdgcn_make_buffer_rsrc(b.codes + sp * (kW * kW / 2), static_cast<int16_t>(0), kW * kW / 2,
                                                   kBufferWord3);
    }
    if constexpr (pos == 4) {
      read_el(std::integral_constant<int, 0>{}, rr[0][0]);  // step 0's elements
      read_el(std::integral_constant<int, 1>{}, rr[0][1]);
    }
    constexpr int m = enc_step_at(pos);
    if constexpr (m >= 0) encode_step(std::integral_constant<int, m>{});
  };

  using F = std::false_type;
  using T = std::true_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto nothing = [](auto, auto) {};
  auto nothing1 = [](auto) {};

  // y starts at zero: the first slice's GEMM2 block of chunk 0 runs code steps of a slice
  // that does not exist (stored nowhere) over it
#pragma unroll
  for (int t = 0; t < kIT; ++t)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) y[t][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  redefine_a_tiles(y);

  // prologue: chunk 0 in LDS, chunks 1 .. D in registers (chunk k in xr[k % D])
  load_chunk(s, 0, xr[0]);
  store_chunk(xr[0], xs[0]);
#pragma unroll
  for (int k = 1; k <= D; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(s, k, xr[k % D]);
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  // the first slice's GEMM1 of chunks 0 and 1 (nothing to encode yet)
  g1_block(I0{}, F{}, T{}, F{}, I0{}, nothing);
  g1_block(I1{}, F{}, F{}, T{}, I0{}, nothing);

  while (true) {
    // the ticket of the slice after the next one, published with this slice's max reduction
    if (tid == 0) tk2 = take_ticket(b.ctr);
    // ---- slice s: G2(0) G1(2) G2(1) G1(3) ... G2(5) G1(7) G2(6+7); each GEMM2 block ends
    // the GEMM1 block before it; G2(0) also runs the last code steps of the previous slice ----
    g2_block(I0{}, T{}, I0{}, I0{}, [&](auto tv) { g2_tail_pre(tv, I1{}, std::integral_constant<int, kBarStage>{}); },
             [&](auto tv, auto ntv) {
               g2_tail_post(tv, ntv, I1{});
               enc_at(std::integral_constant<int, 128 + kNT * decltype(tv)::value + decltype(ntv)::value>{});
             });
    g1_block(std::integral_constant<int, 2>{}, T{}, F{}, T{}, I1{}, nothing);
    static_for<1, 6>([&](auto cv) {
      constexpr int c = decltype(cv)::value;
      // G2(c) ends G1(c + 1) (tb[(c + 1) & 1]); then G1(c + 2), ahead of G2(c + 1)
      g2_block(cv, T{}, std::integral_constant<int, c & 1>{}, I0{},
               [&](auto tv) {
                 g2_tail_pre(tv, std::integral_constant<int, (c + 1) & 1>{}, std::integral_constant<int, kBarStage>{});
               },
               [&](auto tv, auto ntv) { g2_tail_post(tv, ntv, std::integral_constant<int, (c + 1) & 1>{}); });
      g1_block(std::integral_constant<int, c + 2>{}, T{}, F{}, T{}, std::integral_constant<int, c + 1>{}, nothing);
    });
    m67_block();

    // ---- [FQV2] 第3步 pertoken: max|y| over the slice (4 waves).  The partial maxima pass
    // through xs[1] (and with them the ticket of the slice after the next one): its last
    // reader, GEMM1 of chunk 7, is behind the merged block's barrier, and its next writer,
    // G1'(0), starts after the second barrier below. ----
    int64_t s_nx2 = 0;
    {
      float* red = reinterpret_cast<float*>(xs[1]);
      red[w] = wave_max(fmaxf(am[0], am[1]));  // every lane writes the same value
      if (tid == 0) reinterpret_cast<uint32_t*>(red)[4] = tk2;
      lds_barrier();
      amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      s_nx2 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(reinterpret_cast<const uint32_t*>(red)[4]));
      lds_barrier();
      am[0] = 0.0f;
      am[1] = 0.0f;
    }
    sp = s;
    s = s_nx;
    s_nx = s_nx2;

    // ---- the next slice's GEMM1 of chunks 0 and 1 (zeros past K), with slice sp's scale and
    // its first code steps ----
    redefine_a_tiles(y);
    g1_block(I0{}, T{}, T{}, F{}, I0{}, [&](auto kv, auto ntv) {
      enc_at(std::integral_constant<int, kNT * decltype(kv)::value + decltype(ntv)::value>{});
    });
    g1_block(I1{}, F{}, F{}, T{}, I0{}, [&](auto kv, auto ntv) {
      enc_at(std::integral_constant<int, 64 + kNT * decltype(kv)::value + decltype(ntv)::value>{});
    });
    if (s >= pb.K) break;
  }
  // the last slice's remaining code steps (no GEMM2 block follows)
  static_for<128, 192>([&](auto posv) { enc_at(posv); });
}

__global__ void zero_counter(uint32_t* ctr) {
  if (threadIdx.x == 0) *ctr = 0u;
}

}  // namespace

bool mfma_wide2t_supports(const Problem& pb) {
  return pb.M == kW && pb.N == kW && pb.two_sided && (pb.mode == kPerTokenInt32 || pb.mode == kPerTokenInt4);
}

hipError_t launch_mfma_wide2t(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (!mfma_wide2t_supports(pb)) return hipErrorNotSupported;
  if (!b.ctr) return hipErrorInvalidValue;
  static std::atomic<int> cus_cache{0};  // first calls from several threads may race: each stores the same value
  int cus = cus_cache.load(std::memory_order_relaxed);
  if (cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus_cache.store(cus, std::memory_order_relaxed);
  }
  const int grid = static_cast<int>(pb.K < cus ? pb.K : cus);
  // the slice counter starts from zero (a kernel, not a memset: the launch may be captured)
  zero_counter<<<1, 64, 0, s>>>(b.ctr);
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
