// Whole-workgroup MFMA kernels for 256 x 256 slices: both transforms, or P1 only.
//
// [FQV2] 拆开算 第1步/第2步 fused with 第3步/第4步 for M = N = 256.  One workgroup of 4
// waves (one per SIMD, 512 registers each) owns one slice at a time (persistent grid,
// one workgroup per CU):
//   * P1 is staged once in LDS as GEMM2 A fragments (128 KB), with the contraction index
//     relabelled to match GEMM1's accumulator layout;
//   * wave w owns the 64 output columns 64w .. 64w+63 and keeps its strip of P2 as GEMM1
//     B fragments in registers (column label c of n-tile nt is column 64w + 4c + nt, so a
//     lane holds 4 neighbouring columns);
//   * x streams through LDS in chunks of 32 rows (16 KB, XOR-swizzled 16-byte slots so the
//     A-fragment reads are conflict-free), the next chunk prefetched into registers;
//   * per chunk c: T_c = x[32c..32c+31, :] . P2[:, strip] (GEMM1, 64 MFMAs), rounded to
//     the dtype in registers, then y[:, strip] += P1[:, 32c..32c+31] . T_c (GEMM2, 64
//     MFMAs) -- the full intermediate T never exists;
//   * y (256 x 64 per wave, fp32) stays in registers; per token, max|y| is reduced across
//     the 4 waves through LDS; per group, a 32-group is 8 neighbouring lanes of one row.
// PAD: a slice of M x N elements with a side above 128 (M, N <= 256, N a multiple of 8; of
// 32 per group, so that 32-groups stay inside rows) runs in the two-sided kernel at
// 256 x 256: P1 and P2 are staged with zero rows and columns past their own sizes (an empty
// P2 as the identity: T = RNE(x * 1) = x exactly), x's rows and columns past the slice's
// read zeros through the bounded loads, so the padded y is the real one bordered by zeros
// (max|y| and every group maximum unchanged), and only the real rows and columns of the
// codes and e8m0 bytes are stored, at the slice's own row pitch.
#include <hip/hip_runtime.h>

#include <atomic>

#include <type_traits>

#include "fq_mfma_common.h"

namespace fq {
namespace {

constexpr int kWideWaves = 4;
constexpr int kNT = 4;        // n-tiles per wave (64 columns)
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kW = 256;       // M = N
constexpr int kChunk = 32;    // rows of x per chunk
constexpr int kNChunk = kW / kChunk;
constexpr int kIT = kW / 16;  // 16-row tiles of y
// cache policy of the two-sided kernel's per-token code stores: non-temporal (written once, not
// read back here).  The per-group code stores leave short runs per group of lanes, which
// non-temporal stores turn into partial-line writes (17% more HBM writes measured on the
// left-only kernel), so those stay cached.
constexpr int kStoreNT = 2;

// CLAMP (per token): the int4 or INT8 clamp is compiled in.  SV (per group): the e8m0 rule.  Q (per
// token): 0 for int4 codes, else the 8-bit mode (kPerTokenInt8 / E4M3 / E5M2), one byte a code.
// PAD: pb.M x pb.N slices padded to 256 x 256 (see above).
template <int DT, bool PG, bool CLAMP, int SV, int Q, bool PAD>
__global__ __launch_bounds__(kWideThreads, 1) void mfma_wide2_kernel(Problem pb, Buffers b) {
  __shared__ u32x4_t frag1[kIT * kNChunk * 64];   // 128 KB: P1 A fragments
  // 2 x 16 KB: x chunks in GEMM1 A-fragment order.  The 16-byte slot q = 4ks + g of chunk
  // row r = 16h + c (x columns 8q .. 8q+7) sits at (2ks + h)*64 + 16g + (c ^ 4g): a lane's
  // reads are one base address plus immediate offsets, and both the reads and the stores
  // below touch 16 distinct bank groups per 16 lanes.
  __shared__ u32x4_t xs[2][kChunk * 32];
  constexpr int D = 2;                            // chunks in flight in registers (divides 8)
  constexpr int XR = kChunk * kW * 2 / 16 / kWideThreads;  // 16-byte pieces per thread per chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t stride = gridDim.x;

  // ---- P1 -> LDS fragments: P1[i, m] -> frag1[(it*8 + ch)*64 + 16*gg + i%16] element t,
  // m = 32ch + (t < 4 ? 4gg + t : 16 + 4gg + t - 4) ----
  // the slice's own sizes (256 when not padded)
  const int Mr = PAD ? static_cast<int>(pb.M) : kW, Nr = PAD ? static_cast<int>(pb.N) : kW;
  if constexpr (PAD) {
    // element by element, zero past P1's own Mr x Mr
    uint16_t* f1 = reinterpret_cast<uint16_t*>(frag1);
    for (int ch16 = tid; ch16 < kW * kW / 8; ch16 += kWideThreads) {
      const int i = ch16 >> 5, m0 = (ch16 & 31) * 8;
      const int it = i >> 4, rr = i & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = m0 + e, ch = m >> 5, wv = m & 31;
        const int gg = wv < 16 ? (wv >> 2) : ((wv - 16) >> 2);
        const int t = wv < 16 ? (wv & 3) : 4 + ((wv - 16) & 3);
        f1[((it * kNChunk + ch) * 64 + 16 * gg + rr) * 8 + t] = (i < Mr && m < Mr) ? b.p1[i * Mr + m] : uint16_t(0);
      }
    }
  } else {
    uint16_t* f1 = reinterpret_cast<uint16_t*>(frag1);
    for (int base = 0; base < kW * kW / 8; base += kWideThreads * 4) {
      u32x4_t r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = reinterpret_cast<const u32x4_t*>(b.p1)[base + q * kWideThreads + tid];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch16 = base + q * kWideThreads + tid;
        const int i = ch16 >> 5, m0 = (ch16 & 31) * 8;
        const int it = i >> 4, rr = i & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = m0 + e, ch = m >> 5, wv = m & 31;
          const int gg = wv < 16 ? (wv >> 2) : ((wv - 16) >> 2);
          const int t = wv < 16 ? (wv & 3) : 4 + ((wv - 16) & 3);
          f1[((it * kNChunk + ch) * 64 + 16 * gg + rr) * 8 + t] =
              static_cast<uint16_t>(r[q][e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
  // ---- this wave's P2 strip as GEMM1 B fragments: p2f[ks][nt] element t =
  // P2[32ks + 8g + t, 64w + 4c + nt] ----
  u32x4_t p2f[kW / 32][kNT];
  if constexpr (PAD) {
    // zero past P2's own Nr x Nr; an empty P2 is the identity
    const uint16_t one = DT == kBF16 ? uint16_t(0x3F80) : uint16_t(0x3C00);
    auto p2v = [&](int j, int n) -> uint32_t {
      if (j >= Nr || n >= Nr) return 0u;
      return pb.two_sided ? uint32_t(b.p2[j * Nr + n]) : (j == n ? uint32_t(one) : 0u);
    };
#pragma unroll
    for (int ks = 0; ks < kW / 32; ++ks)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int j0 = 32 * ks + 8 * g, n = 64 * w + 4 * c + nt;
        uint32_t v[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) v[p] = p2v(j0 + 2 * p, n) | (p2v(j0 + 2 * p + 1, n) << 16);
        p2f[ks][nt] = u32x4_t{v[0], v[1], v[2], v[3]};
      }
  } else {
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
  }

  // Chunk j of the workgroup: slice blockIdx.x + (j / 8) * gridDim.x, x rows 32 * (j % 8) ..
  // Load h of wave w covers chunk rows 8h + 4(w/2) .. +3, slots 16(w%2) .. +15: lane l takes
  // row + (l % 4), slot + l / 4 (whole 256-byte row halves per instruction).  Bounded buffer
  // loads (zeros past K, no memory access): unconditional, so the compiler's memory-counter
  // waits cover exactly the chunk being consumed.
  u32x4_t xr[D][XR];
  const int ld_off = ((4 * (w >> 1) + (lane & 3)) * 32 + 16 * (w & 1) + (lane >> 2)) * 16;
  auto load_chunk = [&](int64_t j, u32x4_t* r) {
    const int64_t slice = blockIdx.x + (j >> 3) * stride;
    const bool in = slice < pb.K;
    if constexpr (PAD) {
      // a resource over the whole slice; the lane's row (32 (j % 8) + 8h + 4 (w/2) + l%4) and
      // 16-byte piece (columns 8 (16 (w%2) + l/4) ..) in the offset, sent past the range
      // (zeros, no memory access) for rows and columns past the slice's own
      const int bytes = Mr * Nr * 2;
      const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b.x + (in ? slice : 0) * (int64_t(Mr) * Nr)),
                                                          static_cast<int16_t>(0), in ? bytes : 0, kBufferWord3);
      const int row0 = kChunk * static_cast<int>(j & 7) + 4 * (w >> 1) + (lane & 3);
      const int col = 8 * (16 * (w & 1) + (lane >> 2));
#pragma unroll
      for (int h = 0; h < XR; ++h) {
        const int row = row0 + 8 * h;
        const int off = (row < Mr && col < Nr) ? (row * Nr + col) * 2 : bytes;
        r[h] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      }
      return;
    }
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(b.x + (in ? slice : 0) * (kW * kW) + (j & 7) * (kChunk * kW)),
        static_cast<int16_t>(0), in ? kChunk * kW * 2 : 0, kBufferWord3);
#pragma unroll
    for (int h = 0; h < XR; ++h) r[h] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ld_off, h * 8 * kW * 2, 0);
  };
  // the slot of load h: row 8h + 4(w/2) + l%4 (c = 8(h%2) + 4(w/2) + l%4, h_row = h/2),
  // slot 16(w%2) + l/4 (ks = 4(w%2) + l/16, g = (l/4)%4)
  const int sg = (lane >> 2) & 3;
  const int st_even = (4 * (w & 1) + (lane >> 4)) * 2 * 64 + 16 * sg + ((4 * (w >> 1) + (lane & 3)) ^ (4 * sg));
  const int st_odd = st_even ^ 8;
  auto store_chunk = [&](const u32x4_t* r, u32x4_t* dst) {
#pragma unroll
    for (int h = 0; h < XR; ++h) dst[((h & 1) ? st_odd : st_even) + (h >> 1) * 64] = r[h];
  };
  // LDS read bases (opaque, so every fragment read is one of three bases plus an immediate
  // offset below 64 KB instead of an address register of its own hoisted out of the loop):
  // the lane's x-chunk slot, and its P1 fragment slot in the low and high 64 KB of frag1.
  int rd_base = 16 * g + (c ^ (4 * g));
  int f1_lo = lane, f1_hi = lane + kIT / 2 * kNChunk * 64;
  asm volatile("" : "+v"(rd_base), "+v"(f1_lo), "+v"(f1_hi));

  int64_t s = blockIdx.x;
  if (s >= pb.K) return;
  // prologue: chunk 0 in LDS, chunks 1 .. D in registers (chunk k in xr[k % D]), issued in
  // chunk order, so that waiting for one chunk never waits for a later one.
  load_chunk(0, xr[0]);
  store_chunk(xr[0], xs[0]);
#pragma unroll
  for (int k = 1; k <= D; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(k, xr[k % D]);
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();  // chunk 0 is in LDS

  int64_t j0 = 0;  // chunk index of this slice's chunk 0
  f32x4_t y[kIT][kNT];
  float amax_run = 0.0f;  // per token: max|y| of the slice's finished tiles

  // A chunk is 32 stages of 4 products sharing one A fragment: stages 0..15 are GEMM1
  // (k-step k/2 of row half k%2, A from the x chunk), stages 16..31 GEMM2 (row tile k-16,
  // A from P1).  The A fragment of stage k is read P stages ahead into ring[k % 4]; the
  // scheduling barriers keep that order (the compiler cannot see the products' latency).
  constexpr int P = 3;
  u32x4_t ring[P + 1];
  auto read_a = [&](auto chv, auto kv) {
    constexpr int ch = decltype(chv)::value, k = decltype(kv)::value;
    if constexpr (k < 16)
      ring[k % (P + 1)] = xs[ch & 1][rd_base + (2 * (k >> 1) + (k & 1)) * 64];
    else
      ring[k % (P + 1)] = k < 16 + kIT / 2 ? frag1[f1_lo + ((k - 16) * kNChunk + ch) * 64]
                                           : frag1[f1_hi + ((k - 16 - kIT / 2) * kNChunk + ch) * 64];
  };

  // One chunk: T_ch = x[32ch .. 32ch+31, :] . P2[:, strip] (GEMM1), rounded to the dtype in
  // registers, then y[:, strip] += P1[:, 32ch .. 32ch+31] . T_ch (GEMM2).  The barrier sits
  // between the two: before it every wave has stored chunk ch+1 and finished reading chunk
  // ch, so after it the next chunk's first fragments can be read and, in the next step,
  // chunk ch+2 can be stored over chunk ch.  CARRY: stages 0..P-1 of this chunk were read
  // by the previous step.
  auto chunk_step = [&](auto chv, auto carryv) {
    constexpr int ch = decltype(chv)::value;
    constexpr bool carry_in = decltype(carryv)::value;
    constexpr bool carry_out = ch != kNChunk - 1;  // the next slice's chunk 0 starts afresh
    if constexpr (!PG && ch == kNChunk - 1) amax_run = 0.0f;
    if constexpr (!carry_in) {
      read_a(chv, std::integral_constant<int, 0>{});
      read_a(chv, std::integral_constant<int, 1>{});
      read_a(chv, std::integral_constant<int, 2>{});
    }
    store_chunk(xr[(ch + 1) % D], xs[(ch + 1) & 1]);
    load_chunk(j0 + ch + 1 + D, xr[(ch + 1) % D]);
    __builtin_amdgcn_sched_barrier(0);

    f32x4_t acc[2 * kNT];
    u32x4_t tb[kNT];
    static_for<0, 32>([&](auto kv) {
      constexpr int k = decltype(kv)::value;
      if constexpr (k + P < 32)
        read_a(chv, std::integral_constant<int, k + P>{});
      else if constexpr (carry_out)
        read_a(std::integral_constant<int, ch + 1>{}, std::integral_constant<int, k + P - 32>{});
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t a = ring[k % (P + 1)];
      if constexpr (k < 16) {
        constexpr int h = k & 1, ks = k >> 1;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          if constexpr (ks == 0)
            acc[h * kNT + nt] = mfma_v_first<DT>(a, p2f[ks][nt]);
          else
            mfma_v_acc<DT>(acc[h * kNT + nt], a, p2f[ks][nt]);
        }
      } else {
        // per token, last chunk: max|y| of the tile the previous stage finished, a quarter
        // after each product (VALU work issued while the product runs; the last tile
        // follows in the epilogue)
        constexpr bool amax_here = !PG && ch == kNChunk - 1 && k >= 17;
        constexpr int t = amax_here ? k - 17 : 0;
        if constexpr (amax_here) agpr_tiles_done(y[t]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          if constexpr (ch == 0)
            mfma_a_first<DT>(y[k - 16][nt], a, tb[nt]);
          else
            mfma_a_acc<DT>(y[k - 16][nt], a, tb[nt]);
          if constexpr (amax_here) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i) amax_run = fmaxf(amax_run, __builtin_fabsf(y[t][nt][i]));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k == 15) {
        mfma_v_drain(acc);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          tb[nt] = u32x4_t{round16x2<DT>(acc[nt][0], acc[nt][1]), round16x2<DT>(acc[nt][2], acc[nt][3]),
                           round16x2<DT>(acc[kNT + nt][0], acc[kNT + nt][1]),
                           round16x2<DT>(acc[kNT + nt][2], acc[kNT + nt][3])};
        vgpr_fence2(tb);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };

  // Output stores go through buffer resources for this slice: a per-lane offset (made
  // opaque per slice, so no per-row address is hoisted out of the slice loop and held in
  // registers) plus the row as a scalar offset.
  auto epilogue = [&]() {
    agpr_fence<16>(y);
    constexpr int kCodeB = Q ? kW * kW : kW * kW / 2;  // code bytes of a slice
    const int code_bytes = PAD ? (Q ? Mr * Nr : Mr * Nr / 2) : kCodeB;
    const auto rs_codes = __builtin_amdgcn_make_buffer_rsrc(b.codes + s * code_bytes, static_cast<int16_t>(0), code_bytes,
                                                            kBufferWord3);
    // the lane's 4 codes of a row are columns 64 w + 4 c .. +3 (PAD: the column bytes alone;
    // the row goes into the offset below)
    int code_off = PAD ? (Q ? 64 * w + 4 * c : 32 * w + 2 * c)
                       : (Q ? 4 * g * kW + 64 * w + 4 * c : 4 * g * (kW / 2) + 32 * w + 2 * c);
    int prow = 4 * g;  // the lane's row in a tile, less r0
    if constexpr (PAD)
      asm volatile("" : "+v"(code_off), "+v"(prow));
    else
      asm volatile("" : "+v"(code_off));
    // store offsets of the lane's codes of row r0 + 4g (r0 = 16 it + i): vector and scalar
    // part; PAD: the whole offset in the vector part, past the range (no store) for rows and
    // columns past the slice's own
    auto cvo = [&](int r0) -> int {
      if constexpr (PAD)
        return (r0 + prow < Mr && 64 * w + 4 * c < Nr) ? (r0 + prow) * (Q ? Nr : Nr / 2) + code_off : code_bytes;
      else
        return code_off;
    };
    auto cso = [&](int r0) -> int { return PAD ? 0 : r0 * (Q ? kW : kW / 2); };
    // PAD: cached stores (a row of a narrower slice leaves runs shorter than a cache line,
    // which non-temporal stores write to HBM as partial lines: 1.4x the code bytes measured
    // at 224 x 128)
    constexpr int kSt = PAD ? 0 : kStoreNT;
    if constexpr (!PG) {
      // [FQV2] 第3步 pertoken: max|y| over the slice (4 waves), scale, codes.  The partial
      // maxima pass through xs[1], which held the slice's last chunk (every wave finished
      // reading it before the last chunk's barrier) and is written next by the next slice's
      // first chunk step.
      // (the scheduling barriers keep each pass to one 16-row tile of y at a time)
      float amax = amax_run;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, __builtin_fabsf(y[kIT - 1][nt][i]));
      amax = wave_max(amax);
      float* red = reinterpret_cast<float*>(xs[1]);
      // (no lane-dependent branches in this epilogue: with every accumulation register
      // live, a divergent branch costs the register allocator hundreds of spills)
      red[w] = amax;  // every lane writes the same value
      lds_barrier();
      amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      lds_barrier();  // every wave has read `red` before the next chunk is stored over it
      const float scale = amax / pb.d;
      float inv = scale > 0.0f ? 1.0f / scale : 0.0f;
      agpr_pass_end(y, inv);  // the codes pass reads y only once inv is known
      {
        // every lane stores the same 4 bytes
        const auto rs_scale = __builtin_amdgcn_make_buffer_rsrc(static_cast<float*>(b.scale) + s, static_cast<int16_t>(0),
                                                                4, kBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(scale), rs_scale, 0, 0, 0);
      }
      if constexpr (Q != 0) {
        // 8-bit codes (the dequant_swiglu_quant page, section 3.4): 4 bytes a row
#pragma unroll
        for (int it = 0; it < kIT; ++it)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r0 = 16 * it + i;  // row - 4g
            const uint32_t v = code8x4<Q, CLAMP>(y[it][0][i], y[it][1][i], y[it][2][i], y[it][3][i], inv);
            __builtin_amdgcn_raw_buffer_store_b32(v, rs_codes, cvo(r0), cso(r0), kSt);
            if (i == 3) __builtin_amdgcn_sched_barrier(0);
          }
      } else {
#pragma unroll
      for (int it = 0; it < kIT; ++it)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 16 * it + i;  // row - 4g
          const uint32_t b0 = pair_byte(int4_biased<CLAMP>(y[it][0][i], inv), int4_biased<CLAMP>(y[it][1][i], inv));
          const uint32_t b1 = pair_byte(int4_biased<CLAMP>(y[it][2][i], inv), int4_biased<CLAMP>(y[it][3][i], inv));
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(unbias(__builtin_amdgcn_perm(b1, b0, 0x0C0C0400u))),
                                                rs_codes, cvo(r0), cso(r0), kSt);
          if (i == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // [FQV2] 第3步 pergroup / 第4步: a 32-group is 8 neighbouring lanes of one row
      const int e8_bytes = static_cast<int>(e8m0_bytes_per_slice(int64_t(Mr) * Nr));
      const auto rs_e8 = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(b.scale) + s * e8_bytes,
                                                           static_cast<int16_t>(0), e8_bytes, kBufferWord3);
      int e8_off = PAD ? 2 * w + (c >> 3) : 4 * g * (kW / 32) + 2 * w + (c >> 3);
      asm volatile("" : "+v"(e8_off));
      // the group's e8m0 byte of row r0 + 4g (PAD: whole offset, past the range for rows
      // and groups past the slice's own)
      auto evo = [&](int r0) -> int {
        if constexpr (PAD)
          return (r0 + prow < Mr && 64 * w + 32 * (c >> 3) < Nr) ? (r0 + prow) * (Nr / 32) + e8_off : e8_bytes;
        else
          return e8_off;
      };
      auto eso = [&](int r0) -> int { return PAD ? 0 : r0 * (kW / 32); };
      if constexpr (PAD) {
        // an odd count of groups leaves the slice's last e8m0 byte as padding: zero
        const int groups = Mr * Nr / 32;
        __builtin_amdgcn_raw_buffer_store_b8(uint8_t(0), rs_e8, (tid == 0 && (groups & 1)) ? groups : e8_bytes, 0, 0);
      }
#pragma unroll
      for (int it = 0; it < kIT; ++it)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 16 * it + i;  // row - 4g
          float amax = fmaxf(fmaxf(__builtin_fabsf(y[it][0][i]), __builtin_fabsf(y[it][1][i])),
                             fmaxf(__builtin_fabsf(y[it][2][i]), __builtin_fabsf(y[it][3][i])));
          amax = group_max<8>(amax);
          const uint32_t code = e8m0_code_v<SV>(amax, pb.dmax, pb.dmax_inv);
          const float sc = e8m0_to_float(code);
          uint32_t packed = fp4x2<0>(0u, y[it][0][i], y[it][1][i], sc);
          packed = fp4x2<1>(packed, y[it][2][i], y[it][3][i], sc);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(packed), rs_codes, cvo(r0), cso(r0), 0);
          // the 8 lanes of a group hold the same code and all store it (no branch)
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(code), rs_e8, evo(r0), eso(r0), 0);
        }
    }
  };

  // The slice loop is rotated to start at chunk 4: the loop head's waits see the same
  // loads in flight on entry and on every later pass.
  using F = std::false_type;
  using T = std::true_type;
  chunk_step(std::integral_constant<int, 0>{}, F{});
  chunk_step(std::integral_constant<int, 1>{}, T{});
  chunk_step(std::integral_constant<int, 2>{}, T{});
  chunk_step(std::integral_constant<int, 3>{}, T{});
  while (true) {
    chunk_step(std::integral_constant<int, 4>{}, T{});
    chunk_step(std::integral_constant<int, 5>{}, T{});
    chunk_step(std::integral_constant<int, 6>{}, T{});
    chunk_step(std::integral_constant<int, 7>{}, T{});
    epilogue();
    s += stride;
    j0 += kNChunk;
    if (s >= pb.K) break;
    chunk_step(std::integral_constant<int, 0>{}, F{});
    chunk_step(std::integral_constant<int, 1>{}, T{});
    chunk_step(std::integral_constant<int, 2>{}, T{});
    chunk_step(std::integral_constant<int, 3>{}, T{});
  }
}

// ---------------------------------------------------------------------------------------
// Left-only 256 x 256 slices (P2 = [0, 0], per-group mode): y = P1 . x.
//   * 8 waves per workgroup, two per SIMD, one workgroup per CU; wave w computes rows
//     64*(w&3) .. +63 of columns 128*(w>>2) .. +127, so its part of y is 128 fp32 per lane
//     and stays in ordinary registers (the epilogue reads it without moving it out of
//     accumulation registers), and each SIMD has a second wave to run while one waits;
//   * P1 is staged once in LDS as A fragments in natural k order (128 KB);
//   * x streams HBM -> registers -> LDS in chunks of 32 rows (16 KB), two chunks ahead in
//     registers.  x is the B operand with the contraction over rows, so a lane needs 8
//     rows of one column: the transpose is done once per chunk, as it is written to LDS.
//     Thread (r, j) loads rows 2r and 2r+1, columns 8j .. 8j+7, pairs the two rows of each
//     column in one dword (v_perm_b32), and writes the 8 dwords to the places of the B
//     fragments (u, lane, q) they belong to; every wave then reads its operands with plain
//     16-byte reads.  MFMA u of a k-step takes column 8c + u of the lane's block, so after
//     the 8 MFMAs a lane holds 8 neighbouring columns of 4 rows: one 4-byte E2M1 run per
//     row, and a 32-group spans 4 neighbouring lanes (a quad).
constexpr int kLeftWaves = 8;
constexpr int kLeftThreads = 64 * kLeftWaves;

template <int DT, int SV>
__global__ __launch_bounds__(kLeftThreads, 1) void mfma_wide1_kernel(Problem pb, Buffers b) {
  __shared__ u32x4_t frag1[kIT * kNChunk * 64];  // 128 KB: P1 A fragments (natural k order)
  // 2 x 16 KB: one chunk as B fragments, xs[buf][(sc*8 + u)*64 + 16g + c] element q = rows
  // 8g + 2q, 8g + 2q + 1 of column 128sc + 8c + u
  __shared__ u32x4_t xs[2][kChunk * 32];
  constexpr int D = 2;                           // chunks in flight in registers (divides 8)
  constexpr int XR = kChunk * kW * 2 / 16 / kLeftThreads;  // 16-byte pieces per thread per chunk
  constexpr int RT = 4;                          // 16-row tiles per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int rq = w & 3, sc = w >> 2;  // row quarter, column half
  const int64_t stride = gridDim.x;

  u32x4_t xr[D][XR];
  // This thread's pieces of chunk j of the workgroup (slice blockIdx.x + (j / 8) *
  // gridDim.x, x rows 32 * (j % 8) + 2r and 2r + 1, columns 8jj .. 8jj+7, where
  // r = tid / 32, jj = tid % 32).  Bounded buffer loads (zeros past K, no memory access):
  // unconditional, so the compiler's memory-counter waits cover exactly the chunk
  // being consumed.
  const int pr = tid >> 5, pj = tid & 31;
  auto load_chunk = [&](int64_t j, u32x4_t* r) {
    const int64_t slice = blockIdx.x + (j >> 3) * stride;
    const bool in = slice < pb.K;
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(b.x + (in ? slice : 0) * (kW * kW) + (j & 7) * (kChunk * kW)),
        static_cast<int16_t>(0), in ? kChunk * kW * 2 : 0, kBufferWord3);
#pragma unroll
    for (int h = 0; h < XR; ++h)
      r[h] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ((2 * pr) * kW + 8 * pj) * 2, h * kW * 2, 0);
  };
  // pair rows 2r, 2r+1 per column and write each dword to its fragment place:
  // column n = 8jj + e -> sc = jj / 16, c = jj % 16, u = e; row pair 2r -> g = r / 4, q = r % 4
  const int st_base = ((pj >> 4) * 8 * 64 + (pr >> 2) * 16 + (pj & 15)) * 4 + (pr & 3);
  auto store_chunk = [&](const u32x4_t* r, u32x4_t* dst) {
    uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      d32[st_base + e * 64 * 4] = __builtin_amdgcn_perm(r[1][e >> 1], r[0][e >> 1], sel);
    }
  };
  // P1[i, 32ch + 8gg .. +7] -> frag1[(it*8 + ch)*64 + 16*gg + i%16]
  for (int q = tid; q < kW * kW / 8; q += kLeftThreads) {
    const int i = q >> 5, m0 = (q & 31) * 8;
    const int it = i >> 4, ch = m0 >> 5, gg = (m0 & 31) >> 3;
    frag1[(it * kNChunk + ch) * 64 + 16 * gg + (i & 15)] = reinterpret_cast<const u32x4_t*>(b.p1)[q];
  }

  int64_t s = blockIdx.x;
  if (s >= pb.K) return;
  // prologue: chunk 0 in LDS, chunks 1 .. D in registers (chunk k in xr[k % D]), issued
  // in chunk order, so that waiting for one chunk never waits for a later one.
  load_chunk(0, xr[0]);
  store_chunk(xr[0], xs[0]);
#pragma unroll
  for (int k = 1; k <= D; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(k, xr[k % D]);
  }
  __builtin_amdgcn_sched_barrier(0);

  const float dinv = pb.dmax_inv;
  int64_t j0 = 0;  // chunk index of this slice's chunk 0
  f32x4_t y[RT][8];

  // One chunk of the current slice: y[rows, cols] += P1[rows, chunk] . x[chunk, cols].
  auto chunk_step = [&](auto chv) {
    constexpr int ch = decltype(chv)::value;
    // chunk ch is in xs[ch & 1]; every wave is done with the other buffer
    lds_barrier();
    // chunk ch + 1: registers -> the free buffer; then request chunk ch + 1 + D into
    // the registers it frees
    store_chunk(xr[(ch + 1) % D], xs[(ch + 1) & 1]);
    load_chunk(j0 + ch + 1 + D, xr[(ch + 1) % D]);

    u32x4_t a[RT];
#pragma unroll
    for (int it = 0; it < RT; ++it) a[it] = frag1[((RT * rq + it) * kNChunk + ch) * 64 + lane];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4_t bx[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) bx[u] = xs[ch & 1][(sc * 8 + 4 * half + u) * 64 + lane];
#pragma unroll
      for (int it = 0; it < RT; ++it)
#pragma unroll
        for (int u = 0; u < 4; ++u) y[it][4 * half + u] = mfma16x16x32<DT>(a[it], bx[u], y[it][4 * half + u]);
    }
  };

  // [FQV2] 第3步 pergroup / 第4步 for the current slice: 32-groups of 4 neighbouring
  // lanes (a quad).  Stores through buffer resources of the slice: a per-lane offset
  // (opaque per slice, so no per-row address is hoisted and held in registers) plus the
  // row as a scalar offset.  A row's four e8m0 bytes (one per quad) are gathered into
  // one dword, so each 16-row tile costs one e8m0 store instead of four.
  auto epilogue = [&]() {
    const auto rs_codes = __builtin_amdgcn_make_buffer_rsrc(b.codes + s * (kW * kW / 2), static_cast<int16_t>(0),
                                                            kW * kW / 2, kBufferWord3);
    const auto rs_e8 = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(b.scale) + s * e8m0_bytes_per_slice(kW * kW), static_cast<int16_t>(0),
        static_cast<int>(e8m0_bytes_per_slice(kW * kW)), kBufferWord3);
    const int j = c & 3, k = c >> 2;  // lane in its quad, quad (= group) in the row
    int code_off = (64 * rq + 4 * g) * (kW / 2) + 64 * sc + 4 * c;
    int e8_off = (64 * rq + 4 * g + j) * (kW / 32) + 4 * sc;  // the dword of row 4g + j
    asm volatile("" : "+v"(code_off), "+v"(e8_off));
#pragma unroll
    for (int it = 0; it < RT; ++it) {
      uint32_t codes4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 16 * it + i;  // row - 64rq - 4g
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) amax = fmaxf(amax, __builtin_fabsf(y[it][u][i]));
        amax = group_max<4>(amax);
        const uint32_t code = e8m0_code_v<SV>(amax, pb.dmax, dinv);
        codes4[i] = code;
        const float scf = e8m0_to_float(code);
        uint32_t packed = fp4x2<0>(0u, y[it][0][i], y[it][1][i], scf);
        packed = fp4x2<1>(packed, y[it][2][i], y[it][3][i], scf);
        packed = fp4x2<2>(packed, y[it][4][i], y[it][5][i], scf);
        packed = fp4x2<3>(packed, y[it][6][i], y[it][7][i], scf);
        __builtin_amdgcn_raw_buffer_store_b32(packed, rs_codes, code_off, r0 * (kW / 2), 0);  // cached: 32-byte runs
      }
      // lane (k, j) takes row 4g + j's code of group k, places it at byte k, and ORs in
      // the other three quads' bytes (rotations by 4, 8, 12 lanes reach all of them)
      const uint32_t all4 = codes4[0] | (codes4[1] << 8) | (codes4[2] << 16) | (codes4[3] << 24);
      const uint32_t mine = __builtin_amdgcn_ubfe(all4, 8 * j, 8) << (8 * k);
      const uint32_t row4 = mine | dpp_u<kDppRowRor4>(mine) | dpp_u<kDppRowRor8>(mine) | dpp_u<kDppRowRor12>(mine);
      // the four lanes of row 4g + j hold the same dword and all store it (no branch)
      __builtin_amdgcn_raw_buffer_store_b32(row4, rs_e8, e8_off, 16 * it * (kW / 32), 0);
    }
  };

  auto zero_y = [&]() {
#pragma unroll
    for (int it = 0; it < RT; ++it)
#pragma unroll
      for (int u = 0; u < 8; ++u) y[it][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // The slice loop is rotated to start at chunk 4: the loop head's waits see the same
  // loads in flight on entry and on every later pass, while the waits right after the
  // epilogue's stores sit inside the body where they are counted exactly.
  zero_y();
  chunk_step(std::integral_constant<int, 0>{});
  chunk_step(std::integral_constant<int, 1>{});
  chunk_step(std::integral_constant<int, 2>{});
  chunk_step(std::integral_constant<int, 3>{});
  while (true) {
    chunk_step(std::integral_constant<int, 4>{});
    chunk_step(std::integral_constant<int, 5>{});
    chunk_step(std::integral_constant<int, 6>{});
    chunk_step(std::integral_constant<int, 7>{});
    epilogue();
    s += stride;
    j0 += kNChunk;
    if (s >= pb.K) break;
    zero_y();
    chunk_step(std::integral_constant<int, 0>{});
    chunk_step(std::integral_constant<int, 1>{});
    chunk_step(std::integral_constant<int, 2>{});
    chunk_step(std::integral_constant<int, 3>{});
  }
}

template <int DT, int SV>
hipError_t launch_w1(const Problem& pb, const Buffers& b, hipStream_t s) {
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
  mfma_wide1_kernel<DT, SV><<<grid, kLeftThreads, 0, s>>>(pb, b);
  return hipGetLastError();
}

template <int DT, bool PG, bool CLAMP, int SV, int Q, bool PAD>
hipError_t launch_w2(const Problem& pb, const Buffers& b, hipStream_t s) {
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
  mfma_wide2_kernel<DT, PG, CLAMP, SV, Q, PAD><<<grid, kWideThreads, 0, s>>>(pb, b);
  return hipGetLastError();
}

template <int DT, bool PAD>
hipError_t dispatch_w2(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (pb.mode == kPerGroupFp4) {
    switch (e8m0_variant(pb)) {
      case kE8V1: return launch_w2<DT, true, false, kE8V1, 0, PAD>(pb, b, s);
      case kE8V2Pow2: return launch_w2<DT, true, false, kE8V2Pow2, 0, PAD>(pb, b, s);
      default: return launch_w2<DT, true, false, kE8V2Div, 0, PAD>(pb, b, s);
    }
  }
  switch (pb.mode) {
    case kPerTokenInt8:
      // The INT8 clamp can only bite when (127/clipRatio) * (1 + 4 ulp) reaches 127.5.
      if (pb.d >= 127.4999f) return launch_w2<DT, false, true, kE8V1, kPerTokenInt8, PAD>(pb, b, s);
      return launch_w2<DT, false, false, kE8V1, kPerTokenInt8, PAD>(pb, b, s);
    case kPerTokenE4M3: return launch_w2<DT, false, false, kE8V1, kPerTokenE4M3, PAD>(pb, b, s);
    case kPerTokenE5M2: return launch_w2<DT, false, false, kE8V1, kPerTokenE5M2, PAD>(pb, b, s);
    default: break;
  }
  if (pb.d >= 7.4999f) return launch_w2<DT, false, true, kE8V1, 0, PAD>(pb, b, s);
  return launch_w2<DT, false, false, kE8V1, 0, PAD>(pb, b, s);
}

template <int DT>
hipError_t dispatch_w1(const Problem& pb, const Buffers& b, hipStream_t s) {
  switch (e8m0_variant(pb)) {
    case kE8V1: return launch_w1<DT, kE8V1>(pb, b, s);
    case kE8V2Pow2: return launch_w1<DT, kE8V2Pow2>(pb, b, s);
    default: return launch_w1<DT, kE8V2Div>(pb, b, s);
  }
}

}  // namespace

namespace {
// M x N slices that run padded to 256 x 256: a side above 128 (smaller ones fit the
// one-wave-per-slice kernel), N a multiple of 8 (16-byte x pieces inside rows), per group a
// multiple of 32 (32-groups inside rows, as in the padded layout).
bool wide_padded_shape(const Problem& pb) {
  return (pb.M > 128 || pb.N > 128) && pb.M <= kW && pb.N <= kW && !(pb.M == kW && pb.N == kW) && pb.N % 8 == 0 &&
         (pb.mode != kPerGroupFp4 || pb.N % 32 == 0);
}
}  // namespace

bool mfma_wide_supports(const Problem& pb) {
  // two-sided: every mode; left-only: per group (the only mode an empty P2 is valid for)
  return (pb.M == kW && pb.N == kW && (pb.two_sided || pb.mode == kPerGroupFp4)) || wide_padded_shape(pb);
}

hipError_t launch_mfma_wide(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (!mfma_wide_supports(pb)) return hipErrorNotSupported;
  if (wide_padded_shape(pb))  // both sides, an empty P2 as the identity
    return pb.dtype == kBF16 ? dispatch_w2<kBF16, true>(pb, b, s) : dispatch_w2<kF16, true>(pb, b, s);
  if (!pb.two_sided) return pb.dtype == kBF16 ? dispatch_w1<kBF16>(pb, b, s) : dispatch_w1<kF16>(pb, b, s);
  return pb.dtype == kBF16 ? dispatch_w2<kBF16, false>(pb, b, s) : dispatch_w2<kF16, false>(pb, b, s);
}

}  // namespace fq
