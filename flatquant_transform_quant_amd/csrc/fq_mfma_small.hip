// Small-slice MFMA kernel: one wave per slice x_k [M, N] for M in {16, 32, 64, 128},
// N in {32, 64, 128}, both modes, both dtypes; and N = 16 for the int4 per-token codes
// (GEMM1's contraction padded to 32 with zero columns of x and zero rows of P2).  Per token
// above 4096 elements (a slice's y, M*N/64 fp32 a lane, with two slices of x in flight) and
// per group above 8192 (x and T of a slice, M*N/32 registers each) the registers of two
// waves per SIMD do not suffice: those shapes run one wave per SIMD; per token above 8192
// even those cannot hold all of y, and GEMM2 runs twice, one 16-row tile at a time (first
// for max|y|, then for the codes).
// PAD: a per-token slice of M x N elements with M <= 128 and N <= 128 a multiple of 8 runs
// in the instantiation of the next sizes up (16, 32, 64, 128; 32 up for the 8-bit codes), a
// per-group one with M <= 128 and N in {32, 64, 128} in that of the next M up (its 32-groups
// stay inside rows): x's rows and columns past the slice's own read zeros through the
// bounded loads, P1 and P2 are staged with zero rows and columns past their own sizes, so
// the padded y is the real one bordered by zeros (max|y| unchanged), and the codes and e8m0
// bytes are staged and stored for the real rows and columns only.
//
// [FQV2] 拆开算 第1步/第2步 on the matrix cores, fused with 第3步/第4步:
//   GEMM1  T = x_k . P2   A = x rows (straight from HBM, 16 B per lane),
//                         B = P2 fragments (LDS), fp32 accumulate, then RNE to the dtype.
//   GEMM2  y = P1 . T     A = P1 fragments (LDS), B = T taken directly from GEMM1's
//                         accumulator registers: the contraction index m is relabelled
//                         so that a lane's two 4-row accumulator blocks are its 8
//                         k-slots, and P1's columns are stored in the same order.
//   The epilogue quantizes y from registers; y is never stored.
// Column labelling: output column c of n-tile nt is the real column R*c + nt (R = N/16),
// so after the last n-tile every lane holds R consecutive columns of 4 rows -- R/2 code
// bytes per row, and a 32-group spans 32/R neighbouring lanes.  At N = 16 (R = 1) a lane
// holds one column and the two lanes of a column pair form the pair's code byte together.
// An empty P2 ([0, 0]) is run as P2 = I: T = RNE(x * 1) = x exactly.
//
// The waves of a workgroup share P1/P2 fragments staged once in LDS in operand order (one
// 16-byte read per lane, conflict-free); the grid is persistent, each wave walking the
// slices wave_id, wave_id + total_waves, ...  The next slice's x is requested while the
// current slice's GEMM2 and epilogue run.
#include <hip/hip_runtime.h>

#include <atomic>

#include "fq_mfma_common.h"
#include "fq_mfma_pstage.h"

namespace fq {
namespace {

// One wave per SIMD (512 registers a wave): per-token slices above 4096 elements, per-group
// ones above 8192.
template <int M, int N, bool PG>
constexpr bool one_wave_per_simd() {
  return M * N > (PG ? 8192 : 4096);
}

// Slices of x kept in flight per wave: two for slices under 4096 elements (the loads of
// the slice two ahead are issued as soon as the current one's first product has consumed
// its registers) and where one wave runs per SIMD, one otherwise.  At 4096 elements one
// slice in flight in each of two waves per SIMD beats two slices in flight in one wave per
// SIMD by 4-5% (while one wave waits for its x the other computes); three slices in flight
// measured slower still (the extra slice every wave queues at the start delays every
// wave's first slice).
template <int M, int N, bool PG>
constexpr int prefetch_depth() {
  return (M * N < 4096 || one_wave_per_simd<M, N, PG>()) ? 2 : 1;
}

// Waves per workgroup: 8 from 4096 elements up (one workgroup per CU, so the CU stages
// its P fragments once: 6-9% faster at M=64, N=128 than two 4-wave workgroups), 4 for the
// small slices, which fill the CU with as many workgroups as fit.
template <int M, int N, bool PG>
constexpr int small_waves() {
  return prefetch_depth<M, N, PG>() == 1 ? 8 : 4;
}

// CLAMP (per token): the int4 or INT8 clamp is compiled in.  SV (per group): the e8m0 rule.  Q (per
// token): 0 for int4 codes, else the 8-bit mode (kPerTokenInt8 / E4M3 / E5M2), one byte a code.
// PAD: M and N are the padded sizes of a smaller slice (pb.M x pb.N; pb.N == N per group).
template <int DT, int M, int N, bool PG, bool CLAMP, int SV, int Q, bool PAD>
// (The second launch bound is HIP's minimum of waves per SIMD: 2 keeps the 4-wave variants
// to 256 registers, the budget they were written for, also where one wave per SIMD is
// launched; an 8-wave workgroup already puts two on each SIMD; the large per-token slices
// take 512.)
__global__ __launch_bounds__((64 * small_waves<M, N, PG>()),
                             ((small_waves<M, N, PG>() == 8 || one_wave_per_simd<M, N, PG>()) ? 1 : 2)) void mfma_small_kernel(
    Problem pb, Buffers b) {
  constexpr int kSmallWaves = small_waves<M, N, PG>();
  constexpr int kSmallThreads = 64 * kSmallWaves;
  constexpr int MT = M / 16, NT = N / 16, R = N / 16;
  constexpr int KS1 = (N + 31) / 32;       // GEMM1 k-steps over j (N = 16: one, half of it zeros)
  constexpr int KS2 = (M + 31) / 32;       // GEMM2 k-steps over m
  constexpr int MN = M * N;
  constexpr int SPAN = 32 / R;             // lanes per 32-group (per-group mode)
  static_assert(((N % 32 == 0 && R >= 2) || (N == 16 && !PG && Q == 0)) && M % 16 == 0, "unsupported shape");
  // the slice's own sizes (the template's with no padding)
  const int Mr = PAD ? static_cast<int>(pb.M) : M, Nr = PAD ? static_cast<int>(pb.N) : N;

  __shared__ u32x4_t frag2[KS1 * NT * 64];  // B fragments of P2 (or of I)
  __shared__ u32x4_t frag1[MT * KS2 * 64];  // A fragments of P1 (k relabelled)
  // per-wave staging of one slice's output: codes (M*N/2 bytes, M*N for 8-bit codes), then
  // e8m0 bytes
  constexpr int CODE_BYTES = Q ? MN : MN / 2;
  constexpr int E8_BYTES = PG ? MN / 32 : 0;
  constexpr int STAGE_BYTES = (CODE_BYTES + E8_BYTES + 15) / 16 * 16;
  __shared__ u32x4_t stage[kSmallWaves][STAGE_BYTES / 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;

  const int64_t waves = int64_t(gridDim.x) * kSmallWaves;
  // the slice index is wave-uniform: keep it (and every base pointer) in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t s = int64_t(blockIdx.x) * kSmallWaves + wave;

  // x operands of a slice: xa[buf][mt][ks] = x[16mt + c, 32ks + 8g .. +7]
  // The loads go through a buffer resource that covers exactly the requested slice, or
  // nothing when the index is at or past K: such a request returns zeros and touches no
  // memory.  The loads are therefore issued unconditionally, which keeps the count of
  // memory operations in flight the same on every path, so the compiler's waits for a
  // buffer cover that buffer's loads only and not the ones issued after them.
  // (a two-pass slice with 8-bit codes keeps one slice in flight: with two the kernel spills)
  constexpr int PF = (Q != 0 && !PG && MN > 8192) ? 1 : prefetch_depth<M, N, PG>();
  u32x4_t xa[PF][MT][KS1];
  // x's slice and row strides (M*N and N for a contiguous x; a strided x is read in place)
  const int64_t xs_k = pb.xs_k;
  const int xs_m = static_cast<int>(pb.xs_m);
  const int x_span = ((Mr - 1) * xs_m + Nr) * 2;  // bytes a slice spans
  auto load_x = [&](int buf, int64_t slice) {
    const bool in = slice < pb.K;
    if constexpr (PAD) {
      // A resource per row tile whose range ends with the slice's last row in it (none past
      // the slice's rows), so lanes on rows past it read zeros; columns past the slice's are
      // sent past every range.
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int rows = Mr - 16 * mt < 16 ? Mr - 16 * mt : 16;
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(b.x + (in ? slice : 0) * xs_k + int64_t(16 * mt) * xs_m), static_cast<int16_t>(0),
            (in && rows > 0) ? ((rows - 1) * xs_m + Nr) * 2 : 0, kBufferWord3);
#pragma unroll
        for (int ks = 0; ks < KS1; ++ks)
          xa[buf][mt][ks] = __builtin_amdgcn_raw_buffer_load_b128(
              rs, ((N >= 32 || 8 * g < N) && 32 * ks + 8 * g < Nr) ? (c * xs_m + 32 * ks + 8 * g) * 2 : 16 * xs_m * 2, 0,
              0);
      }
      return;
    }
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b.x + (in ? slice : 0) * xs_k),
                                                        static_cast<int16_t>(0), in ? x_span : 0, kBufferWord3);
    // row tile in the scalar offset, k-step in the immediate: one address register
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks)
        xa[buf][mt][ks] = __builtin_amdgcn_raw_buffer_load_b128(
            rsrc, (N >= 32 || 8 * g < N) ? (c * xs_m + 32 * ks + 8 * g) * 2 : x_span,  // past N: zeros
            16 * mt * xs_m * 2, 0);
  };
  // ---- stage P2 / P1 fragments (once per workgroup) ----
  // The P loads go first and the x loads of the first slices right after them, so the
  // staging waits for P alone (the memory counter completes in issue order) while x is
  // still arriving.
  {
    PStage<DT, M, N, kSmallThreads, PAD> ps;
    if constexpr (PF > 1) {
      ps.issue(pb, b, tid);
      __builtin_amdgcn_sched_barrier(0);  // keep the issue order: P, then x
      // With two slices in flight their loads are issued now, overlapping the staging,
      // in slice order (the loop's first wait is for the first slice).
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        load_x(q, s + q * waves);
        __builtin_amdgcn_sched_barrier(0);
      }
      ps.scatter(pb, frag2, frag1, tid);
    } else {
      // One slice in flight: P2 and P1 are staged one after the other and the first x
      // load waits for the slice loop (issuing it before the staging measured 4% slower
      // at 4096 elements: the staging then waits behind it).
      ps.issue_p2(pb, b, tid);
      ps.scatter_p2(pb, frag2, tid);
      ps.issue_p1(pb, b, tid);
      ps.scatter_p1(frag1, tid);
    }
  }
  lds_barrier();
  if (s >= pb.K) return;
  if constexpr (PF == 1) load_x(0, s);

  uint8_t* const st = reinterpret_cast<uint8_t*>(stage[wave]);
  // write the staged output of slice `slice` with 16-byte stores
  auto flush = [&](int64_t slice) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if constexpr (PAD) {
      // the slice's own codes, a multiple of 4 bytes (N is a multiple of 8)
      const int cb = Q ? Mr * Nr : Mr * Nr / 2;
      uint32_t* g32 = reinterpret_cast<uint32_t*>(b.codes + slice * cb);
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(st);
      for (int q = lane; q < cb / 4; q += 64) __builtin_nontemporal_store(s32[q], &g32[q]);
    } else {
      u32x4_t* gcodes = reinterpret_cast<u32x4_t*>(b.codes + slice * CODE_BYTES);
#pragma unroll
      // the codes are written once and not read back by this kernel: non-temporal stores
      for (int q = 0; q < CODE_BYTES / 16 / 64; ++q) __builtin_nontemporal_store(stage[wave][q * 64 + lane], &gcodes[q * 64 + lane]);
      if constexpr ((CODE_BYTES / 16) % 64 != 0) {
        constexpr int q = CODE_BYTES / 16 / 64;
        if (q * 64 + lane < CODE_BYTES / 16) __builtin_nontemporal_store(stage[wave][q * 64 + lane], &gcodes[q * 64 + lane]);
      }
    }
    if constexpr (PG && PAD) {
      // the slice's e8m0 bytes and, after an odd count of groups, the zero pad byte
      const int cb = Mr * Nr / 2, groups = Mr * Nr / 32, e8b = static_cast<int>(e8m0_bytes_per_slice(Mr * Nr));
      uint8_t* ge = static_cast<uint8_t*>(b.scale) + slice * e8b;
      for (int q = lane; q < e8b; q += 64) ge[q] = q < groups ? st[cb + q] : uint8_t(0);
    } else if constexpr (PG) {
      const uint32_t* se = reinterpret_cast<const uint32_t*>(st + CODE_BYTES);
      uint32_t* ge = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(b.scale) +
                                                 slice * e8m0_bytes_per_slice(MN));
      for (int q = lane; q < E8_BYTES / 4; q += 64) __builtin_nontemporal_store(se[q], &ge[q]);
    }
    // the staging buffer is reused by the next slice
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  auto process = [&](const int buf, const int64_t s) {
    // Keep the P fragments in LDS: without this the compiler hoists the loop-invariant
    // fragment reads into registers, which costs occupancy.
    asm volatile("" ::: "memory");
    // The lane's offsets into the staging buffer (codes of row 4g, column group R*c; its
    // e8m0 byte).  Made opaque per slice so the per-row addresses are formed here, with
    // the row as an immediate offset, instead of being hoisted out of the slice loop and
    // held in registers.
    // (codes staged as the slice's own rows: NROW elements a row)
    const int NROW = PAD ? Nr : N;
    int code_off = Q ? 4 * g * NROW + R * c : 4 * g * (NROW / 2) + (R >= 2 ? (R / 2) * c : c / 2);
    // the slice's own code bytes (the e8m0 bytes are staged after them)
    const int CB = PAD ? (Q ? Mr * Nr : Mr * Nr / 2) : CODE_BYTES;
    int e8_off = CB + 4 * g * (N / 32) + (R * c) / 32;
    asm volatile("" : "+v"(code_off), "+v"(e8_off));
    // ---- GEMM1: T = x . P2 (fp32), rounded to the dtype and written straight into the
    // GEMM2 B operands: bt[ks2][nt] = {T rows 32ks2 + 4g + 0..3, T rows 32ks2 + 16 + 4g + 0..3}
    // of column R*c + nt (2 x 16 bit per dword).
    u32x4_t bt[KS2][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4_t acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks) {
        // bound the fragment reads in flight to one k-step (register pressure)
        if constexpr (KS1 * NT > 8) asm volatile("" ::: "memory");
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = mfma16x16x32<DT>(xa[buf][mt][ks], frag2[(ks * NT + nt) * 64 + lane], acc[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int h = 2 * (mt & 1);
        bt[mt >> 1][nt][h] = round16x2<DT>(acc[nt][0], acc[nt][1]);
        bt[mt >> 1][nt][h + 1] = round16x2<DT>(acc[nt][2], acc[nt][3]);
        if (MT == 1) {  // M = 16: the second half of the k-step is empty
          bt[0][nt][2] = 0u;
          bt[0][nt][3] = 0u;
        }
      }
    }
    // this buffer is free again: request the slice PF steps ahead
    load_x(buf, s + PF * waves);

    if constexpr (!PG) {
      // The codes of 16-row tile it of y (yt: its NT accumulator tiles), inv = 1 / scale.
      auto encode_tile = [&](const int it, const f32x4_t* yt, const float inv) {
        if constexpr (Q != 0) {
          // 8-bit codes (the dequant_swiglu_quant page, section 3.4): the lane's R codes of a
          // row are R consecutive bytes
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r0 = 16 * it + i;  // row - 4g
            uint32_t w[(R + 3) / 4];
            if constexpr (R == 2) {
              w[0] = code8x2<Q>(yt[0][i] * inv, yt[1][i] * inv);
            } else {
#pragma unroll
              for (int q = 0; q < R / 4; ++q)
                w[q] = code8x4<Q, CLAMP>(yt[4 * q][i], yt[4 * q + 1][i], yt[4 * q + 2][i],
                                         yt[4 * q + 3][i], inv);
            }
            uint8_t* dst = st + code_off + r0 * NROW;
            if (!PAD || (r0 + 4 * g < Mr && R * c < Nr)) {  // the slice's own rows and columns
              if constexpr (R == 2) {
                *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(w[0]);
              } else {
#pragma unroll
                for (int q = 0; q < R / 4; ++q) reinterpret_cast<uint32_t*>(dst)[q] = w[q];
              }
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r0 = 16 * it + i;  // row - 4g
            uint32_t by[R >= 2 ? R / 2 : 1];
            if constexpr (R == 1) {
              // columns c and c ^ 1 (lane c ^ 1 holds the other): both lanes form the same byte
              const uint32_t own = int4_biased<CLAMP>(yt[0][i], inv);
              const uint32_t nbr = dpp_u<kDppQuadXor1>(own);
              by[0] = (c & 1) ? pair_byte(nbr, own) : pair_byte(own, nbr);
            } else {
#pragma unroll
              for (int p = 0; p < R / 2; ++p)
                by[p] = pair_byte(int4_biased<CLAMP>(yt[2 * p][i], inv),
                                  int4_biased<CLAMP>(yt[2 * p + 1][i], inv));
            }
            uint8_t* dst = st + code_off + r0 * (NROW / 2);
            if (!PAD || (r0 + 4 * g < Mr && R * c < Nr)) {  // the slice's own rows and columns
              if constexpr (R <= 2) {
                *dst = static_cast<uint8_t>(by[0] ^ 0x88u);
              } else if constexpr (R == 4) {
                *reinterpret_cast<uint16_t*>(dst) =
                    static_cast<uint16_t>(unbias(__builtin_amdgcn_perm(by[1], by[0], 0x0C0C0400u)));
              } else {
                *reinterpret_cast<uint32_t*>(dst) = unbias(gather4(by[0], by[1], by[2], by[3]));
              }
            }
          }
        }
      };
      if constexpr (MN <= 8192) {
        // ---- GEMM2: y = P1 . T, all of y (the scale needs max|y| over the slice) ----
        f32x4_t y[MT][NT];
#pragma unroll
        for (int it = 0; it < MT; ++it)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) y[it][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2)
#pragma unroll
          for (int it = 0; it < MT; ++it) {
            const u32x4_t a = frag1[(it * KS2 + ks2) * 64 + lane];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) y[it][nt] = mfma16x16x32<DT>(a, bt[ks2][nt], y[it][nt]);
          }
        // [FQV2] 第3步 pertoken: scale = max|y| / (7/clipRatio); code = RNE(y / scale)
        float amax = 0.0f;
#pragma unroll
        for (int it = 0; it < MT; ++it)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) amax = fmaxf(amax, __builtin_fabsf(y[it][nt][i]));
        amax = wave_max(amax);
        // (every lane holds the same maximum; the scale is made wave-uniform so the branch
        // below is a scalar one)
        const float scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(amax / pb.d)));
        const TokenRecip rc = token_recip(scale);
        if (rc.tiny) {
          // a scale below 2^-126: y * 2^64 exactly, and inv = 1 / (scale * 2^64)
#pragma unroll
          for (int it = 0; it < MT; ++it)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) y[it][nt] *= rc.pre;
        }
        if (lane == 0) static_cast<float*>(b.scale)[s] = scale;
#pragma unroll
        for (int it = 0; it < MT; ++it) encode_tile(it, y[it], rc.inv);
      } else {
        // Above 8192 elements all of y does not fit the registers: GEMM2 runs twice, one
        // 16-row tile at a time, first for max|y| (the scale), then for the codes.
        auto gemm2_tile = [&](const int it, f32x4_t* yt) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) yt[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks2 = 0; ks2 < KS2; ++ks2) {
            const u32x4_t a = frag1[(it * KS2 + ks2) * 64 + lane];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) yt[nt] = mfma16x16x32<DT>(a, bt[ks2][nt], yt[nt]);
          }
        };
        // [FQV2] 第3步 pertoken: scale = max|y| / (7/clipRatio); code = RNE(y / scale)
        float amax = 0.0f;
#pragma unroll
        for (int it = 0; it < MT; ++it) {
          asm volatile("" ::: "memory");  // one row tile live at a time
          f32x4_t yt[NT];
          gemm2_tile(it, yt);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) amax = fmaxf(amax, __builtin_fabsf(yt[nt][i]));
        }
        amax = wave_max(amax);
        const float scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(amax / pb.d)));
        const TokenRecip rc = token_recip(scale);
        if (lane == 0) static_cast<float*>(b.scale)[s] = scale;
#pragma unroll
        for (int it = 0; it < MT; ++it) {
          asm volatile("" ::: "memory");
          f32x4_t yt[NT];
          gemm2_tile(it, yt);  // the same products in the same order: the same y
          if (rc.tiny) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) yt[nt] *= rc.pre;
          }
          encode_tile(it, yt, rc.inv);
        }
      }
    } else {
      // [FQV2] 第3步 pergroup / 第4步: one e8m0 scale per 32 consecutive elements of a row.
      // GEMM2 and the encoding run one 16-row tile at a time.
#pragma unroll
      for (int it = 0; it < MT; ++it) {
        if constexpr (MT * NT > 16) asm volatile("" ::: "memory");  // one row tile live at a time
        f32x4_t y[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) y[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2) {
          const u32x4_t a = frag1[(it * KS2 + ks2) * 64 + lane];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) y[nt] = mfma16x16x32<DT>(a, bt[ks2][nt], y[nt]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 16 * it + i;  // row - 4g
          float amax = 0.0f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) amax = fmaxf(amax, __builtin_fabsf(y[nt][i]));
          amax = group_max<SPAN>(amax);
          const uint32_t code = e8m0_code_v<SV>(amax, pb.dmax, pb.dmax_inv);
          const float sc = e8m0_to_float(code);
          uint32_t packed = 0;
          packed = fp4x2<0>(packed, y[0][i], y[1][i], sc);
          if constexpr (R >= 4) packed = fp4x2<1>(packed, y[2][i], y[3][i], sc);
          if constexpr (R >= 8) {
            packed = fp4x2<2>(packed, y[4][i], y[5][i], sc);
            packed = fp4x2<3>(packed, y[6][i], y[7][i], sc);
          }
          uint8_t* dst = st + code_off + r0 * (N / 2);
          if (!PAD || r0 + 4 * g < Mr) {  // the slice's own rows
            if constexpr (R == 2) {
              *dst = static_cast<uint8_t>(packed);
            } else if constexpr (R == 4) {
              *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(packed);
            } else {
              *reinterpret_cast<uint32_t*>(dst) = packed;
            }
            // Group index (row*N + R*c)/32.  Every lane of a group holds the same code, so
            // all of them store it (no branch).
            st[e8_off + r0 * (N / 32)] = static_cast<uint8_t>(code);
          }
        }
      }
      // (M*N/32 is even for every shape of the template sizes; with PAD the flush writes
      // the pad byte of an odd count of groups)
    }
    flush(s);
  };

  // PF slices per iteration, then the last few: no exit from the middle of the loop body
  for (; s + (PF - 1) * waves < pb.K; s += PF * waves) {
#pragma unroll
    for (int q = 0; q < PF; ++q) process(q, s + q * waves);
  }
#pragma unroll
  for (int q = 0; q + 1 < PF; ++q)
    if (s + q * waves < pb.K) process(q, s + q * waves);
}

template <int DT, int M, int N, bool PG, bool CLAMP, int SV, int Q = 0, bool PAD = false>
hipError_t launch_one(const Problem& pb, const Buffers& b, hipStream_t s) {
  constexpr int kWaves = small_waves<M, N, PG>(), kThreads = 64 * kWaves;
  // workgroups that fit the device at once (per instantiation); first calls from several
  // threads may race here, and each stores the same value
  static std::atomic<int> grid_cap_cache{0};
  int grid_cap = grid_cap_cache.load(std::memory_order_relaxed);
  if (grid_cap == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mfma_small_kernel<DT, M, N, PG, CLAMP, SV, Q, PAD>,
                                                       kThreads, 0);
    if (e != hipSuccess) return e;
    grid_cap = cus * (per_cu > 0 ? per_cu : 1);
    grid_cap_cache.store(grid_cap, std::memory_order_relaxed);
  }
  const int64_t need = (pb.K + kWaves - 1) / kWaves;
  const int grid = static_cast<int>(need < grid_cap ? need : grid_cap);
  mfma_small_kernel<DT, M, N, PG, CLAMP, SV, Q, PAD><<<grid, kThreads, 0, s>>>(pb, b);
  return hipGetLastError();
}

// int4 per-token codes (INT32 / INT4 out)
template <int DT, int M, int N, bool PAD>
hipError_t dispatch_int4(const Problem& pb, const Buffers& b, hipStream_t s) {
  // The int4 clamp can only bite when (7/clipRatio) * (1 + 4 ulp) reaches 7.5.
  if (pb.d >= 7.4999f) return launch_one<DT, M, N, false, true, kE8V1, 0, PAD>(pb, b, s);
  return launch_one<DT, M, N, false, false, kE8V1, 0, PAD>(pb, b, s);
}

template <int DT, int M, int N, bool PG, bool PAD>
hipError_t dispatch_clamp(const Problem& pb, const Buffers& b, hipStream_t s) {
  if constexpr (PG) {
    switch (e8m0_variant(pb)) {
      case kE8V1: return launch_one<DT, M, N, true, false, kE8V1, 0, PAD>(pb, b, s);
      case kE8V2Pow2: return launch_one<DT, M, N, true, false, kE8V2Pow2, 0, PAD>(pb, b, s);
      default: return launch_one<DT, M, N, true, false, kE8V2Div, 0, PAD>(pb, b, s);
    }
  } else {
    switch (pb.mode) {
      case kPerTokenInt8:
        // The INT8 clamp can only bite when (127/clipRatio) * (1 + 4 ulp) reaches 127.5.
        if (pb.d >= 127.4999f) return launch_one<DT, M, N, false, true, kE8V1, kPerTokenInt8, PAD>(pb, b, s);
        return launch_one<DT, M, N, false, false, kE8V1, kPerTokenInt8, PAD>(pb, b, s);
      case kPerTokenE4M3: return launch_one<DT, M, N, false, false, kE8V1, kPerTokenE4M3, PAD>(pb, b, s);
      case kPerTokenE5M2: return launch_one<DT, M, N, false, false, kE8V1, kPerTokenE5M2, PAD>(pb, b, s);
      default: break;
    }
    return dispatch_int4<DT, M, N, PAD>(pb, b, s);
  }
}

template <int DT, int M, int N, bool PAD>
hipError_t dispatch_mode(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (pb.mode == kPerGroupFp4) return dispatch_clamp<DT, M, N, true, PAD>(pb, b, s);
  return dispatch_clamp<DT, M, N, false, PAD>(pb, b, s);
}

bool int4_codes(const Problem& pb) { return pb.mode == kPerTokenInt32 || pb.mode == kPerTokenInt4; }

// The sizes an instantiation is chosen by: the slice's own, or with padding the next of
// 16, 32, 64, 128 (N from 32 for the 8-bit codes, whose layout needs two columns a lane;
// N unpadded per group).
int pad_up(int v) { return v <= 16 ? 16 : v <= 32 ? 32 : v <= 64 ? 64 : 128; }
int padded_m(const Problem& pb) { return pad_up(static_cast<int>(pb.M)); }
int padded_n(const Problem& pb) {
  if (pb.mode == kPerGroupFp4) return static_cast<int>(pb.N);
  const int n = pad_up(static_cast<int>(pb.N));
  return (n == 16 && !int4_codes(pb)) ? 32 : n;
}

template <int DT, int M, bool PAD>
hipError_t dispatch_n(const Problem& pb, const Buffers& b, hipStream_t s) {
  switch (PAD ? padded_n(pb) : static_cast<int>(pb.N)) {
    case 16:
      if (int4_codes(pb)) return dispatch_int4<DT, M, 16, PAD>(pb, b, s);
      break;
    case 32: return dispatch_mode<DT, M, 32, PAD>(pb, b, s);
    case 64: return dispatch_mode<DT, M, 64, PAD>(pb, b, s);
    case 128: return dispatch_mode<DT, M, 128, PAD>(pb, b, s);
  }
  return hipErrorNotSupported;
}

template <int DT, bool PAD>
hipError_t dispatch_m(const Problem& pb, const Buffers& b, hipStream_t s) {
  switch (PAD ? padded_m(pb) : static_cast<int>(pb.M)) {
    case 16: return dispatch_n<DT, 16, PAD>(pb, b, s);
    case 32: return dispatch_n<DT, 32, PAD>(pb, b, s);
    case 64: return dispatch_n<DT, 64, PAD>(pb, b, s);
    case 128: return dispatch_n<DT, 128, PAD>(pb, b, s);
  }
  return hipErrorNotSupported;
}

// Runs at the slice's own sizes (no padding).
bool exact_shape(const Problem& pb) {
  const bool m_ok = pb.M == 16 || pb.M == 32 || pb.M == 64 || pb.M == 128;
  // N = 16: int4 per-token codes only (one code a lane per row: the 8-bit and per-group
  // layouts are not implemented for it)
  const bool n_ok = pb.N == 32 || pb.N == 64 || pb.N == 128 || (pb.N == 16 && int4_codes(pb));
  return m_ok && n_ok;
}

// Runs padded: per token, M and N up to 128, N a multiple of 8; per group, M up to 128 and
// N one of 32, 64, 128.
bool padded_shape(const Problem& pb) {
  if (pb.M < 1 || pb.M > 128) return false;
  if (pb.mode == kPerGroupFp4) return pb.N == 32 || pb.N == 64 || pb.N == 128;
  return pb.N >= 8 && pb.N <= 128 && pb.N % 8 == 0;
}

}  // namespace

bool mfma_small_supports(const Problem& pb) { return exact_shape(pb) || padded_shape(pb); }

hipError_t launch_mfma_small(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (exact_shape(pb)) return pb.dtype == kBF16 ? dispatch_m<kBF16, false>(pb, b, s) : dispatch_m<kF16, false>(pb, b, s);
  if (padded_shape(pb)) return pb.dtype == kBF16 ? dispatch_m<kBF16, true>(pb, b, s) : dispatch_m<kF16, true>(pb, b, s);
  return hipErrorNotSupported;
}

}  // namespace fq
