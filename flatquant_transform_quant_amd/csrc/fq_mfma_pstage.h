// Staging of the transforms as MFMA fragments in LDS, shared by the small-slice kernels.
//
//   P2[j, n]  -> frag2[(ks*NT + nt)*64 + 16*g + c], element t   (j = 32ks + 8g + t, n = R*c + nt)
//   P1[i, m]  -> frag1[(it*KS2 + ks2)*64 + 16*g + i%16], element t, where m = 32ks2 + w and
//                w = 4g + t (t < 4) or 16 + 4g + (t - 4) (t >= 4); columns past M are zero
//
// With PAD the transforms are smaller than the fragments (M x M and N x N are the padded
// sizes, the problem's own are pb.M and pb.N, N a multiple of 8): rows and columns past
// them are zero, so the padded products equal the real ones on the real rows and columns.
//
// P2's layout makes it GEMM1's B operand with output column R*c + nt in lane c of n-tile
// nt; P1's relabels the contraction index m so that GEMM1's accumulator registers are
// GEMM2's B operand as they stand (a lane's two 4-row accumulator blocks are its 8
// k-slots).  An empty P2 ([0, 0]) is staged as the identity.
#pragma once

#include "fq_mfma_common.h"

namespace fq {

template <int DT, int M, int N, int THREADS, bool PAD = false>
struct PStage {
  static constexpr int MT = M / 16, NT = N / 16, R = N / 16, KS1 = (N + 31) / 32, KS2 = (M + 31) / 32;
  static constexpr int FRAG2 = KS1 * NT * 64, FRAG1 = MT * KS2 * 64;  // u32x4 slots
  // P2 goes by 8x8 blocks (rows 32ks + 8g .. +7, columns 8cb .. 8cb+7): one thread loads
  // the block's 8 rows (16 bytes each), pairs the rows of each column with v_perm_b32 and
  // writes the 8 columns as 8 whole fragments.
  static constexpr int B2 = (N / 8) * (N / 8);          // blocks of P2
  static constexpr int L2 = (B2 + THREADS - 1) / THREADS;
  // A P1 fragment is two 8-byte pieces of one row of P1 (its 8 relabelled k-slots are
  // columns 32ks2 + 4g .. +3 and 32ks2 + 16 + 4g .. +3).
  static constexpr int L1 = (FRAG1 + THREADS - 1) / THREADS;
  u32x4_t r2[L2][8];
  uint32_t r1[L1][4];

  // The loads (one memory latency each for P2 and P1).  Loads past the end of P1/P2 (or
  // all of P2 when it is empty) read zeros through bounded buffer resources, so no load
  // is conditional.
  __device__ __forceinline__ void issue(const Problem& pb, const Buffers& b, int tid) {
    issue_p2(pb, b, tid);
    issue_p1(pb, b, tid);
  }
  __device__ __forceinline__ void issue_p2(const Problem& pb, const Buffers& b, int tid) {
    // the staging's own copy of the thread index: its lane arithmetic is not shared with
    // (and kept live for) the kernel's slice loop
    asm volatile("" : "+v"(tid));
    const bool two = pb.two_sided != 0;
    const int Nr = PAD ? static_cast<int>(pb.N) : N;  // P2's own size (a multiple of 8 with PAD)
    const auto rs2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(two ? b.p2 : b.p1),
                                                      static_cast<int16_t>(0), two ? Nr * Nr * 2 : 0, kBufferWord3);
#pragma unroll
    for (int q = 0; q < L2; ++q) {
      const int blk = tid + q * THREADS;
      const int rb = blk / (N / 8), cb = blk % (N / 8);  // rows 8rb .. +7, columns 8cb .. +7
      const bool in = blk < B2 && (!PAD || (8 * rb < Nr && 8 * cb < Nr));
      const int off = in ? ((8 * rb) * Nr + 8 * cb) * 2 : Nr * Nr * 2;  // past the end: zeros
#pragma unroll
      for (int t = 0; t < 8; ++t) r2[q][t] = __builtin_amdgcn_raw_buffer_load_b128(rs2, off + t * Nr * 2, 0, 0);
    }
  }
  __device__ __forceinline__ void issue_p1(const Problem& pb, const Buffers& b, int tid) {
    asm volatile("" : "+v"(tid));
    if constexpr (PAD) {
      // element by element (P1's own size need not be a multiple of 4); zeros past it
      const int Mr = static_cast<int>(pb.M);
      const auto rs1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b.p1), static_cast<int16_t>(0),
                                                        Mr * Mr * 2, kBufferWord3);
#pragma unroll
      for (int q = 0; q < L1; ++q) {
        const int slot = tid + q * THREADS;
        const int l = slot & 63, f = slot >> 6, it = f / KS2, ks2 = f % KS2;
        const int i = 16 * it + (l & 15), gg = l >> 4;
        uint32_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int m = 32 * ks2 + (t < 4 ? 4 * gg + t : 16 + 4 * gg + (t - 4));
          const bool in = slot < FRAG1 && i < Mr && m < Mr;
          e[t] = __builtin_amdgcn_raw_buffer_load_b16(rs1, in ? (i * Mr + m) * 2 : Mr * Mr * 2, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) r1[q][p] = e[2 * p] | (e[2 * p + 1] << 16);
      }
      return;
    }
    const auto rs1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b.p1), static_cast<int16_t>(0),
                                                      M * M * 2, kBufferWord3);
#pragma unroll
    for (int q = 0; q < L1; ++q) {
      const int slot = tid + q * THREADS;
      const int l = slot & 63, f = slot >> 6, it = f / KS2, ks2 = f % KS2;
      const int i = 16 * it + (l & 15), gg = l >> 4;
      const int m0 = 32 * ks2 + 4 * gg, m1 = m0 + 16;
      const bool in = slot < FRAG1;
      const int o0 = in ? (i * M + m0) * 2 : M * M * 2;
      const int o1 = (in && m1 < M) ? (i * M + m1) * 2 : M * M * 2;  // columns past M are zero
      const auto v0 = __builtin_amdgcn_raw_buffer_load_b64(rs1, o0, 0, 0);
      const auto v1 = __builtin_amdgcn_raw_buffer_load_b64(rs1, o1, 0, 0);
      r1[q][0] = v0[0];
      r1[q][1] = v0[1];
      r1[q][2] = v1[0];
      r1[q][3] = v1[1];
    }
  }

  // Fragments to LDS; the caller puts a barrier after this.
  __device__ __forceinline__ void scatter(const Problem& pb, u32x4_t* frag2, u32x4_t* frag1, int tid) {
    scatter_p2(pb, frag2, tid);
    scatter_p1(frag1, tid);
  }
  __device__ __forceinline__ void scatter_p2(const Problem& pb, u32x4_t* frag2, int tid) {
    asm volatile("" : "+v"(tid));
    if (pb.two_sided != 0) {
      if constexpr (N < 32) {
        // N = 16: the k-slots 16 .. 31 of the padded contraction (lane groups 2 and 3) are zero
        for (int idx = tid; idx < FRAG2; idx += THREADS)
          if (((idx & 63) >> 4) >= N / 8) frag2[idx] = u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < L2; ++q) {
        const int blk = tid + q * THREADS;
        if (blk < B2) {
          const int rb = blk / (N / 8), cb = blk % (N / 8);
          const int ks = rb >> 2, gg = rb & 3;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t v;
#pragma unroll
            for (int p = 0; p < 4; ++p) v[p] = __builtin_amdgcn_perm(r2[q][2 * p + 1][e >> 1], r2[q][2 * p][e >> 1], sel);
            const int n = 8 * cb + e, cc = n / R, nt = n % R;
            frag2[(ks * NT + nt) * 64 + 16 * gg + cc] = v;
          }
        }
      }
    } else {
      // an empty P2 is run as the identity
      const uint16_t one = DT == kBF16 ? uint16_t(0x3F80) : uint16_t(0x3C00);
      for (int idx = tid; idx < FRAG2; idx += THREADS) {
        const int l = idx & 63, f = idx >> 6, ks = f / NT, nt = f % NT;
        const int n = R * (l & 15) + nt, j0 = 32 * ks + 8 * (l >> 4);
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          w[p] = uint32_t(j0 + 2 * p == n ? one : 0) | (uint32_t(j0 + 2 * p + 1 == n ? one : 0) << 16);
        frag2[idx] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    }
  }
  __device__ __forceinline__ void scatter_p1(u32x4_t* frag1, int tid) {
    asm volatile("" : "+v"(tid));
#pragma unroll
    for (int q = 0; q < L1; ++q) {
      const int slot = tid + q * THREADS;
      if (slot < FRAG1) frag1[slot] = u32x4_t{r1[q][0], r1[q][1], r1[q][2], r1[q][3]};
    }
  }
};

}  // namespace fq
