// Staging of the transforms as MFMA fragments in LDS, shared by the small-slice kernels.
//
//   P2[j, n]  -> frag2[(ks*NT + nt)*64 + 16*g + c], element t   (j = 32ks + 8g + t, n = R*c + nt)
//   P1[i, m]  -> frag1[(it*KS2 + ks2)*64 + 16*g + i%16], element t, where m = 32ks2 + w and
//                w = 4g + t (t < 4) or 16 + 4g + (t - 4) (t >= 4)
//
// P2's layout makes it GEMM1's B operand with output column R*c + nt in lane c of n-tile
// nt; P1's relabels the contraction index m so that GEMM1's accumulator registers are
// GEMM2's B operand as they stand (a lane's two 4-row accumulator blocks are its 8
// k-slots).  An empty P2 ([0, 0]) is staged as the identity.
#pragma once

#include "fq_mfma_common.h"

namespace fq {

template <int DT, int M, int N, int THREADS>
struct PStage {
  static constexpr int MT = M / 16, NT = N / 16, R = N / 16, KS1 = N / 32, KS2 = (M + 31) / 32;
  static constexpr int C2 = N * N / 8, C1 = M * M / 8;  // 16-byte chunks of P2 and P1
  static constexpr int L2 = (C2 + THREADS - 1) / THREADS;
  static constexpr int L1 = (C1 + THREADS - 1) / THREADS;
  static constexpr int FRAG2 = KS1 * NT * 64, FRAG1 = MT * KS2 * 64;  // u32x4 slots
  u32x4_t r2[L2], r1[L1];

  // All coalesced 16-byte loads of P1 and P2 (one memory latency).  Chunks past the end
  // (or all of P2 when it is empty) read zeros through bounded buffer resources, so no
  // load is conditional.
  __device__ __forceinline__ void issue(const Problem& pb, const Buffers& b, int tid) {
    const bool two = pb.two_sided != 0;
    const auto rs2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(two ? b.p2 : b.p1),
                                                      static_cast<int16_t>(0), two ? N * N * 2 : 0, kBufferWord3);
    const auto rs1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b.p1), static_cast<int16_t>(0),
                                                      M * M * 2, kBufferWord3);
#pragma unroll
    for (int q = 0; q < L2; ++q) r2[q] = __builtin_amdgcn_raw_buffer_load_b128(rs2, (tid + q * THREADS) * 16, 0, 0);
#pragma unroll
    for (int q = 0; q < L1; ++q) r1[q] = __builtin_amdgcn_raw_buffer_load_b128(rs1, (tid + q * THREADS) * 16, 0, 0);
  }

  // Each 2-byte value to its fragment slot; the caller puts a barrier after this.
  __device__ __forceinline__ void scatter(const Problem& pb, u32x4_t* frag2, u32x4_t* frag1, int tid) {
    uint16_t* f2 = reinterpret_cast<uint16_t*>(frag2);
    uint16_t* f1 = reinterpret_cast<uint16_t*>(frag1);
    if (pb.two_sided != 0) {
#pragma unroll
      for (int q = 0; q < L2; ++q) {
        const int ch = tid + q * THREADS;
        if (ch < C2) {
          const int j = ch / (N / 8), n0 = (ch % (N / 8)) * 8;
          const int ks = j >> 5, gg = (j >> 3) & 3, t = j & 7;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int n = n0 + e, cc = n / R, nt = n % R;
            f2[((ks * NT + nt) * 64 + 16 * gg + cc) * 8 + t] = static_cast<uint16_t>(r2[q][e >> 1] >> (16 * (e & 1)));
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
    // P1 columns beyond M (M = 16: the second half of the k-step) hold zeros
    if (M < 32) {
      for (int idx = tid; idx < FRAG1; idx += THREADS) frag1[idx] = u32x4_t{0u, 0u, 0u, 0u};
      lds_barrier();
    }
#pragma unroll
    for (int q = 0; q < L1; ++q) {
      const int ch = tid + q * THREADS;
      if (ch < C1) {
        const int i = ch / (M / 8), m0 = (ch % (M / 8)) * 8;
        const int it = i >> 4, r = i & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = m0 + e, ks2 = m >> 5, w = m & 31;
          const int gg = w < 16 ? (w >> 2) : ((w - 16) >> 2);
          const int t = w < 16 ? (w & 3) : 4 + ((w - 16) & 3);
          f1[((it * KS2 + ks2) * 64 + 16 * gg + r) * 8 + t] = static_cast<uint16_t>(r1[q][e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
};

}  // namespace fq
