// Streaming MFMA kernel for 256 x 256 slices with the left transform only (P2 empty) and
// per-group E2M1 codes.
//
// [FQV2] 拆开算 第1步 (y = P1 . x) fused with 第3步 / 第4步 (pergroup: e8m0 scale of each
// 32-group, E2M1 codes) for M = N = 256 and an empty P2.  One workgroup of 4 waves per CU
// (one wave per SIMD, 512 registers each), persistent over the slices:
//   * the product is taken transposed, y^T = x^T . P1^T.  Wave w owns y rows 64w .. 64w+63;
//     P1's rows 64w .. 64w+63 are the second MFMA operand (P1^T), held in 128 registers for
//     the whole launch, so LDS holds nothing but x;
//   * x streams through a ring of ten 16 KB chunks of 32 rows (all 160 KB of LDS), filled
//     by LDS-DMA loads (buffer_load ... lds: memory to LDS without registers), so nine chunks
//     are in flight per CU while one is consumed;
//   * the first operand (x^T: k = x's row) is read from the ring with gfx950's transposing
//     16-bit LDS read, ds_read_b64_tr_b16: in each 16-lane group, lanes 4j .. 4j+3 fetch 16
//     values of row j (8 bytes each) and lane i receives the four values of column i.  Two
//     such reads give a lane its eight k-slots;
//   * y (64 rows x 256 columns a wave, fp32) lives in the 256 accumulation registers.  The
//     x columns are labelled so that lane l ends with the 64 columns of two whole 32-groups
//     of each of its rows: the group max needs no cross-lane step, and a group's 16 code
//     bytes leave in one 16-byte store.
// Column labels.  Column tile ct (0..15) reads, in lane group G's four runs q = 0..3 (4
// columns each), the 4-column unit u(ct, q) = 8 (q + 4 (ct >> 3)) + ((ct & 7) ^ (q & 1)).
// An accumulator lane l holds C rows 4 (l >> 4) .. +3, i.e. run q = l >> 4, so its columns
// are 4 u(ct, l >> 4) + 0..3: for ct = 0..7 group l >> 4, for ct = 8..15 group 4 + (l >> 4).
// The (q & 1) term alternates the 8-byte half a run sits in, which with the ring's XOR
// layout below makes every transposing read free of bank conflicts.
// Ring layout.  A chunk's 16-byte piece pi (columns 8 pi .. +7) of row rho is stored at
// slot 32 rho + (pi ^ x), x = (rho & 3) | (((pi >> 3) & 1) ^ g) << 2 | g << 3 with
// g = (rho >> 3) & 1: each DMA load writes 1 KB of consecutive slots (lane l at +16 l) and
// takes its sources in that order.  The LDS serves the 8-byte reads of 32 lanes a cycle
// from 64 banks; under this layout the 32 lanes of every transposing read hit 32 distinct
// 8-byte bank pairs (rows 8 apart, which would share banks, differ in g).
// Memory counter.  The DMA loads are written in inline assembly, so the compiler neither
// sees them nor adds its conservative wait (the memory counter drained before every LDS
// read); the kernel waits for each chunk itself with a count of the memory operations
// issued after it (the DMA loads of the chunks ahead, and an epilogue's stores).
#include <hip/hip_runtime.h>

#include <atomic>

#include <type_traits>

#include "fq_mfma_common.h"

namespace fq {
namespace {

constexpr int kW = 256;                     // M = N
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;                  // rows of x per chunk (one k-step)
constexpr int kNChunk = kW / kChunk;        // chunks per slice
constexpr int kChunkB = kChunk * kW * 2;    // 16 KB
constexpr int kRing = 10;                   // chunks in LDS
constexpr int kDmaPerWave = kChunkB / 1024 / kWaves;  // 1 KB DMA loads per wave and chunk
constexpr int kStoresPerSlice = 12;         // memory stores of a wave's epilogue
constexpr int kSliceB = kW * kW * 2;
constexpr int kAhead = 4;                   // first-operand fragments read ahead of their products

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

// Buffer resource (as four scalar registers) over `bytes` bytes from p; 0 bytes: every
// access is out of range (a load returns zeros and touches no memory).
__device__ __forceinline__ i32x4 rsrc4(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4{static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFF),
               static_cast<int>(bytes), kBufferWord3};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One LDS-DMA load: lane l's 16 bytes at rsrc + voff + soff go to LDS lds + 16 l.
__device__ __forceinline__ void dma16(uint32_t lds, int voff, i32x4 rs, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N memory operations of this wave are outstanding and its LDS reads
// are done, then the workgroup barrier.  No compiler fence: one on LDS would also wait
// for every DMA load in flight.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N <= 63, "memory counter range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ u32x4_t tr_frag(const lds_u8* p0, const lds_u8* p1) {
  const bf16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
  const bf16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1);
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a), ub = __builtin_bit_cast(u32x2_t, b);
  return u32x4_t{ua[0], ua[1], ub[0], ub[1]};
}

template <int DT, int SV>
__global__ __launch_bounds__(kThreads, 1) void mfma_wide1s_kernel(Problem pb, Buffers b) {
  __shared__ __align__(16) uint8_t ring[kRing * kChunkB];
  lds_u8* const ring_l = (lds_u8*)ring;
  const uint32_t ring_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring_l));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, qc = lane >> 4;  // accumulator roles: y row 16 it + r16, run qc
  const int64_t K = pb.K, stride = gridDim.x;
  int64_t s = blockIdx.x;
  if (s >= K) return;

  // P1 rows 64w + 16 it + r16 as second operands: k-step ks, k-slots 8 (lane >> 4) .. +7
  u32x4_t pf[4][kNChunk];
  {
    const auto rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b.p1), static_cast<int16_t>(0),
                                                      kW * kW * 2, kBufferWord3);
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int ks = 0; ks < kNChunk; ++ks)
        pf[it][ks] = __builtin_amdgcn_raw_buffer_load_b128(
            rp, ((64 * w + 16 * it + r16) * kW + 32 * ks + 8 * (lane >> 4)) * 2, 0, 0);
  }
  // every P1 load complete before the first DMA load (the compiler tracks this wait, so it
  // adds none of its own later, which would also wait for the DMA loads behind it)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // DMA sources: load i of wave w fills slots 64 (4w + i) + lane of a chunk
  int dma_off[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int rho = 2 * (kDmaPerWave * w + i) + (lane >> 5), p = lane & 31, g = (rho >> 3) & 1;
    const int pi = p ^ ((rho & 3) | ((((p >> 3) & 1) ^ g) << 2) | (g << 3));
    dma_off[i] = rho * (kW * 2) + 16 * pi;
  }
  // transposing reads: fetch lane (G, j, q) = (lane >> 4, (lane >> 2) & 3, lane & 3) reads
  // row 8G + 4h + j, run q of column tile ct; the byte offset is
  //   512 (8G + j) + 2048 h + 256 (ct >> 3) + 16 p_low + 8 half, with
  //   p_low = 8 ((q >> 1) ^ (G & 1)) + 4 ((q & 1) ^ (q >> 1)) + (((ct & 7) >> 1) ^ j),
  //   half = (ct & 1) ^ (q & 1).
  int tr_off[4][2];
  {
    const int G = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
    const int l0 = 512 * (8 * G + j) + 128 * ((q >> 1) ^ (G & 1)) + 64 * ((q & 1) ^ (q >> 1));
#pragma unroll
    for (int c0 = 0; c0 < 4; ++c0)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) tr_off[c0][hb] = l0 + 16 * (c0 ^ j) + 8 * (hb ^ (q & 1));
  }

  // DMA issue state: the workgroup's next chunk to load (slice, chunk in slice, ring slot)
  int64_t d_slice = s;
  int d_ch = 0, d_slot = 0;
  auto dma_next = [&]() {
    const bool in = d_slice < K;
    const i32x4 rs = rsrc4(b.x + (in ? d_slice : 0) * (kW * kW), in ? kSliceB : 0);
    const uint32_t base = ring_addr + d_slot * kChunkB + 1024 * kDmaPerWave * w;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) dma16(base + 1024 * i, dma_off[i], rs, d_ch * kChunkB);
    if (++d_ch == kNChunk) {
      d_ch = 0;
      d_slice += stride;
    }
    if (++d_slot == kRing) d_slot = 0;
  };

  f32x4_t acc[16][4];  // [column tile][row tile]
  u32x4_t af[16];      // first operands of the chunk being multiplied
  int r_slot = 0;      // ring slot of that chunk
  int n_slot = 0;      // ring slot of the next chunk
  int pub = 1;         // the next chunk to publish (workgroup chunk index)
  auto read_frag = [&](int slot, int ct, u32x4_t& f) __attribute__((always_inline)) {
    const lds_u8* base = ring_l + slot * kChunkB + 256 * (ct >> 3) + tr_off[(ct & 7) >> 1][ct & 1];
    f = tr_frag(base, base + 2048);
  };

  // prologue: chunks 0 .. kRing-2 requested, chunk 0 published, chunk kRing-1 requested
#pragma unroll 1
  for (int t = 0; t < kRing - 1; ++t) dma_next();
  wait_barrier<kDmaPerWave * (kRing - 2)>();
  dma_next();
#pragma unroll
  for (int ct = 0; ct < kAhead; ++ct) read_frag(0, ct, af[ct]);

  // One chunk: y^T[ct, it] += x^T[ct, chunk] . P1^T[chunk, it] over the 16 column tiles,
  // the fragment of tile ct + kAhead read while tile ct's products run.  Before tile
  // 16 - kAhead the next chunk is published (its DMA loads waited for, then the barrier,
  // after which every wave is done with this wave's previous chunk, whose slot takes the
  // next DMA loads), and the next chunk's first kAhead fragments are read from then on, one
  // a tile, into the registers of tiles whose products have been issued.
  auto chunk_step = [&](auto chv) __attribute__((always_inline)) {
    constexpr int ch = decltype(chv)::value;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
      if (ct + kAhead < 16) read_frag(r_slot, ct + kAhead, af[ct + kAhead]);
      if (ct == 16 - kAhead) {
        // operations issued after the published chunk's DMA loads: the loads of the
        // kRing - 2 chunks after it, plus an epilogue's stores once one can lie between
        // (from the tenth chunk on; at most one is counted, which waits longer, never less)
        if (pub >= 9)
          wait_barrier<kDmaPerWave * (kRing - 2) + kStoresPerSlice>();
        else
          wait_barrier<kDmaPerWave * (kRing - 2)>();
        dma_next();
        ++pub;
        n_slot = r_slot + 1 == kRing ? 0 : r_slot + 1;
      }
      if (ct >= 16 - kAhead) read_frag(n_slot, ct - (16 - kAhead), af[ct - (16 - kAhead)]);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t a = af[ct];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        if constexpr (ch == 0)
          mfma_a_first<DT>(acc[ct][it], a, pf[it][ch]);
        else
          mfma_a_acc<DT>(acc[ct][it], a, pf[it][ch]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    r_slot = n_slot;
  };

  const float dmax = pb.dmax, dinv = pb.dmax_inv;
  // [FQV2] 第3步 pergroup / 第4步 for slice s: lane l, row tile it holds y row
  // 64w + 16 it + r16, columns 32 g .. 32 g + 31 of group g = qc (tiles 0..7) and g = qc + 4
  // (tiles 8..15).  Codes: one 16-byte store per group (bytes of units 2d, 2d+1 in dword d;
  // odd runs hold the units of a pair in swapped tiles, undone by a 16-bit rotation).
  // e8m0: a row's 8 bytes are gathered over the four lanes that share it.
  auto epilogue = [&]() __attribute__((always_inline)) {
    const auto rs_codes = __builtin_amdgcn_make_buffer_rsrc(b.codes + s * (kW * kW / 2), static_cast<int16_t>(0),
                                                            kW * kW / 2, kBufferWord3);
    const auto rs_e8 = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(b.scale) + s * e8m0_bytes_per_slice(kW * kW), static_cast<int16_t>(0),
        static_cast<int>(e8m0_bytes_per_slice(kW * kW)), kBufferWord3);
    int code_off = r16 * (kW / 2) + 16 * qc;
    int e8_off = r16 * (kW / 32);
    uint32_t rot = 16 * (qc & 1);
    asm volatile("" : "+v"(code_off), "+v"(e8_off), "+v"(rot));
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      uint32_t e8[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float am = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const f32x4_t& v = acc[8 * hh + t][it];
          asm("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(am) : "v"(v[0]), "v"(v[1]));
          asm("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(am) : "v"(v[2]), "v"(v[3]));
        }
        const uint32_t code = e8m0_code_v<SV>(am, dmax, dinv);
        e8[hh] = code;
        const float scf = e8m0_to_float(code);
        u32x4_t out;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const f32x4_t& v0 = acc[8 * hh + 2 * d][it];
          const f32x4_t& v1 = acc[8 * hh + 2 * d + 1][it];
          uint32_t pk = fp4x2<0>(0u, v0[0], v0[1], scf);
          pk = fp4x2<1>(pk, v0[2], v0[3], scf);
          pk = fp4x2<2>(pk, v1[0], v1[1], scf);
          pk = fp4x2<3>(pk, v1[2], v1[3], scf);
          out[d] = __builtin_amdgcn_alignbit(pk, pk, rot);
        }
        __builtin_amdgcn_raw_buffer_store_b128(out, rs_codes, code_off, (64 * w + 16 * it) * (kW / 2) + 64 * hh, 0);
      }
      // row 64w + 16 it + r16: byte g of its 8 e8m0 bytes is group g's code; lane group qc
      // holds groups qc and qc + 4
      uint32_t lo = e8[0] << (8 * qc), hi = e8[1] << (8 * qc);
      {
        auto r = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        lo = r[0] | r[1];
        auto t = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        hi = t[0] | t[1];
      }
      {
        auto r = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        lo = r[0] | r[1];
        auto t = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        hi = t[0] | t[1];
      }
      // the four lanes of a row hold the same 8 bytes and all store them (no branch)
      typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
      const u32x2_t both = {lo, hi};
      __builtin_amdgcn_raw_buffer_store_b64(both, rs_e8, e8_off, (64 * w + 16 * it) * (kW / 32), 0);
    }
  };

  while (true) {
    chunk_step(std::integral_constant<int, 0>{});
    chunk_step(std::integral_constant<int, 1>{});
    chunk_step(std::integral_constant<int, 2>{});
    chunk_step(std::integral_constant<int, 3>{});
    chunk_step(std::integral_constant<int, 4>{});
    chunk_step(std::integral_constant<int, 5>{});
    chunk_step(std::integral_constant<int, 6>{});
    chunk_step(std::integral_constant<int, 7>{});
    agpr_fence<16>(acc);
    epilogue();
    s += stride;
    if (s >= K) break;
  }
  // DMA loads still in flight (chunks past the last slice) land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int DT, int SV>
hipError_t launch_w1s(const Problem& pb, const Buffers& b, hipStream_t s) {
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
  mfma_wide1s_kernel<DT, SV><<<grid, kThreads, 0, s>>>(pb, b);
  return hipGetLastError();
}

template <int DT>
hipError_t dispatch_w1s(const Problem& pb, const Buffers& b, hipStream_t s) {
  switch (e8m0_variant(pb)) {
    case kE8V1: return launch_w1s<DT, kE8V1>(pb, b, s);
    case kE8V2Pow2: return launch_w1s<DT, kE8V2Pow2>(pb, b, s);
    default: return launch_w1s<DT, kE8V2Div>(pb, b, s);
  }
}

}  // namespace

bool mfma_wide1s_supports(const Problem& pb) {
  return pb.M == kW && pb.N == kW && !pb.two_sided && pb.mode == kPerGroupFp4;
}

hipError_t launch_mfma_wide1s(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (!mfma_wide1s_supports(pb)) return hipErrorNotSupported;
  return pb.dtype == kBF16 ? dispatch_w1s<kBF16>(pb, b, s) : dispatch_w1s<kF16>(pb, b, s);
}

}  // namespace fq
