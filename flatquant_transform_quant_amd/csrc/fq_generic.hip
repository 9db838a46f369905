// Generic libfq kernel: any shape 1 <= M, N <= 256, every mode, both dtypes.
//
// One workgroup per slice (grid-stride over K).  Step 1 ([FQV2] 第1步) forms
// T = round_dtype(fl32(x_k . P2)) element by element with an fp64 FMA chain rounded once
// to fp32, and keeps T in LDS (at most 256 x 256 x 2 B = 128 KB).  Step 2 ([FQV2] 第2步)
// forms each y the same way over m and feeds it straight to the encoder, so y is never
// stored.  Per token, y is formed twice -- once for max|y|, once to encode -- by the
// same code, so both passes see identical values.  Per group, one thread forms the 32
// values of a group, its scale and its 16 code bytes.
//
// This is the correctness-first path that covers every shape; the MFMA kernels take
// the shapes they support.  Also here: the strided gather / scatter kernels that stage
// non-contiguous tensors through the workspace.
#include <hip/hip_runtime.h>

#include "fq_codec.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int kGenericThreads = 256;

// The sums are accumulated in fp64 (the 16-bit products are exact there) and rounded once
// to fp32: y and T are then the correctly rounded fp32 values of the products, whatever
// the length of the contraction.
template <int DT>
__device__ __forceinline__ float y_at(const uint16_t* __restrict__ p1, const uint16_t* Ts, int M, int N,
                                      int i, int n) {
  double acc = 0.0;
  const uint16_t* prow = p1 + static_cast<int64_t>(i) * M;
  for (int m = 0; m < M; ++m)
    acc = __builtin_fma(static_cast<double>(load16<DT>(prow[m])), static_cast<double>(load16<DT>(Ts[m * N + n])), acc);
  return static_cast<float>(acc);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kGenericThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

// FIXUP: redo only the per-token slices whose stored scale is below 2^-126 (and above 0).
// The 256-class two-sided kernel encodes y * (1 / scale), and 1 / scale overflows for a
// scale below 2^-128; its slices with such tiny scales are recomputed here, where the
// codes come from y / scale.  Workgroup g looks at slices [256 g, 256 g + 256): each thread
// reads one scale (all in parallel), and only the flagged slices are recomputed.
__device__ __forceinline__ bool tiny_scale(float s) { return s > 0.0f && s < 0x1p-126f; }

template <int DT, bool FIXUP>
__global__ __launch_bounds__(kGenericThreads) void generic_kernel(Problem pb, Buffers b) {
  extern __shared__ uint16_t Ts[];  // M * N
  __shared__ float red[kGenericThreads / 64];
  __shared__ uint32_t flags[kGenericThreads / 32];
  const int M = static_cast<int>(pb.M), N = static_cast<int>(pb.N), MN = M * N;
  const int tid = threadIdx.x;
  int64_t k_begin = blockIdx.x, k_end = pb.K, k_step = gridDim.x;
  if constexpr (FIXUP) {
    k_begin = int64_t(blockIdx.x) * kGenericThreads;
    k_end = k_begin + kGenericThreads < pb.K ? k_begin + kGenericThreads : pb.K;
    k_step = 1;
    if (tid < kGenericThreads / 32) flags[tid] = 0u;
    __syncthreads();
    const int64_t mine = k_begin + tid;
    if (mine < k_end && tiny_scale(static_cast<const float*>(b.scale)[mine]))
      atomicOr(&flags[tid >> 5], 1u << (tid & 31));
    __syncthreads();
    // none flagged (the usual case): the workgroup is done
    uint32_t any = 0;
#pragma unroll
    for (int i = 0; i < kGenericThreads / 32; ++i) any |= flags[i];
    if (any == 0u) return;
  }
  for (int64_t k = k_begin; k < k_end; k += k_step) {
    if constexpr (FIXUP) {
      const int i = static_cast<int>(k - k_begin);  // the same for every thread
      if (!((flags[i >> 5] >> (i & 31)) & 1u)) continue;
    }
    const uint16_t* xk = b.x + k * pb.xs_k;  // row m of the slice at xk + m * xs_m
    const int64_t xs_m = pb.xs_m;
    // [FQV2] 第1步: T = x_k . P2, rounded to the dtype; skipped for an empty P2.
    for (int e = tid; e < MN; e += kGenericThreads) {
      if (pb.two_sided) {
        const int m = e / N, n = e % N;
        double acc = 0.0;
        for (int j = 0; j < N; ++j)
          acc = __builtin_fma(static_cast<double>(load16<DT>(xk[m * xs_m + j])),
                              static_cast<double>(load16<DT>(b.p2[j * N + n])), acc);
        // T is the fp32 value rounded to the dtype: two roundings.  The register barrier
        // keeps the compiler from merging them into one fp64 -> dtype rounding, which
        // differs where the fp32 value is a tie of the dtype.
        float t32 = static_cast<float>(acc);
        asm volatile("" : "+v"(t32));
        Ts[e] = round16<DT>(t32);
      } else {
        Ts[e] = xk[(e / N) * xs_m + e % N];
      }
    }
    __syncthreads();
    uint8_t* codes = b.codes + k * (byte_codes(pb.mode) ? MN : MN / 2);
    if (pb.mode == kPerGroupFp4) {
      const int G = static_cast<int>(ceil_div(MN, 32));
      const int GS = static_cast<int>(e8m0_bytes_per_slice(MN));
      uint8_t* e8 = static_cast<uint8_t*>(b.scale) + k * GS;
      for (int g = tid; g < G; g += kGenericThreads) {
        float v[32];
        float amax = 0.0f;
        const int f0 = g * 32, cnt = min(32, MN - f0);
#pragma unroll
        for (int t = 0; t < 32; ++t) {
          v[t] = 0.0f;
          if (t < cnt) {
            const int f = f0 + t;
            v[t] = y_at<DT>(b.p1, Ts, M, N, f / N, f % N);
            amax = fmaxf(amax, __builtin_fabsf(v[t]));
          }
        }
        const uint32_t code = e8m0_code(amax, pb.dmax);
        e8[g] = static_cast<uint8_t>(code);
#pragma unroll
        for (int t = 0; t < 32; t += 2)
          if (t < cnt)
            codes[(f0 + t) >> 1] = static_cast<uint8_t>(e2m1_code(apply_e8m0(v[t], code)) |
                                                         (e2m1_code(apply_e8m0(v[t + 1], code)) << 4));
      }
      if (tid == 0 && GS > G) e8[G] = 0;
    } else {
      // [FQV2] 第3步 pertoken: scale = max|y| / (max_val / clipRatio), codes = y / scale
      // (max_val 7 for int4; 127 / 448 / 57344 for the 8-bit codes of the dequant_swiglu_quant
      // page, section 3.4).
      float amax = 0.0f;
      for (int e = tid; e < MN; e += kGenericThreads)
        amax = fmaxf(amax, __builtin_fabsf(y_at<DT>(b.p1, Ts, M, N, e / N, e % N)));
      amax = block_max(amax, red);
      const float scale = amax / pb.d;
      if (tid == 0) static_cast<float*>(b.scale)[k] = scale;
      if (byte_codes(pb.mode)) {
        for (int e = tid; e < MN; e += kGenericThreads) {
          uint32_t c = 0;
          if (scale > 0.0f) {
            const float q = y_at<DT>(b.p1, Ts, M, N, e / N, e % N) / scale;
            c = (pb.mode == kPerTokenInt8 ? int8_code(q) : (pb.mode == kPerTokenE4M3 ? e4m3x2(q, q) : e5m2x2(q, q))) & 0xFFu;
          }
          codes[e] = static_cast<uint8_t>(c);
        }
      }
      for (int p = tid; p < (byte_codes(pb.mode) ? 0 : MN / 2); p += kGenericThreads) {
        const int e = 2 * p;
        uint32_t c0 = 0, c1 = 0;
        if (scale > 0.0f) {
          c0 = int4_nibble(y_at<DT>(b.p1, Ts, M, N, e / N, e % N) / scale);
          c1 = int4_nibble(y_at<DT>(b.p1, Ts, M, N, (e + 1) / N, (e + 1) % N) / scale);
        }
        codes[p] = static_cast<uint8_t>(c0 | (c1 << 4));
      }
    }
    __syncthreads();  // T is rewritten for the next slice
  }
}

__global__ void gather16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t d0,
                                int64_t d1, int64_t d2, int64_t s0, int64_t s1, int64_t s2) {
  const int64_t total = d0 * d1 * d2;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t i2 = i % d2, i1 = (i / d2) % d1, i0 = i / (d1 * d2);
    dst[i] = src[i0 * s0 + i1 * s1 + i2 * s2];
  }
}

template <typename T>
__global__ void scatter_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t d0, int64_t d1,
                               int64_t d2, int64_t s0, int64_t s1, int64_t s2) {
  const int64_t total = d0 * d1 * d2;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t i2 = i % d2, i1 = (i / d2) % d1, i0 = i / (d1 * d2);
    dst[i0 * s0 + i1 * s1 + i2 * s2] = src[i];
  }
}

int grid_for(int64_t total, int threads) {
  int64_t g = (total + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  return static_cast<int>(g);
}

template <bool FIXUP>
hipError_t launch_generic_t(const Problem& pb, const Buffers& b, hipStream_t s, int max_grid) {
  const size_t lds = static_cast<size_t>(pb.M * pb.N) * 2;
  const int grid = static_cast<int>(pb.K < max_grid ? pb.K : max_grid);
  const void* fn = pb.dtype == kBF16 ? reinterpret_cast<const void*>(generic_kernel<kBF16, FIXUP>)
                                     : reinterpret_cast<const void*>(generic_kernel<kF16, FIXUP>);
  hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  if (pb.dtype == kBF16)
    generic_kernel<kBF16, FIXUP><<<grid, kGenericThreads, lds, s>>>(pb, b);
  else
    generic_kernel<kF16, FIXUP><<<grid, kGenericThreads, lds, s>>>(pb, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_generic(const Problem& pb, const Buffers& b, hipStream_t s) {
  return launch_generic_t<false>(pb, b, s, 4096);
}

hipError_t launch_tiny_scale_fixup(const Problem& pb, const Buffers& b, hipStream_t s) {
  if (byte_codes(pb.mode) || pb.mode == kPerTokenInt32 || pb.mode == kPerTokenInt4) {
    // one workgroup per 256 slices (the kernel's own grid rule for FIXUP)
    const int64_t groups = (pb.K + kGenericThreads - 1) / kGenericThreads;
    return launch_generic_t<true>(pb, b, s, static_cast<int>(groups));
  }
  return hipSuccess;  // per group: the scales are powers of two, nothing overflows
}

hipError_t launch_gather16(const uint16_t* src, uint16_t* dst, const int64_t shape[3],
                           const int64_t strides[3], hipStream_t s) {
  const int64_t total = shape[0] * shape[1] * shape[2];
  if (total == 0) return hipSuccess;
  gather16_kernel<<<grid_for(total, 256), 256, 0, s>>>(src, dst, shape[0], shape[1], shape[2], strides[0],
                                                      strides[1], strides[2]);
  return hipGetLastError();
}

hipError_t launch_scatter(const void* src, void* dst, int elem_bytes, const int64_t shape[3],
                          const int64_t strides[3], hipStream_t s) {
  const int64_t total = shape[0] * shape[1] * shape[2];
  if (total == 0) return hipSuccess;
  if (elem_bytes == 4)
    scatter_kernel<uint32_t><<<grid_for(total, 256), 256, 0, s>>>(
        static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), shape[0], shape[1], shape[2],
        strides[0], strides[1], strides[2]);
  else
    scatter_kernel<uint8_t><<<grid_for(total, 256), 256, 0, s>>>(
        static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), shape[0], shape[1], shape[2],
        strides[0], strides[1], strides[2]);
  return hipGetLastError();
}

}  // namespace fq
