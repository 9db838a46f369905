// Internal interface between the libfq host code and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fq {

enum Dtype16 : int32_t { kF16 = 1, kBF16 = 2 };
enum Mode : int32_t {
  kPerTokenInt32 = 0,
  kPerTokenInt4 = 1,
  kPerGroupFp4 = 2,
  kPerTokenInt8 = 3,  // one byte a code: INT8, FP8 E4M3FN, FP8 E5M2
  kPerTokenE4M3 = 4,
  kPerTokenE5M2 = 5
};
// codes of one byte each (the 8-bit per-token modes) rather than two codes a byte
__host__ __device__ inline bool byte_codes(int32_t mode) { return mode >= kPerTokenInt8; }
enum Kernel : int32_t { kAuto = 0, kGeneric = 1, kMfmaSmall = 2, kMfmaWide = 3, kMfmaWideT = 4, kMfmaWideL = 5 };

// One planned problem, as the kernels see it (all tensors contiguous).
struct Problem {
  int32_t dtype;      // kF16 | kBF16
  int32_t mode;       // Mode
  int64_t K, M, N;
  int32_t two_sided;  // 0: P2 is [0, 0], the right multiply is skipped
  float d;            // fl32(max_val / clipRatio), the per-token divisor (max_val 7, 127, 448, 57344)
  float dmax;         // fl32(dstTypeMax); 0 selects V1
  float dmax_inv;     // 1/dmax when dmax is a power of two (then exact), else 0
  int64_t xs_k, xs_m; // x's slice and row strides in elements (M*N and N when contiguous);
                      // the innermost stride is 1; only the generic and small kernels take
                      // other values (x read in place)
};

// Device buffers of one launch, in the packed contiguous layouts:
//   x [K, M, N], p1 [M, M], p2 [N, N] (16-bit bits);
//   codes: K * M*N/2 bytes, low nibble = lower flattened index (K * M*N bytes for the
//          8-bit modes);
//   scale: float [K] (per token) or uint8 [K, 2*ceil(M*N/64)] (e8m0).
struct Buffers {
  const uint16_t* x;
  const uint16_t* p1;
  const uint16_t* p2;
  uint8_t* codes;
  void* scale;
  uint32_t* ctr = nullptr;  // slice counter of the kernels that hand out slices at run time (4 bytes)
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Which e8m0 rule a per-group launch compiles in (the E8Variant of the codec):
// 0 = V1 (dmax 0), 1 = V2 with dmax a power of two, 2 = V2 with a division.
inline int e8m0_variant(const Problem& pb) { return pb.dmax == 0.0f ? 0 : (pb.dmax_inv != 0.0f ? 1 : 2); }
__host__ __device__ inline int64_t e8m0_bytes_per_slice(int64_t MN) { return 2 * ceil_div(MN, 64); }

// Launchers (enqueue only; return the launch status).
hipError_t launch_generic(const Problem& pb, const Buffers& b, hipStream_t s);
// Re-encodes, after a kernel that encodes y * (1 / scale), the per-token slices whose scale
// is below 2^-126 (where 1 / scale can overflow), with y / scale; skips every other slice.
hipError_t launch_tiny_scale_fixup(const Problem& pb, const Buffers& b, hipStream_t s);
bool mfma_small_supports(const Problem& pb);
hipError_t launch_mfma_small(const Problem& pb, const Buffers& b, hipStream_t s);
bool mfma_wide_supports(const Problem& pb);
hipError_t launch_mfma_wide(const Problem& pb, const Buffers& b, hipStream_t s);
// The pipelined 256 x 256 two-sided per-token int4 kernel (codes formed under the next
// slice's first products).
bool mfma_wide2t_supports(const Problem& pb);
hipError_t launch_mfma_wide2t(const Problem& pb, const Buffers& b, hipStream_t s);
// The streaming 256 x 256 left-only per-group kernel (x through an LDS-DMA ring, P1 in
// registers).
bool mfma_wide1s_supports(const Problem& pb);
hipError_t launch_mfma_wide1s(const Problem& pb, const Buffers& b, hipStream_t s);

// Dequantization of contiguous codes/scales into a contiguous [K, M, N] 16-bit output.
hipError_t launch_dequant(int32_t dtype, bool per_group, int64_t K, int64_t M, int64_t N, const uint8_t* codes,
                          const void* scale, uint16_t* out, hipStream_t s);

// Dequantization of contiguous 8-bit per-token codes [K, M*N] with fp32 scales [K].
hipError_t launch_dequant8(int32_t dtype, int32_t mode, int64_t K, int64_t M, int64_t N, const uint8_t* codes,
                           const float* scale, uint16_t* out, hipStream_t s);

// int4 consumer GEMM over contiguous operands: C[T, O] = sa[t] sw[o] . A[T, H] . W[O, H]^T.
hipError_t launch_int4_gemm(int64_t T, int64_t O, int64_t H, const uint8_t* a, const float* sa, const uint8_t* w,
                            const float* sw, void* c, bool f32_out, hipStream_t s);

// MXFP4 consumer GEMM over contiguous operands: C[T, O] = A[T, H] . W[O, H]^T (bf16 or fp32 C).
hipError_t launch_mx_gemm(int64_t T, int64_t O, int64_t H, const uint8_t* a, const uint8_t* a_e8, const uint8_t* w,
                          const uint8_t* w_e8, void* c, bool f32_out, hipStream_t s);

// Strided 16-bit gather into a contiguous buffer: dst[i0, i1, i2] = src[i0*s0 + i1*s1 + i2*s2].
hipError_t launch_gather16(const uint16_t* src, uint16_t* dst, const int64_t shape[3],
                           const int64_t strides[3], hipStream_t s);
// Strided scatter of a contiguous buffer of 1- or 4-byte elements:
// dst[i0*s0 + i1*s1 + i2*s2] = src[i0, i1, i2].
hipError_t launch_scatter(const void* src, void* dst, int elem_bytes, const int64_t shape[3],
                          const int64_t strides[3], hipStream_t s);

}  // namespace fq
