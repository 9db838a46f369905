/*
 * libfq -- fused small-matrix transform + dynamic low-bit quantization for AMD
 * Instinct MI355X (gfx950).
 *
 * The operator is the one stated on the page "aclnnFlatQuantV2 算子拆解：两步矩阵乘 +
 * 动态量化，CANN 上怎么写一次讲清" (cited as [FQV2] with the page's section names).
 * For every slice x_k [M, N] of x [K, M, N]:
 *
 *   T   = round_to_dtype(x_k . P2)          [FQV2] 拆开算, 第1步 (skipped when P2 is [0, 0])
 *   y_k = P1 . T   (fp32, never stored)     [FQV2] 拆开算, 第2步
 *
 * then one of two dynamic quantizations ([FQV2] 拆开算, 第3步 and 第4步):
 *
 *   per token (out INT32 or INT4):
 *       quantScale[k] = max|y_k| / (7 / clipRatio)              (fp32)
 *       code          = clamp(round_half_even(y / quantScale[k]), -8, 7)
 *   per group of 32 consecutive elements of the flattened slice (out FLOAT4_E2M1):
 *       dstTypeMax == 0  (V1): e8m0 = floor(log2(group max)) - 2 + 127, clamped to [0, 254]
 *       dstTypeMax in [6, 12] (V2): S = group max / dstTypeMax (fp32); e8m0 = the biased
 *           exponent of S, plus one when S is normal, the exponent is below 254 and the
 *           mantissa is non-zero
 *       code = E2M1(y * 2^(127 - e8m0)), round half to even, saturating at +-6
 *
 * Readings of points the page leaves open: the intermediate T is rounded to x's dtype
 * (the transforms must have x's dtype), y stays fp32, rounding is half-to-even
 * everywhere, int4 clamps to [-8, 7], the V1 exponent offset is 2 (E2M1's largest value
 * 6 = 1.5 * 2^2), 4-bit codes are packed low nibble first (INT32 words little-endian),
 * groups may span rows, a last partial group uses the elements present, the pad byte of
 * an odd group count is 0, and an all-zero slice or group gets scale 0 and codes 0.
 *
 * Calling pattern ([FQV2] 两段式接口): the first call validates, sizes the workspace
 * and returns an executor that holds every parameter; the caller allocates the
 * workspace only when its size is non-zero; the second call enqueues the work on a HIP
 * stream and takes no tensors.
 */
#ifndef FQ_H
#define FQ_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ([FQV2] 容易踩的坑) ------------------------------------------
 * FQ_ERR_PARAM_NULLPTR: one of the five tensors (or its data pointer) is NULL, or an
 *   output pointer of the call is NULL.
 * FQ_ERR_PARAM_INVALID: every other failed check -- shape, dtype, clipRatio,
 *   dstTypeMax, an empty P2 outside the per-group mode, a workspace that is too small,
 *   an executor that is not live.
 * FQ_ERR_RUNTIME: the device is not gfx950, or a HIP call failed while enqueueing. */
typedef int32_t fq_status;
#define FQ_SUCCESS 0
#define FQ_ERR_PARAM_NULLPTR 161001
#define FQ_ERR_PARAM_INVALID 161002
#define FQ_ERR_RUNTIME 161003

/* ---- tensor descriptors ----------------------------------------------------------
 * [FQV2] 参数速查: all tensors are ND.
 *   x            FLOAT16 | BFLOAT16       [K, M, N], 1 <= K <= 262144, 1 <= M, N <= 256
 *   kroneckerP1  same dtype as x          [M, M]
 *   kroneckerP2  same dtype as x          [N, N], or [0, 0] (per-group mode only)
 *   out          INT32        [K, M, N/8]  (N % 8 == 0; 8 int4 codes per word)
 *                INT4         [K, M, N]    (N even; 2 codes per byte)
 *                FLOAT4_E2M1  [K, M*N]     (N even; 2 codes per byte)
 *                INT8 | FLOAT8_E4M3FN | FLOAT8_E5M2  [K, M, N]   (1 code per byte)
 *   quantScale   FLOAT32      [K]                          with INT32 / INT4 / 8-bit out
 *                FLOAT8_E8M0  [K, ceilDiv(M*N, 64), 2]     with FLOAT4_E2M1 out
 * The 8-bit outputs extend the per-token mode with the dynamic per-row quantization of
 * the dequant_swiglu_quant page (section 3.4): scale_k = fl32(max|y_k| /
 * fl32(max_val / clipRatio)) with max_val 127 (INT8), 448 (FLOAT8_E4M3FN), 57344
 * (FLOAT8_E5M2); INT8 codes clamp(RNE(y / scale), -127, 127) as two's-complement bytes;
 * FP8 codes the OCP E4M3FN / E5M2 value nearest clamp(y / scale, -max_val, max_val), a
 * tie to the even code, keeping y's sign.  They need a [N, N] P2 (as INT32 / INT4 do).
 * `data` is a device pointer; it is never dereferenced by fq_get_workspace_size.
 * `strides` are in elements of the tensor's dtype (for INT4 and FLOAT4_E2M1, in 4-bit
 * elements).  Inputs may have any non-negative strides.  Outputs may be strided too,
 * but the innermost dimension of INT4 / FLOAT4_E2M1 must have stride 1 and their other
 * strides must be even (whole bytes).  Non-contiguous tensors are staged through the
 * workspace, except an x whose innermost stride is 1 and whose other strides are multiples
 * of 8 elements (16-byte aligned data): the generic and one-wave-per-slice kernels read such
 * an x in place.  The caller owns all tensor memory; it must stay valid until the work
 * enqueued by fq_run has completed on the stream. */
typedef enum {
  FQ_DT_FLOAT16 = 1,
  FQ_DT_BFLOAT16 = 2,
  FQ_DT_FLOAT32 = 3,
  FQ_DT_INT32 = 4,
  FQ_DT_INT4 = 5,
  FQ_DT_FLOAT4_E2M1 = 6,
  FQ_DT_FLOAT8_E8M0 = 7,
  FQ_DT_INT8 = 8,           /* per-token 8-bit codes (see fq_get_workspace_size) */
  FQ_DT_FLOAT8_E4M3FN = 9,
  FQ_DT_FLOAT8_E5M2 = 10
} fq_dtype;

typedef struct {
  void* data;
  int32_t dtype;      /* fq_dtype */
  int32_t ndim;       /* 0 .. 4 */
  int64_t shape[4];
  int64_t strides[4];
} fq_tensor;

typedef struct fq_executor fq_executor; /* opaque, owned by the library */

/* ---- first stage ([FQV2] 两段式接口, 容易踩的坑) ------------------------------------
 * Validates the call, chooses the kernels and sizes the workspace.
 *   clipRatio   in (0, 1]; used by the per-token mode only ([FQV2] 标量参数).
 *   dstTypeMax  0.0 or in [6.0, 12.0]; used by the FLOAT4_E2M1 mode only; 0.0 is V1.
 * Checks run in this order: NULL pointers (FQ_ERR_PARAM_NULLPTR), then clipRatio and
 * the ranges of x's dimensions, then dtypes, shapes and dstTypeMax
 * (FQ_ERR_PARAM_INVALID).  On success *workspaceSize holds the bytes fq_run needs and
 * *executor a new executor: the staged copies of non-contiguous tensors, plus 256 bytes
 * for a slice counter when the pipelined 256 x 256 kernel (variant 4: both transforms,
 * int4 per-token codes) can run the call; 0 when every tensor is contiguous and that kernel
 * does not apply.  On failure no executor is created.  Host only: makes no HIP call and
 * may run without a GPU. */
fq_status fq_get_workspace_size(const fq_tensor* x, const fq_tensor* kroneckerP1,
                                const fq_tensor* kroneckerP2, double clipRatio, double dstTypeMax,
                                const fq_tensor* out, const fq_tensor* quantScale,
                                uint64_t* workspaceSize, fq_executor** executor);

/* The first stage in the V1 form ([FQV2] V1 还是 V2): the same call without dstTypeMax.
 * The page states that V2 with dstTypeMax = 0.0 behaves exactly as V1, so this plans the
 * V2 call with dstTypeMax = 0.0 -- same checks, same statuses, same executor, run with
 * fq_run. */
fq_status fq_v1_get_workspace_size(const fq_tensor* x, const fq_tensor* kroneckerP1,
                                   const fq_tensor* kroneckerP2, double clipRatio, const fq_tensor* out,
                                   const fq_tensor* quantScale, uint64_t* workspaceSize, fq_executor** executor);

/* ---- second stage ------------------------------------------------------------------
 * Enqueues the fused computation on `stream` (0 = the null stream) and returns without
 * synchronizing.  `workspace` is device memory of at least workspaceSize bytes (may be
 * NULL when the planned size is 0); its contents need not be initialised (fq_run sets
 * what it reads, on the stream), and work enqueued with one workspace must not overlap in
 * time with other work using the same bytes.  By default the executor is single-use: fq_run
 * releases it, whether it succeeds or fails.  A repeatable executor
 * (fq_executor_set_repeatable) survives and must be released with fq_executor_destroy.
 * Results are deterministic: the same inputs give the same bits on every run.
 * Errors: NULL executor -> FQ_ERR_PARAM_NULLPTR; workspace NULL while needed ->
 * FQ_ERR_PARAM_NULLPTR; workspace too small or executor not live ->
 * FQ_ERR_PARAM_INVALID; not a gfx950 device, or a launch failure -> FQ_ERR_RUNTIME.
 * Calls with distinct executors may come from different host threads. */
fq_status fq_run(void* workspace, uint64_t workspaceSize, fq_executor* executor, hipStream_t stream);

/* ---- second stage without a workspace allocation ------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid hipMalloc, harnesses that forbid it): fq_run with the staging buffer of
 * non-contiguous tensors taken from a device array inside the library instead of a
 * caller-allocated workspace.  The array holds FQ_NO_ALLOC_SCRATCH_BYTES (64 MiB) on every
 * device the library runs on, until the process ends.  No hipMalloc, hipFree or other
 * allocating call is made.  Behaviour otherwise as fq_run (single-use executors are released
 * whatever the outcome).  Errors: NULL executor -> FQ_ERR_PARAM_NULLPTR; executor not live,
 * or a planned workspace above FQ_NO_ALLOC_SCRATCH_BYTES -> FQ_ERR_PARAM_INVALID (checked
 * before any HIP call; fq_last_error() names the sizes); not a gfx950 device or a launch
 * failure -> FQ_ERR_RUNTIME.  Every call on one device shares that device's array: calls that
 * overlap in time on one device (different streams, or different host threads) race on it and
 * must be ordered by the caller.  The array is overwritten before it is read on every call. */
#define FQ_NO_ALLOC_SCRATCH_BYTES (64ull << 20)
fq_status fq_run_no_alloc(fq_executor* executor, hipStream_t stream);

/* ---- dequantization ------------------------------------------------------------------
 * The values of the codes fq_run writes, in a 16-bit float dtype: the second half of a
 * quantize -> dequantize ("fake-quant") round trip, e.g. to measure the RMS error
 * (the APT-LLM page, section 5.2, checks |dequantize(quantize(x)) - x| this way; the
 * ModelOpt page, section 6.4, uses such a round trip as a reference).
 *   per token (codes INT32 [K, M, N/8] or INT4 [K, M, N], scale FLOAT32 [K]):
 *       value = q * scale[k], q the two's-complement int4 code (the APT-LLM page, section
 *       2.1: the symmetric integer format dequantizes as q * scale)
 *   per group (codes FLOAT4_E2M1 [K, M*N], scale FLOAT8_E8M0 [K, ceilDiv(M*N, 64), 2]):
 *       value = E2M1(code) * 2^(e8m0 - 127), E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with
 *       the sign bit on top (the ModelOpt page, section 6.1; [FQV2] 第3步 pergroup)
 *   per token, 8-bit (codes INT8 | FLOAT8_E4M3FN | FLOAT8_E5M2 [K, M, N], scale FLOAT32 [K]):
 *       value = q * scale[k], q the INT8 integer or the FP8 value of the code (the codes of
 *       the dynamic per-row quantization of the dequant_swiglu_quant page, section 3.4);
 *       INT8 -128 and the FP8 NaN / infinity encodings, which fq_run never writes, are
 *       outside the domain
 * The product is formed in IEEE fp32 (per group it is exact, or overflows to infinity; an
 * e8m0 byte 0xFF, NaN in the MX encoding, makes its group NaN) and rounded once, to
 * nearest even, to out's dtype.
 *   out   FLOAT16 | BFLOAT16 [K, M, N]; K, M, N in the ranges of x above; 4-byte aligned.
 * All three tensors must be contiguous device memory owned by the caller (valid until the
 * work completes on the stream).  The work is enqueued on `stream` without synchronizing;
 * no workspace.  Errors: a NULL tensor or data pointer -> FQ_ERR_PARAM_NULLPTR; any shape,
 * dtype, stride or alignment mismatch -> FQ_ERR_PARAM_INVALID (these checks make no HIP
 * call); not a gfx950 device, or a launch failure -> FQ_ERR_RUNTIME. */
fq_status fq_dequant(const fq_tensor* codes, const fq_tensor* scale, const fq_tensor* out, hipStream_t stream);

/* ---- int4 consumer GEMM ------------------------------------------------------------
 * The product that follows the per-token int4 quantizer in a FlatQuant linear layer:
 *     C[t, o] = fl32( fl32(acc[t, o]) * fl32(a_scale[t] * w_scale[o]) ),
 *     acc[t, o] = sum_h qa[t, h] * qw[o, h]   (exact: int32 accumulation, |acc| <= 64 H)
 * with qa the int4 codes fq_run writes per token ([FQV2] 第3步 pertoken; its INT32 and INT4
 * outputs are the same bytes, so out viewed as INT4 [K, M*N] is a with T = K, H = M*N) and its
 * FLOAT32 [K] quantScale as a_scale; W int4 weights with one fp32 scale per output channel.
 * The symmetric integer format dequantizes as q * scale (the APT-LLM page, section 2.1).
 *   a        INT4    [T, H]     two's complement, 2 codes per byte, low nibble first; H % 128 == 0
 *   a_scale  FLOAT32 [T]
 *   w        INT4    [O, H]
 *   w_scale  FLOAT32 [O]
 *   c        BFLOAT16 | FLOAT32 [T, O]   (a bf16 C is the fp32 value rounded to nearest even)
 * All tensors contiguous device memory owned by the caller; a and w 16-byte aligned, the
 * scales 4-byte aligned; (T + 256) * H / 2 and (O + 256) * H / 2 below 2^31.  Enqueued on
 * `stream` without synchronizing; no workspace.  Errors: a NULL tensor or data pointer ->
 * FQ_ERR_PARAM_NULLPTR; any shape, dtype, stride, size or alignment mismatch ->
 * FQ_ERR_PARAM_INVALID (no HIP call is made before these checks); not a gfx950 device, or a
 * launch failure -> FQ_ERR_RUNTIME. */
fq_status fq_int4_gemm(const fq_tensor* a, const fq_tensor* a_scale, const fq_tensor* w, const fq_tensor* w_scale,
                       const fq_tensor* c, hipStream_t stream);

/* ---- MXFP4 consumer GEMM ----------------------------------------------------------------
 * The product that follows the quantizer in a FlatQuant linear layer:
 *     C[t, o] = sum_h value(a[t, h]) * value(w[o, h])
 * with both operands in the per-group format fq_run writes ([FQV2] 第3步 pergroup / 第4步:
 * E2M1 codes, one e8m0 power of two per 32 consecutive elements of a row; the E2M1 values
 * from the ModelOpt page, section 6.1), so the quantizer's out / quantScale of a FLOAT4_E2M1
 * call feed it directly as a / a_scale (T = K, H = M*N).
 *   a        FLOAT4_E2M1  [T, H]                     H a multiple of 128
 *   a_scale  FLOAT8_E8M0  [T, ceilDiv(H, 64), 2]
 *   w        FLOAT4_E2M1  [O, H]
 *   w_scale  FLOAT8_E8M0  [O, ceilDiv(H, 64), 2]
 *   c        BFLOAT16 | FLOAT32 [T, O]
 * The products are accumulated in fp32 (the order is unspecified: the result lies within
 * gamma(H) * sum|terms| of the exact sum, gamma(n) = n u / (1 - n u), u = 2^-24) and rounded
 * once to c's dtype (round to nearest even).  Scales whose products leave the fp32 normal
 * range, and the e8m0 byte 0xFF (NaN), are outside the supported domain; the quantizer
 * writes neither.  All tensors contiguous device memory owned by the caller; a and w 16-byte
 * aligned; (T + 256) * H / 2 and (O + 256) * H / 2 below 2^31.  Enqueued on `stream` without
 * synchronizing; no workspace.  Errors: a NULL tensor or data pointer -> FQ_ERR_PARAM_NULLPTR;
 * any shape, dtype, stride, size or alignment mismatch -> FQ_ERR_PARAM_INVALID (no HIP call
 * is made before these checks); not a gfx950 device, or a launch failure -> FQ_ERR_RUNTIME. */
fq_status fq_mx_gemm(const fq_tensor* a, const fq_tensor* a_scale, const fq_tensor* w, const fq_tensor* w_scale,
                     const fq_tensor* c, hipStream_t stream);

/* Releases an executor that will not be run (or a repeatable one).  NULL is a no-op. */
void fq_executor_destroy(fq_executor* executor);

/* Keeps the executor alive across fq_run calls (repeat != 0), e.g. to launch the same
 * problem many times.  Returns FQ_ERR_PARAM_NULLPTR / FQ_ERR_PARAM_INVALID for a NULL or
 * dead executor. */
fq_status fq_executor_set_repeatable(fq_executor* executor, int32_t repeat);

/* Kernel variant the executor will launch: 0 = the automatic choice, 1 = the generic
 * kernel (any shape), 2 = the small-slice MFMA kernel (one wave per slice; M and N up to
 * 128, run at the next of 16, 32, 64, 128 with zero padding where they are not one of
 * them: per token N a multiple of 8, per group N one of 32, 64, 128), 3 = the
 * whole-workgroup MFMA kernel for 256 x 256 slices, which also takes the slices with a side
 * above 128 (M, N up to 256; N a multiple of 8, per group of 32), zero-padded to 256 x 256
 * (an empty P2 as the identity), 4 = its pipelined form for 256 x 256
 * slices with both transforms and per-token int4 codes (INT32 / INT4 out; the automatic
 * choice there), 5 = the streaming MFMA kernel for 256 x 256 slices with an empty P2 and
 * FLOAT4_E2M1 out (x through an LDS ring filled by DMA, P1 in registers; the automatic
 * choice there).  Selecting a variant that does not support the planned problem returns
 * FQ_ERR_PARAM_INVALID and leaves the executor unchanged.  Meant for tests and
 * benchmarks. */
fq_status fq_executor_set_kernel(fq_executor* executor, int32_t variant);

/* The variant the executor will launch (1 .. 5), or a negative value for NULL. */
int32_t fq_executor_kernel(const fq_executor* executor);

/* A static, human-readable name for a status code. */
const char* fq_status_string(fq_status status);

/* Detail of the last FQ_ERR_RUNTIME returned on the calling thread: the HIP call that
 * failed and the runtime's error text, or "" when there was none.  The string is owned by
 * the library and stays valid until the thread's next call into it. */
const char* fq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
