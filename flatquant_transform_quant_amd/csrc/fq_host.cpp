// libfq host side: the C ABI of include/fq.h -- validation, planning, workspace
// staging of non-contiguous tensors, and kernel dispatch.
//
// The call pattern and the checks follow the page "aclnnFlatQuantV2 算子拆解" (cited
// as [FQV2]): sections 两段式接口 (two-stage call, the executor carries everything),
// 参数速查 / 标量参数 (dtypes, shapes, scalar ranges) and 容易踩的坑 (error codes and
// the order of the checks).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "fq.h"
#include "fq_internal.h"

using fq::ceil_div;

namespace {

constexpr uint32_t kLiveMagic = 0xF0A17E55u;
constexpr uint32_t kDeadMagic = 0xDEADF00Du;
constexpr int64_t kMaxK = 262144;
constexpr int64_t kMaxMN = 256;

}  // namespace

struct fq_executor {
  uint32_t magic;
  fq::Problem pb;
  int32_t kernel;       // fq::Kernel actually launched (never kAuto)
  int32_t repeatable;
  fq_tensor x, p1, p2, out, scale;
  bool stage_x, stage_p1, stage_p2, stage_out, stage_scale;
  bool x_direct;  // a non-contiguous x read in place through its strides (no gather)
  uint64_t off_x, off_p1, off_p2, off_out, off_scale, off_ctr, ws_size;
};

namespace {

bool is_contiguous(const fq_tensor& t) {
  int64_t expect = 1;
  for (int d = t.ndim - 1; d >= 0; --d) {
    if (t.shape[d] != 1 && t.strides[d] != expect) return false;
    expect *= t.shape[d];
  }
  return true;
}

bool strides_ok(const fq_tensor& t) {
  if (t.ndim < 0 || t.ndim > 4) return false;
  for (int d = 0; d < t.ndim; ++d)
    if (t.shape[d] < 0 || t.strides[d] < 0) return false;
  return true;
}

bool shape_is(const fq_tensor& t, int nd, int64_t a, int64_t b = 0, int64_t c = 0) {
  if (t.ndim != nd) return false;
  const int64_t want[3] = {a, b, c};
  for (int d = 0; d < nd; ++d)
    if (t.shape[d] != want[d]) return false;
  return true;
}

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// Detail of the last runtime failure on this thread (fq_last_error).
thread_local char g_last_error[256];

fq_status fail_runtime(const char* what, hipError_t err) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (hipError %d)", what,
                err == hipSuccess ? "failed" : hipGetErrorString(err), static_cast<int>(err));
  return FQ_ERR_RUNTIME;
}

// gfx950 check, cached per device id.
std::mutex g_arch_mu;
int g_arch_ok[64];  // 0 unknown, 1 yes, -1 no

bool device_is_gfx950() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_ok[dev]) return g_arch_ok[dev] > 0;
  }
  hipDeviceProp_t prop;
  bool ok = false;
  if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
    ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    g_arch_ok[dev] = ok ? 1 : -1;
  }
  return ok;
}

// Executors handed out and not yet released.  fq_run and the other calls look a pointer
// up here before touching it, so a released (single-use, already run) executor is
// reported as invalid instead of being read after free.
std::mutex g_live_mu;
std::unordered_set<const fq_executor*> g_live;

bool live(const fq_executor* e) {
  if (!e) return false;
  std::lock_guard<std::mutex> lk(g_live_mu);
  return g_live.count(e) != 0 && e->magic == kLiveMagic;
}

// The MFMA kernels load x, P1 and P2 16 bytes at a time and store codes and scales up
// to 4 bytes at a time; staged tensors live in the (256-byte aligned) workspace.
bool vector_aligned(const fq_executor* e) {
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  return (e->stage_x || al(e->x.data, 16)) && (e->stage_p1 || al(e->p1.data, 16)) &&
         (!e->pb.two_sided || e->stage_p2 || al(e->p2.data, 16)) &&
         (e->stage_out || al(e->out.data, 4)) && (e->stage_scale || al(e->scale.data, 4));
}

bool kernel_supports(int32_t k, const fq_executor* e) {
  switch (k) {
    case fq::kGeneric: return true;
    case fq::kMfmaSmall: return vector_aligned(e) && fq::mfma_small_supports(e->pb);
    case fq::kMfmaWide: return !e->x_direct && vector_aligned(e) && fq::mfma_wide_supports(e->pb);
    case fq::kMfmaWideT: return !e->x_direct && vector_aligned(e) && fq::mfma_wide2t_supports(e->pb);
    case fq::kMfmaWideL: return !e->x_direct && vector_aligned(e) && fq::mfma_wide1s_supports(e->pb);
    default: return false;
  }
}

int32_t auto_kernel(const fq_executor* e) {
  if (kernel_supports(fq::kMfmaWideT, e)) return fq::kMfmaWideT;
  if (kernel_supports(fq::kMfmaWideL, e)) return fq::kMfmaWideL;
  if (kernel_supports(fq::kMfmaWide, e)) return fq::kMfmaWide;
  if (kernel_supports(fq::kMfmaSmall, e)) return fq::kMfmaSmall;
  return fq::kGeneric;
}

}  // namespace

extern "C" {

fq_status fq_get_workspace_size(const fq_tensor* x, const fq_tensor* kroneckerP1,
                                const fq_tensor* kroneckerP2, double clipRatio, double dstTypeMax,
                                const fq_tensor* out, const fq_tensor* quantScale,
                                uint64_t* workspaceSize, fq_executor** executor) {
  g_last_error[0] = '\0';
  // [FQV2] 容易踩的坑: a NULL among the three inputs and two outputs -> 161001.
  if (!x || !kroneckerP1 || !kroneckerP2 || !out || !quantScale || !workspaceSize || !executor)
    return FQ_ERR_PARAM_NULLPTR;
  const bool p2_empty = kroneckerP2->ndim == 2 && kroneckerP2->shape[0] == 0 &&
                        kroneckerP2->shape[1] == 0;
  if (!x->data || !kroneckerP1->data || !out->data || !quantScale->data ||
      (!kroneckerP2->data && !p2_empty))
    return FQ_ERR_PARAM_NULLPTR;

  // Then clipRatio in (0, 1] and x's dimension ranges [1,262144] x [1,256] x [1,256].
  if (!(clipRatio > 0.0 && clipRatio <= 1.0)) return FQ_ERR_PARAM_INVALID;
  if (x->ndim != 3) return FQ_ERR_PARAM_INVALID;
  const int64_t K = x->shape[0], M = x->shape[1], N = x->shape[2];
  if (K < 1 || K > kMaxK || M < 1 || M > kMaxMN || N < 1 || N > kMaxMN) return FQ_ERR_PARAM_INVALID;

  // Then the remaining rules ([FQV2] 参数速查, 标量参数, 容易踩的坑).
  for (const fq_tensor* t : {x, kroneckerP1, kroneckerP2, out, quantScale})
    if (!strides_ok(*t)) return FQ_ERR_PARAM_INVALID;
  const int32_t dt = x->dtype;
  if (dt != FQ_DT_FLOAT16 && dt != FQ_DT_BFLOAT16) return FQ_ERR_PARAM_INVALID;
  if (kroneckerP1->dtype != dt || kroneckerP2->dtype != dt) return FQ_ERR_PARAM_INVALID;
  if (!shape_is(*kroneckerP1, 2, M, M)) return FQ_ERR_PARAM_INVALID;
  if (!p2_empty && !shape_is(*kroneckerP2, 2, N, N)) return FQ_ERR_PARAM_INVALID;

  int32_t mode;
  const int64_t MN = M * N;
  switch (out->dtype) {
    case FQ_DT_INT32:
      if (N % 8 != 0 || !shape_is(*out, 3, K, M, N / 8)) return FQ_ERR_PARAM_INVALID;
      mode = fq::kPerTokenInt32;
      break;
    case FQ_DT_INT4:
      if (N % 2 != 0 || !shape_is(*out, 3, K, M, N)) return FQ_ERR_PARAM_INVALID;
      mode = fq::kPerTokenInt4;
      break;
    case FQ_DT_FLOAT4_E2M1:
      if (N % 2 != 0 || !shape_is(*out, 2, K, MN)) return FQ_ERR_PARAM_INVALID;
      mode = fq::kPerGroupFp4;
      break;
    case FQ_DT_INT8:
    case FQ_DT_FLOAT8_E4M3FN:
    case FQ_DT_FLOAT8_E5M2:
      if (!shape_is(*out, 3, K, M, N)) return FQ_ERR_PARAM_INVALID;
      mode = out->dtype == FQ_DT_INT8 ? fq::kPerTokenInt8
                                      : (out->dtype == FQ_DT_FLOAT8_E4M3FN ? fq::kPerTokenE4M3 : fq::kPerTokenE5M2);
      break;
    default:
      return FQ_ERR_PARAM_INVALID;
  }
  if (mode == fq::kPerGroupFp4) {
    if (quantScale->dtype != FQ_DT_FLOAT8_E8M0 || !shape_is(*quantScale, 3, K, ceil_div(MN, 64), 2))
      return FQ_ERR_PARAM_INVALID;
  } else {
    if (quantScale->dtype != FQ_DT_FLOAT32 || !shape_is(*quantScale, 1, K)) return FQ_ERR_PARAM_INVALID;
    if (p2_empty) return FQ_ERR_PARAM_INVALID;  // [0, 0] P2 is for the per-group mode only
  }
  if (!(dstTypeMax == 0.0 || (dstTypeMax >= 6.0 && dstTypeMax <= 12.0))) return FQ_ERR_PARAM_INVALID;
  // 4-bit outputs: innermost stride 1, other strides whole bytes.
  if (out->dtype == FQ_DT_INT4 || out->dtype == FQ_DT_FLOAT4_E2M1) {
    if (out->strides[out->ndim - 1] != 1) return FQ_ERR_PARAM_INVALID;
    for (int d = 0; d + 1 < out->ndim; ++d)
      if (out->strides[d] % 2 != 0) return FQ_ERR_PARAM_INVALID;
  }

  fq_executor* e = new (std::nothrow) fq_executor();
  if (!e) return fail_runtime("executor allocation", hipErrorOutOfMemory);
  e->magic = kLiveMagic;
  e->pb.dtype = dt == FQ_DT_FLOAT16 ? fq::kF16 : fq::kBF16;
  e->pb.mode = mode;
  e->pb.K = K;
  e->pb.M = M;
  e->pb.N = N;
  e->pb.two_sided = p2_empty ? 0 : 1;
  // per-token divisor max_val / clipRatio: int4 7 ([FQV2] 第3步 pertoken); INT8 127, FP8
  // E4M3FN 448, FP8 E5M2 57344 (the dequant_swiglu_quant page, section 3.4)
  const double qmax = mode == fq::kPerTokenInt8 ? 127.0
                      : mode == fq::kPerTokenE4M3 ? 448.0
                      : mode == fq::kPerTokenE5M2 ? 57344.0
                                                  : 7.0;
  e->pb.d = static_cast<float>(qmax / clipRatio);
  e->pb.dmax = static_cast<float>(dstTypeMax);
  {
    int ex = 0;
    const double mant = std::frexp(dstTypeMax, &ex);
    e->pb.dmax_inv = (dstTypeMax > 0.0 && mant == 0.5) ? static_cast<float>(1.0 / dstTypeMax) : 0.0f;
  }
  e->repeatable = 0;
  e->x = *x;
  e->p1 = *kroneckerP1;
  e->p2 = *kroneckerP2;
  e->out = *out;
  e->scale = *quantScale;
  e->stage_x = !is_contiguous(*x);
  e->x_direct = false;
  e->pb.xs_k = MN;
  e->pb.xs_m = N;
  e->stage_p1 = !is_contiguous(*kroneckerP1);
  e->stage_p2 = !p2_empty && !is_contiguous(*kroneckerP2);
  e->stage_out = !is_contiguous(*out);
  e->stage_scale = !is_contiguous(*quantScale);
  uint64_t off = 0;
  auto take = [&](bool need, uint64_t bytes) -> uint64_t {
    if (!need) return 0;
    uint64_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (e->stage_x) {
    // Strided-input fast path: with a unit innermost stride and slice / row strides of whole
    // 16-byte units the generic and one-wave-per-slice kernels read x in place (no gather
    // into the workspace); the 256-class kernels keep the gather.
    const int64_t sk = x->strides[0], sm = x->strides[1], sn = x->strides[2];
    const bool ok = (sn == 1 || N == 1) && (sk % 8 == 0 || K == 1) && (sm % 8 == 0 || M == 1) &&
                    reinterpret_cast<uintptr_t>(x->data) % 16 == 0 && (M - 1) * sm + N < (int64_t(1) << 30) &&
                    (K - 1) * sk + (M - 1) * sm + N < (int64_t(1) << 62);
    if (ok && auto_kernel(e) != fq::kMfmaWide && auto_kernel(e) != fq::kMfmaWideT && auto_kernel(e) != fq::kMfmaWideL) {
      e->stage_x = false;
      e->x_direct = true;
      e->pb.xs_k = K == 1 ? MN : sk;
      e->pb.xs_m = M == 1 ? N : sm;
    }
  }
  e->off_x = take(e->stage_x, uint64_t(K * MN) * 2);
  e->off_p1 = take(e->stage_p1, uint64_t(M * M) * 2);
  e->off_p2 = take(e->stage_p2, uint64_t(N * N) * 2);
  e->off_out = take(e->stage_out, uint64_t(fq::byte_codes(mode) ? K * MN : K * MN / 2));
  e->off_scale = take(e->stage_scale, mode == fq::kPerGroupFp4
                                          ? uint64_t(K * fq::e8m0_bytes_per_slice(MN))
                                          : uint64_t(K) * 4);
  // the slice counter of the pipelined 256 x 256 kernel (it hands out slices at run time)
  e->off_ctr = take(kernel_supports(fq::kMfmaWideT, e), 4);
  e->ws_size = off;
  e->kernel = auto_kernel(e);
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.insert(e);
  }
  *workspaceSize = off;
  *executor = e;
  return FQ_SUCCESS;
}

static void release(fq_executor* e) {
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.erase(e);
  }
  e->magic = kDeadMagic;
  delete e;
}

fq_status fq_run(void* workspace, uint64_t workspaceSize, fq_executor* executor, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!executor) return FQ_ERR_PARAM_NULLPTR;
  if (!live(executor)) return FQ_ERR_PARAM_INVALID;
  fq_executor* e = executor;
  fq_status st = FQ_SUCCESS;
  do {
    if (e->ws_size > 0 && !workspace) { st = FQ_ERR_PARAM_NULLPTR; break; }
    if (workspaceSize < e->ws_size) { st = FQ_ERR_PARAM_INVALID; break; }
    if (!device_is_gfx950()) { st = fail_runtime("the current device is not gfx950", hipSuccess); break; }
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const fq::Problem& pb = e->pb;
    const int64_t MN = pb.M * pb.N;
    fq::Buffers b;
    hipError_t err = hipSuccess;
    auto gather = [&](const fq_tensor& t, bool stage, uint64_t off, int nd) -> const uint16_t* {
      if (!stage) return static_cast<const uint16_t*>(t.data);
      int64_t shape[3] = {1, 1, 1}, strides[3] = {0, 0, 0};
      for (int d = 0; d < nd; ++d) {
        shape[3 - nd + d] = t.shape[d];
        strides[3 - nd + d] = t.strides[d];
      }
      uint16_t* dst = reinterpret_cast<uint16_t*>(ws + off);
      if (err == hipSuccess) err = fq::launch_gather16(static_cast<const uint16_t*>(t.data), dst, shape,
                                                       strides, stream);
      return dst;
    };
    b.x = gather(e->x, e->stage_x, e->off_x, 3);
    b.p1 = gather(e->p1, e->stage_p1, e->off_p1, 2);
    b.p2 = pb.two_sided ? gather(e->p2, e->stage_p2, e->off_p2, 2) : nullptr;
    b.codes = e->stage_out ? ws + e->off_out : static_cast<uint8_t*>(e->out.data);
    b.scale = e->stage_scale ? static_cast<void*>(ws + e->off_scale) : e->scale.data;
    if (err != hipSuccess) { st = fail_runtime("strided input gather launch", err); break; }
    switch (e->kernel) {
      case fq::kMfmaSmall: err = fq::launch_mfma_small(pb, b, stream); break;
      case fq::kMfmaWide:
        err = fq::launch_mfma_wide(pb, b, stream);
        // its per-token epilogue multiplies by 1 / scale: slices with a scale below 2^-126
        // are re-encoded by division
        if (err == hipSuccess && pb.two_sided && pb.mode != fq::kPerGroupFp4)
          err = fq::launch_tiny_scale_fixup(pb, b, stream);
        break;
      case fq::kMfmaWideT:
        b.ctr = reinterpret_cast<uint32_t*>(ws + e->off_ctr);
        err = fq::launch_mfma_wide2t(pb, b, stream);
        if (err == hipSuccess) err = fq::launch_tiny_scale_fixup(pb, b, stream);  // as above
        break;
      case fq::kMfmaWideL: err = fq::launch_mfma_wide1s(pb, b, stream); break;
      default: err = fq::launch_generic(pb, b, stream); break;
    }
    if (err != hipSuccess) { st = fail_runtime("transform-quantize kernel launch", err); break; }
    if (e->stage_out) {
      // The codes as bytes: INT32 [K, M, N/8] words, INT4 [K, M, N/2] and
      // FLOAT4_E2M1 [K, M*N/2] byte rows (strides in 4-bit elements halve), the 8-bit
      // codes [K, M, N] bytes.
      int64_t shape[3], strides[3];
      int eb;
      if (e->out.dtype == FQ_DT_INT32) {
        eb = 4;
        for (int d = 0; d < 3; ++d) { shape[d] = e->out.shape[d]; strides[d] = e->out.strides[d]; }
      } else if (e->out.dtype == FQ_DT_INT4) {
        eb = 1;
        shape[0] = pb.K; shape[1] = pb.M; shape[2] = pb.N / 2;
        strides[0] = e->out.strides[0] / 2; strides[1] = e->out.strides[1] / 2; strides[2] = 1;
      } else if (fq::byte_codes(pb.mode)) {
        eb = 1;
        for (int d = 0; d < 3; ++d) { shape[d] = e->out.shape[d]; strides[d] = e->out.strides[d]; }
      } else {
        eb = 1;
        shape[0] = 1; shape[1] = pb.K; shape[2] = MN / 2;
        strides[0] = 0; strides[1] = e->out.strides[0] / 2; strides[2] = 1;
      }
      err = fq::launch_scatter(b.codes, e->out.data, eb, shape, strides, stream);
    }
    if (err == hipSuccess && e->stage_scale) {
      int64_t shape[3], strides[3];
      int eb;
      if (pb.mode == fq::kPerGroupFp4) {
        eb = 1;
        for (int d = 0; d < 3; ++d) { shape[d] = e->scale.shape[d]; strides[d] = e->scale.strides[d]; }
      } else {
        eb = 4;
        shape[0] = 1; shape[1] = 1; shape[2] = pb.K;
        strides[0] = 0; strides[1] = 0; strides[2] = e->scale.strides[0];
      }
      err = fq::launch_scatter(b.scale, e->scale.data, eb, shape, strides, stream);
    }
    if (err != hipSuccess) { st = fail_runtime("strided output scatter launch", err); break; }
  } while (false);
  if (!e->repeatable) release(e);
  return st;
}

void fq_executor_destroy(fq_executor* executor) {
  if (live(executor)) release(executor);
}

}  // extern "C"

// ---- fq_run without a caller-allocated workspace ------------------------------------------
// The staging buffer of non-contiguous tensors (the workspace of fq_run) taken from a
// file-scope device array instead.  Each device the library runs on holds its own copy
// (FQ_NO_ALLOC_SCRATCH_BYTES) until the process ends.  Host code never uses the array's
// name as an address: the device address of the current device's copy is looked up once
// per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) uint8_t scratch[FQ_NO_ALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device id, set on the first call on that device

fq_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail_runtime("hipGetDevice", err);
  if (dev < 0 || dev >= 64) return fail_runtime("device id beyond the scratch table", hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p) return fail_runtime("hipGetSymbolAddress of the scratch array", err);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FQ_SUCCESS;
}

}  // namespace

extern "C" {

fq_status fq_run_no_alloc(fq_executor* executor, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!executor) return FQ_ERR_PARAM_NULLPTR;
  if (!live(executor)) return FQ_ERR_PARAM_INVALID;
  fq_executor* e = executor;
  if (e->ws_size > FQ_NO_ALLOC_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "the planned workspace of %llu bytes exceeds the %llu-byte scratch of fq_run_no_alloc",
                  static_cast<unsigned long long>(e->ws_size),
                  static_cast<unsigned long long>(FQ_NO_ALLOC_SCRATCH_BYTES));
    if (!e->repeatable) release(e);
    return FQ_ERR_PARAM_INVALID;
  }
  void* ws = nullptr;
  if (e->ws_size > 0) {
    fq_status st = device_is_gfx950() ? scratch_of_current_device(&ws)
                                      : fail_runtime("the current device is not gfx950", hipSuccess);
    if (st != FQ_SUCCESS) {
      if (!e->repeatable) release(e);
      return st;
    }
  }
  // the same launches as fq_run, with the scratch array as the workspace (no allocation)
  return fq_run(ws, e->ws_size, e, stream);
}

fq_status fq_v1_get_workspace_size(const fq_tensor* x, const fq_tensor* kroneckerP1,
                                   const fq_tensor* kroneckerP2, double clipRatio, const fq_tensor* out,
                                   const fq_tensor* quantScale, uint64_t* workspaceSize, fq_executor** executor) {
  // [FQV2] V1 还是 V2: V2 with dstTypeMax 0.0 is V1
  return fq_get_workspace_size(x, kroneckerP1, kroneckerP2, clipRatio, 0.0, out, quantScale, workspaceSize, executor);
}

fq_status fq_dequant(const fq_tensor* codes, const fq_tensor* scale, const fq_tensor* out, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!codes || !scale || !out || !codes->data || !scale->data || !out->data) return FQ_ERR_PARAM_NULLPTR;
  // out: the values, [K, M, N] in x's dtype (its sizes fix K, M and N)
  if (out->ndim != 3 || !strides_ok(*out)) return FQ_ERR_PARAM_INVALID;
  const int64_t K = out->shape[0], M = out->shape[1], N = out->shape[2];
  if (K < 1 || K > kMaxK || M < 1 || M > kMaxMN || N < 1 || N > kMaxMN) return FQ_ERR_PARAM_INVALID;
  if (out->dtype != FQ_DT_FLOAT16 && out->dtype != FQ_DT_BFLOAT16) return FQ_ERR_PARAM_INVALID;
  const int64_t MN = M * N;
  // codes and scales as the quantizer writes them ([FQV2] 参数速查)
  bool per_group;
  int32_t mode8 = -1;  // the 8-bit per-token mode, if the codes are one a byte
  switch (codes->dtype) {
    case FQ_DT_INT32:
      if (N % 8 != 0 || !shape_is(*codes, 3, K, M, N / 8)) return FQ_ERR_PARAM_INVALID;
      per_group = false;
      break;
    case FQ_DT_INT8:
    case FQ_DT_FLOAT8_E4M3FN:
    case FQ_DT_FLOAT8_E5M2:
      if (!shape_is(*codes, 3, K, M, N)) return FQ_ERR_PARAM_INVALID;
      per_group = false;
      mode8 = codes->dtype == FQ_DT_INT8 ? fq::kPerTokenInt8
                                        : (codes->dtype == FQ_DT_FLOAT8_E4M3FN ? fq::kPerTokenE4M3 : fq::kPerTokenE5M2);
      break;
    case FQ_DT_INT4:
      if (N % 2 != 0 || !shape_is(*codes, 3, K, M, N)) return FQ_ERR_PARAM_INVALID;
      per_group = false;
      break;
    case FQ_DT_FLOAT4_E2M1:
      if (N % 2 != 0 || !shape_is(*codes, 2, K, MN)) return FQ_ERR_PARAM_INVALID;
      per_group = true;
      break;
    default:
      return FQ_ERR_PARAM_INVALID;
  }
  if (per_group) {
    if (scale->dtype != FQ_DT_FLOAT8_E8M0 || !shape_is(*scale, 3, K, ceil_div(MN, 64), 2)) return FQ_ERR_PARAM_INVALID;
  } else {
    if (scale->dtype != FQ_DT_FLOAT32 || !shape_is(*scale, 1, K)) return FQ_ERR_PARAM_INVALID;
  }
  // contiguous tensors only; the output is written 4 bytes at a time
  if (!strides_ok(*codes) || !strides_ok(*scale) || !is_contiguous(*codes) || !is_contiguous(*scale) ||
      !is_contiguous(*out))
    return FQ_ERR_PARAM_INVALID;
  if (reinterpret_cast<uintptr_t>(out->data) % 4 != 0 || (!per_group && reinterpret_cast<uintptr_t>(scale->data) % 4 != 0))
    return FQ_ERR_PARAM_INVALID;
  if (!device_is_gfx950()) return fail_runtime("the current device is not gfx950", hipSuccess);
  const int32_t odt = out->dtype == FQ_DT_FLOAT16 ? fq::kF16 : fq::kBF16;
  const hipError_t err =
      mode8 >= 0 ? fq::launch_dequant8(odt, mode8, K, M, N, static_cast<const uint8_t*>(codes->data),
                                       static_cast<const float*>(scale->data), static_cast<uint16_t*>(out->data), stream)
                 : fq::launch_dequant(odt, per_group, K, M, N, static_cast<const uint8_t*>(codes->data), scale->data,
                                      static_cast<uint16_t*>(out->data), stream);
  if (err != hipSuccess) return fail_runtime("dequant kernel launch", err);
  return FQ_SUCCESS;
}

fq_status fq_int4_gemm(const fq_tensor* a, const fq_tensor* a_scale, const fq_tensor* w, const fq_tensor* w_scale,
                       const fq_tensor* c, hipStream_t stream) {
  g_last_error[0] = '\0';
  for (const fq_tensor* t : {a, a_scale, w, w_scale, c})
    if (!t || !t->data) return FQ_ERR_PARAM_NULLPTR;
  for (const fq_tensor* t : {a, a_scale, w, w_scale, c})
    if (!strides_ok(*t) || !is_contiguous(*t)) return FQ_ERR_PARAM_INVALID;
  if (a->dtype != FQ_DT_INT4 || w->dtype != FQ_DT_INT4 || a->ndim != 2 || w->ndim != 2) return FQ_ERR_PARAM_INVALID;
  const int64_t T = a->shape[0], H = a->shape[1], O = w->shape[0];
  if (T < 1 || O < 1 || H < 128 || H % 128 != 0 || w->shape[1] != H) return FQ_ERR_PARAM_INVALID;
  if (a_scale->dtype != FQ_DT_FLOAT32 || !shape_is(*a_scale, 1, T)) return FQ_ERR_PARAM_INVALID;
  if (w_scale->dtype != FQ_DT_FLOAT32 || !shape_is(*w_scale, 1, O)) return FQ_ERR_PARAM_INVALID;
  if ((c->dtype != FQ_DT_BFLOAT16 && c->dtype != FQ_DT_FLOAT32) || !shape_is(*c, 2, T, O)) return FQ_ERR_PARAM_INVALID;
  // 32-bit buffer offsets, with a tile's worth of rows past the end
  const int64_t lim = int64_t(1) << 31;
  if ((T + 256) * (H / 2) >= lim || (O + 256) * (H / 2) >= lim || (T + 256) * 4 >= lim || (O + 256) * 4 >= lim)
    return FQ_ERR_PARAM_INVALID;
  auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(a->data, 16) || !al(w->data, 16) || !al(a_scale->data, 4) || !al(w_scale->data, 4) ||
      !al(c->data, c->dtype == FQ_DT_FLOAT32 ? 4 : 2))
    return FQ_ERR_PARAM_INVALID;
  if (!device_is_gfx950()) return fail_runtime("the current device is not gfx950", hipSuccess);
  const hipError_t err = fq::launch_int4_gemm(T, O, H, static_cast<const uint8_t*>(a->data),
                                              static_cast<const float*>(a_scale->data),
                                              static_cast<const uint8_t*>(w->data),
                                              static_cast<const float*>(w_scale->data), c->data,
                                              c->dtype == FQ_DT_FLOAT32, stream);
  if (err != hipSuccess) return fail_runtime("int4 GEMM kernel launch", err);
  return FQ_SUCCESS;
}

fq_status fq_mx_gemm(const fq_tensor* a, const fq_tensor* a_scale, const fq_tensor* w, const fq_tensor* w_scale,
                     const fq_tensor* c, hipStream_t stream) {
  g_last_error[0] = '\0';
  for (const fq_tensor* t : {a, a_scale, w, w_scale, c})
    if (!t || !t->data) return FQ_ERR_PARAM_NULLPTR;
  for (const fq_tensor* t : {a, a_scale, w, w_scale, c})
    if (!strides_ok(*t) || !is_contiguous(*t)) return FQ_ERR_PARAM_INVALID;
  if (a->dtype != FQ_DT_FLOAT4_E2M1 || w->dtype != FQ_DT_FLOAT4_E2M1 || a->ndim != 2 || w->ndim != 2)
    return FQ_ERR_PARAM_INVALID;
  const int64_t T = a->shape[0], H = a->shape[1], O = w->shape[0];
  if (T < 1 || O < 1 || H < 128 || H % 128 != 0 || w->shape[1] != H) return FQ_ERR_PARAM_INVALID;
  const int64_t gs = 2 * ceil_div(H, 64);
  if (a_scale->dtype != FQ_DT_FLOAT8_E8M0 || !shape_is(*a_scale, 3, T, gs / 2, 2)) return FQ_ERR_PARAM_INVALID;
  if (w_scale->dtype != FQ_DT_FLOAT8_E8M0 || !shape_is(*w_scale, 3, O, gs / 2, 2)) return FQ_ERR_PARAM_INVALID;
  if ((c->dtype != FQ_DT_BFLOAT16 && c->dtype != FQ_DT_FLOAT32) || !shape_is(*c, 2, T, O)) return FQ_ERR_PARAM_INVALID;
  // 32-bit buffer offsets, with a tile's worth of rows past the end
  const int64_t lim = int64_t(1) << 31;
  if ((T + 256) * (H / 2) >= lim || (O + 256) * (H / 2) >= lim || (T + 256) * gs >= lim || (O + 256) * gs >= lim)
    return FQ_ERR_PARAM_INVALID;
  auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(a->data, 16) || !al(w->data, 16) || !al(c->data, c->dtype == FQ_DT_FLOAT32 ? 4 : 2))
    return FQ_ERR_PARAM_INVALID;
  if (!device_is_gfx950()) return fail_runtime("the current device is not gfx950", hipSuccess);
  const hipError_t err = fq::launch_mx_gemm(T, O, H, static_cast<const uint8_t*>(a->data),
                                            static_cast<const uint8_t*>(a_scale->data), static_cast<const uint8_t*>(w->data),
                                            static_cast<const uint8_t*>(w_scale->data), c->data,
                                            c->dtype == FQ_DT_FLOAT32, stream);
  if (err != hipSuccess) return fail_runtime("MXFP4 GEMM kernel launch", err);
  return FQ_SUCCESS;
}

fq_status fq_executor_set_repeatable(fq_executor* executor, int32_t repeat) {
  if (!executor) return FQ_ERR_PARAM_NULLPTR;
  if (!live(executor)) return FQ_ERR_PARAM_INVALID;
  executor->repeatable = repeat ? 1 : 0;
  return FQ_SUCCESS;
}

fq_status fq_executor_set_kernel(fq_executor* executor, int32_t variant) {
  if (!executor) return FQ_ERR_PARAM_NULLPTR;
  if (!live(executor)) return FQ_ERR_PARAM_INVALID;
  int32_t k = variant == fq::kAuto ? auto_kernel(executor) : variant;
  if (!kernel_supports(k, executor)) return FQ_ERR_PARAM_INVALID;
  executor->kernel = k;
  return FQ_SUCCESS;
}

int32_t fq_executor_kernel(const fq_executor* executor) {
  if (!live(executor)) return -1;
  return executor->kernel;
}

const char* fq_last_error(void) { return g_last_error; }

const char* fq_status_string(fq_status status) {
  switch (status) {
    case FQ_SUCCESS: return "FQ_SUCCESS";
    case FQ_ERR_PARAM_NULLPTR: return "FQ_ERR_PARAM_NULLPTR: a required pointer is NULL";
    case FQ_ERR_PARAM_INVALID: return "FQ_ERR_PARAM_INVALID: a parameter failed validation";
    case FQ_ERR_RUNTIME: return "FQ_ERR_RUNTIME: device is not gfx950 or a HIP call failed";
    default: return "unknown libfq status";
  }
}

}  // extern "C"
