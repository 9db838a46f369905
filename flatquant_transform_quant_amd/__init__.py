"""Python binding of libfq (include/fq.h): argument marshalling only.

Every step of the operator runs in the HIP kernels of ``libfq.so``; this module only
turns torch tensors into ``fq_tensor`` descriptors, calls the two C entry points and
allocates the workspace through torch.  If the shared library has not been built the
import fails loudly -- there is no fallback path.

Output storage in torch:
  * ``int32`` mode: out is ``torch.int32`` [K, M, N/8] (8 int4 codes per word, low nibble
    first), quantScale ``torch.float32`` [K];
  * ``int4``  mode: out is ``torch.uint8`` [K, M, N/2] holding the logical INT4 [K, M, N]
    (2 codes per byte, low nibble first), quantScale ``torch.float32`` [K];
  * ``fp4``   mode: out is ``torch.uint8`` (or ``torch.float4_e2m1fn_x2``) [K, M*N/2]
    holding the logical FLOAT4_E2M1 [K, M*N], quantScale ``torch.uint8`` (or
    ``torch.float8_e8m0fnu``) [K, ceilDiv(M*N, 64), 2];
  * ``int8`` / ``e4m3`` / ``e5m2`` modes (per-token 8-bit codes): out is ``torch.int8`` /
    ``torch.float8_e4m3fn`` / ``torch.float8_e5m2`` (or ``torch.uint8``) [K, M, N],
    quantScale ``torch.float32`` [K].
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfq.so")

FQ_SUCCESS = 0
FQ_ERR_PARAM_NULLPTR = 161001
FQ_ERR_PARAM_INVALID = 161002
FQ_ERR_RUNTIME = 161003

DT_FLOAT16, DT_BFLOAT16, DT_FLOAT32, DT_INT32, DT_INT4, DT_FLOAT4_E2M1, DT_FLOAT8_E8M0 = range(1, 8)
DT_INT8, DT_FLOAT8_E4M3FN, DT_FLOAT8_E5M2 = range(8, 11)
BYTE_MODES = {"int8": DT_INT8, "e4m3": DT_FLOAT8_E4M3FN, "e5m2": DT_FLOAT8_E5M2}
PER_TOKEN_MODES = ("int32", "int4") + tuple(BYTE_MODES)
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_MFMA_SMALL, KERNEL_MFMA_WIDE, KERNEL_MFMA_WIDE_T, KERNEL_MFMA_WIDE_L = 0, 1, 2, 3, 4, 5


class FqTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("strides", ctypes.c_int64 * 4)]


class FqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = lib.fq_last_error().decode() if status == FQ_ERR_RUNTIME else ""
        self.detail = detail
        super().__init__(f"{what}: {status_string(status)} ({status})" + (f": {detail}" if detail else ""))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libfq is not built ({LIB_PATH} missing): run __graft_entry__.build()")
    # torch ships its own HIP runtime under the same soname as the system one.  Loading
    # torch first makes libfq bind to that copy, so the process holds one HIP runtime and
    # the device pointers and streams torch hands over are valid handles in libfq too.
    # (Loaded the other way round, two runtimes coexist, each with its own device state.)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(FqTensor)
    vp = ctypes.c_void_p
    L.fq_get_workspace_size.argtypes = [P, P, P, ctypes.c_double, ctypes.c_double, P, P,
                                        ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(vp)]
    L.fq_get_workspace_size.restype = ctypes.c_int32
    L.fq_run.argtypes = [vp, ctypes.c_uint64, vp, vp]
    L.fq_run.restype = ctypes.c_int32
    L.fq_run_no_alloc.argtypes = [vp, vp]
    L.fq_run_no_alloc.restype = ctypes.c_int32
    L.fq_executor_destroy.argtypes = [vp]
    L.fq_executor_destroy.restype = None
    L.fq_executor_set_repeatable.argtypes = [vp, ctypes.c_int32]
    L.fq_executor_set_repeatable.restype = ctypes.c_int32
    L.fq_executor_set_kernel.argtypes = [vp, ctypes.c_int32]
    L.fq_executor_set_kernel.restype = ctypes.c_int32
    L.fq_executor_kernel.argtypes = [vp]
    L.fq_executor_kernel.restype = ctypes.c_int32
    L.fq_status_string.argtypes = [ctypes.c_int32]
    L.fq_status_string.restype = ctypes.c_char_p
    L.fq_last_error.argtypes = []
    L.fq_last_error.restype = ctypes.c_char_p
    L.fq_v1_get_workspace_size.argtypes = [P, P, P, ctypes.c_double, P, P,
                                           ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(vp)]
    L.fq_v1_get_workspace_size.restype = ctypes.c_int32
    L.fq_mx_gemm.argtypes = [P, P, P, P, P, vp]
    L.fq_mx_gemm.restype = ctypes.c_int32
    L.fq_int4_gemm.argtypes = [P, P, P, P, P, vp]
    L.fq_int4_gemm.restype = ctypes.c_int32
    L.fq_dequant.argtypes = [P, P, P, vp]
    L.fq_dequant.restype = ctypes.c_int32
    return L


lib = _load()
EXPORTS = ("fq_get_workspace_size", "fq_run", "fq_executor_destroy", "fq_executor_set_repeatable",
           "fq_executor_set_kernel", "fq_executor_kernel", "fq_status_string", "fq_last_error", "fq_dequant",
           "fq_v1_get_workspace_size", "fq_mx_gemm", "fq_int4_gemm", "fq_run_no_alloc")
NO_ALLOC_SCRATCH_BYTES = 64 << 20  # FQ_NO_ALLOC_SCRATCH_BYTES of include/fq.h


def status_string(status: int) -> str:
    return lib.fq_status_string(status).decode()


# ---- raw C entry points, same names as the C ABI ------------------------------------

def make_tensor(data_ptr: int, dtype: int, shape, strides=None) -> FqTensor:
    shape = list(shape)
    if strides is None:
        strides, acc = [], 1
        for d in reversed(shape):
            strides.insert(0, acc)
            acc *= d
    t = FqTensor()
    t.data = data_ptr or None
    t.dtype = dtype
    t.ndim = len(shape)
    for i, (s, st) in enumerate(zip(shape, strides)):
        t.shape[i] = int(s)
        t.strides[i] = int(st)
    return t


def fq_get_workspace_size(x: FqTensor, p1: FqTensor, p2: FqTensor, clip_ratio: float,
                          dst_type_max: float, out: FqTensor, quant_scale: FqTensor):
    """Returns (status, workspace_size, executor_handle)."""
    ws = ctypes.c_uint64(0)
    ex = ctypes.c_void_p(None)
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    st = lib.fq_get_workspace_size(ref(x), ref(p1), ref(p2), float(clip_ratio), float(dst_type_max),
                                   ref(out), ref(quant_scale), ctypes.byref(ws), ctypes.byref(ex))
    return st, ws.value, ex.value


def fq_v1_get_workspace_size(x: FqTensor, p1: FqTensor, p2: FqTensor, clip_ratio: float,
                             out: FqTensor, quant_scale: FqTensor):
    """The V1 form (no dstTypeMax). Returns (status, workspace_size, executor_handle)."""
    ws = ctypes.c_uint64(0)
    ex = ctypes.c_void_p(None)
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    st = lib.fq_v1_get_workspace_size(ref(x), ref(p1), ref(p2), float(clip_ratio), ref(out), ref(quant_scale),
                                      ctypes.byref(ws), ctypes.byref(ex))
    return st, ws.value, ex.value


def fq_run(workspace_ptr: int, workspace_size: int, executor: int, stream_ptr: int) -> int:
    return lib.fq_run(workspace_ptr or None, workspace_size, executor, stream_ptr or None)


def fq_run_no_alloc(executor: int, stream_ptr: int) -> int:
    return lib.fq_run_no_alloc(executor, stream_ptr or None)


def fq_executor_destroy(executor: int) -> None:
    lib.fq_executor_destroy(executor)


def fq_executor_set_repeatable(executor: int, repeat: bool) -> int:
    return lib.fq_executor_set_repeatable(executor, 1 if repeat else 0)


def fq_executor_set_kernel(executor: int, variant: int) -> int:
    return lib.fq_executor_set_kernel(executor, variant)


def fq_executor_kernel(executor: int) -> int:
    return lib.fq_executor_kernel(executor)


def fq_status_string(status: int) -> str:
    return status_string(status)


def fq_last_error() -> str:
    return lib.fq_last_error().decode()


def fq_int4_gemm(a: FqTensor, a_scale: FqTensor, w: FqTensor, w_scale: FqTensor, c: FqTensor, stream_ptr: int) -> int:
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lib.fq_int4_gemm(ref(a), ref(a_scale), ref(w), ref(w_scale), ref(c), stream_ptr or None)


def fq_mx_gemm(a: FqTensor, a_scale: FqTensor, w: FqTensor, w_scale: FqTensor, c: FqTensor, stream_ptr: int) -> int:
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lib.fq_mx_gemm(ref(a), ref(a_scale), ref(w), ref(w_scale), ref(c), stream_ptr or None)


def fq_dequant(codes: FqTensor, scale: FqTensor, out: FqTensor, stream_ptr: int) -> int:
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lib.fq_dequant(ref(codes), ref(scale), ref(out), stream_ptr or None)


# ---- torch marshalling ---------------------------------------------------------------

def _torch():
    import torch
    return torch


def describe_input(t) -> FqTensor:
    torch = _torch()
    dt = {torch.float16: DT_FLOAT16, torch.bfloat16: DT_BFLOAT16}.get(t.dtype)
    if dt is None:
        dt = -1  # rejected by validation
    return make_tensor(t.data_ptr(), dt, t.shape, t.stride())


def describe_out(out, mode: str, K: int, M: int, N: int) -> FqTensor:
    """Logical descriptor of the code tensor stored in `out` (see the module docstring)."""
    if mode == "int32":
        return make_tensor(out.data_ptr(), DT_INT32, out.shape, out.stride())
    st = list(out.stride())
    if mode == "int4":
        # uint8 [K, M, N/2] storage -> INT4 [K, M, N]: strides in nibbles
        return make_tensor(out.data_ptr(), DT_INT4, (K, M, N), (2 * st[0], 2 * st[1], 1 if st[2] == 1 else 2 * st[2]))
    if mode == "fp4":
        return make_tensor(out.data_ptr(), DT_FLOAT4_E2M1, (K, M * N), (2 * st[0], 1 if st[1] == 1 else 2 * st[1]))
    if mode in BYTE_MODES:
        return make_tensor(out.data_ptr(), BYTE_MODES[mode], out.shape, out.stride())
    raise ValueError(f"unknown mode {mode!r}")


def describe_scale(scale, mode: str) -> FqTensor:
    dt = DT_FLOAT32 if mode in PER_TOKEN_MODES else DT_FLOAT8_E8M0
    return make_tensor(scale.data_ptr(), dt, scale.shape, scale.stride())


def empty_outputs(K: int, M: int, N: int, mode: str, device="cuda"):
    """Allocate (out, quant_scale) for a mode, in the storage described above."""
    torch = _torch()
    if mode == "int32":
        return (torch.empty((K, M, N // 8), dtype=torch.int32, device=device),
                torch.empty((K,), dtype=torch.float32, device=device))
    if mode == "int4":
        return (torch.empty((K, M, N // 2), dtype=torch.uint8, device=device),
                torch.empty((K,), dtype=torch.float32, device=device))
    if mode == "fp4":
        return (torch.empty((K, M * N // 2), dtype=torch.uint8, device=device),
                torch.empty((K, -(-(M * N) // 64), 2), dtype=torch.uint8, device=device))
    if mode in BYTE_MODES:
        dt = {"int8": torch.int8, "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[mode]
        return (torch.empty((K, M, N), dtype=dt, device=device),
                torch.empty((K,), dtype=torch.float32, device=device))
    raise ValueError(f"unknown mode {mode!r}")


class Executor:
    """A planned call (first stage).  Repeatable: run() may be called many times."""

    def __init__(self, x, p1, p2, out, quant_scale, mode: str, clip_ratio: float = 1.0,
                 dst_type_max: float = 0.0, kernel: int = KERNEL_AUTO, repeatable: bool = True):
        torch = _torch()
        K, M, N = x.shape
        if p2 is None:
            p2 = torch.empty((0, 0), dtype=x.dtype, device=x.device)
        self._keep = (x, p1, p2, out, quant_scale)
        st, ws, ex = fq_get_workspace_size(describe_input(x), describe_input(p1), describe_input(p2),
                                           clip_ratio, dst_type_max, describe_out(out, mode, K, M, N),
                                           describe_scale(quant_scale, mode))
        if st != FQ_SUCCESS:
            raise FqError(st, "fq_get_workspace_size")
        self.handle = ex
        self.workspace_size = ws
        self.workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=x.device) if ws else None
        # streams (handles) the caching allocator knows the workspace is used on: the
        # allocating one, then every other stream a run was enqueued on
        self._ws_streams = set()
        if self.workspace is not None and x.device.type == "cuda":
            self._ws_streams.add(torch.cuda.current_stream(x.device).cuda_stream)
        if repeatable:
            fq_executor_set_repeatable(ex, True)
        self.repeatable = repeatable
        if kernel != KERNEL_AUTO:
            st = fq_executor_set_kernel(ex, kernel)
            if st != FQ_SUCCESS:
                self.destroy()
                raise FqError(st, f"fq_executor_set_kernel({kernel})")

    @property
    def kernel(self) -> int:
        return fq_executor_kernel(self.handle)

    def run(self, stream=None) -> None:
        torch = _torch()
        if self.handle is None:
            raise RuntimeError("executor already released")
        s = stream if stream is not None else torch.cuda.current_stream(self._keep[0].device)
        wsp = self.workspace.data_ptr() if self.workspace is not None else 0
        if self.workspace is not None and s.cuda_stream not in self._ws_streams:
            # The workspace was allocated on the planning thread's current stream; the
            # kernels may run on another one.  Tell the caching allocator (once per stream:
            # it keeps the set until the block is freed), so that a workspace freed right
            # after this call (quantize() drops its executor) is not handed to work on the
            # allocating stream while these kernels still use it.
            self.workspace.record_stream(s)
            self._ws_streams.add(s.cuda_stream)
        st = fq_run(wsp, self.workspace_size, self.handle, s.cuda_stream)
        if not self.repeatable:
            self.handle = None
        if st != FQ_SUCCESS:
            raise FqError(st, "fq_run")

    def destroy(self) -> None:
        if self.handle is not None:
            fq_executor_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def quantize(x, p1, p2, out, quant_scale, mode: str, clip_ratio: float = 1.0,
             dst_type_max: float = 0.0, stream=None, kernel: int = KERNEL_AUTO) -> None:
    """One fused call: plan (single-use executor) and enqueue on `stream`."""
    ex = Executor(x, p1, p2, out, quant_scale, mode, clip_ratio, dst_type_max, kernel=kernel,
                  repeatable=False)
    ex.run(stream)


def dequantize(codes, quant_scale, mode: str, M: int, N: int, dtype, out=None, stream=None):
    """Values of quantizer outputs (as stored by ``empty_outputs``) in ``dtype``
    (torch.bfloat16 or torch.float16): a [K, M, N] tensor, ``out`` when given."""
    torch = _torch()
    K = codes.shape[0]
    if out is None:
        out = torch.empty((K, M, N), dtype=dtype, device=codes.device)
    dt = {torch.float16: DT_FLOAT16, torch.bfloat16: DT_BFLOAT16}.get(out.dtype, -1)
    st = fq_dequant(describe_out(codes, mode, K, M, N), describe_scale(quant_scale, mode),
                    make_tensor(out.data_ptr(), dt, out.shape, out.stride()),
                    (stream if stream is not None else torch.cuda.current_stream(codes.device)).cuda_stream)
    if st != FQ_SUCCESS:
        raise FqError(st, "fq_dequant")
    return out


def mx_gemm(a_codes, a_scale, w_codes, w_scale, H: int, out_dtype=None, out=None, stream=None):
    """C [T, O] = A . W^T for operands in the quantizer's per-group storage: codes uint8
    [rows, H/2] (or the fp4 out of ``empty_outputs``), e8m0 uint8 [rows, ceilDiv(H, 64), 2].
    C is torch.bfloat16 (default) or torch.float32."""
    torch = _torch()
    for t in (a_codes, a_scale, w_codes, w_scale):
        if not t.is_contiguous():
            raise ValueError("mx_gemm operands must be contiguous")
    T, O = a_codes.shape[0], w_codes.shape[0]
    if out is None:
        out = torch.empty((T, O), dtype=out_dtype or torch.bfloat16, device=a_codes.device)
    cdt = {torch.bfloat16: DT_BFLOAT16, torch.float32: DT_FLOAT32}.get(out.dtype, -1)
    G = -(-H // 64)
    st = fq_mx_gemm(make_tensor(a_codes.data_ptr(), DT_FLOAT4_E2M1, (T, H)),
                    make_tensor(a_scale.data_ptr(), DT_FLOAT8_E8M0, (T, G, 2)),
                    make_tensor(w_codes.data_ptr(), DT_FLOAT4_E2M1, (O, H)),
                    make_tensor(w_scale.data_ptr(), DT_FLOAT8_E8M0, (O, G, 2)),
                    make_tensor(out.data_ptr(), cdt, out.shape, out.stride()),
                    (stream if stream is not None else torch.cuda.current_stream(a_codes.device)).cuda_stream)
    if st != FQ_SUCCESS:
        raise FqError(st, "fq_mx_gemm")
    return out


def int4_gemm(a_codes, a_scale, w_codes, w_scale, H: int, out_dtype=None, out=None, stream=None):
    """C [T, O] = a_scale[t] w_scale[o] (A . W^T) for int4 codes in the quantizer's per-token
    storage: codes uint8 [rows, H/2] (the int4 / int32 out of ``empty_outputs`` viewed as
    bytes), scales float32 [rows].  C is torch.bfloat16 (default) or torch.float32."""
    torch = _torch()
    for t in (a_codes, a_scale, w_codes, w_scale):
        if not t.is_contiguous():
            raise ValueError("int4_gemm operands must be contiguous")
    T, O = a_codes.shape[0], w_codes.shape[0]
    if out is None:
        out = torch.empty((T, O), dtype=out_dtype or torch.bfloat16, device=a_codes.device)
    cdt = {torch.bfloat16: DT_BFLOAT16, torch.float32: DT_FLOAT32}.get(out.dtype, -1)
    st = fq_int4_gemm(make_tensor(a_codes.data_ptr(), DT_INT4, (T, H)),
                      make_tensor(a_scale.data_ptr(), DT_FLOAT32, (T,)),
                      make_tensor(w_codes.data_ptr(), DT_INT4, (O, H)),
                      make_tensor(w_scale.data_ptr(), DT_FLOAT32, (O,)),
                      make_tensor(out.data_ptr(), cdt, out.shape, out.stride()),
                      (stream if stream is not None else torch.cuda.current_stream(a_codes.device)).cuda_stream)
    if st != FQ_SUCCESS:
        raise FqError(st, "fq_int4_gemm")
    return out
