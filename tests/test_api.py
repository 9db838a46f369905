"""The C ABI: exported symbols, validation matrix, check order, workspace sizing and
executor lifetime (CPU only: planning never touches a device).

Error codes and the check order follow the aclnnFlatQuantV2 page, section 容易踩的坑:
a NULL among the five tensors gives 161001; every other failure 161002; clipRatio and
x's dimension ranges are checked before the other rules.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import flatquant_transform_quant_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DUMMY = 0x10000  # never dereferenced by the planner
NULLP, INVAL, OK = fq.FQ_ERR_PARAM_NULLPTR, fq.FQ_ERR_PARAM_INVALID, fq.FQ_SUCCESS


def header_functions():
    src = open(os.path.join(ROOT, "include", "fq.h"), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert "fq_get_workspace_size" in names and "fq_run" in names
    for n in names:
        assert hasattr(fq.lib, n), n
    assert set(names) == set(fq.EXPORTS)


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


def tens(dtype, shape, strides=None, data=DUMMY):
    return fq.make_tensor(data, dtype, shape, strides)


def problem(K=4, M=16, N=16, dt=fq.DT_BFLOAT16, mode="int32", p2_empty=False):
    x = tens(dt, (K, M, N))
    p1 = tens(dt, (M, M))
    p2 = tens(dt, (0, 0), data=0) if p2_empty else tens(dt, (N, N))
    if mode == "int32":
        out, sc = tens(fq.DT_INT32, (K, M, N // 8)), tens(fq.DT_FLOAT32, (K,))
    elif mode == "int4":
        out, sc = tens(fq.DT_INT4, (K, M, N)), tens(fq.DT_FLOAT32, (K,))
    elif mode in fq.BYTE_MODES:
        out, sc = tens(fq.BYTE_MODES[mode], (K, M, N)), tens(fq.DT_FLOAT32, (K,))
    else:
        out = tens(fq.DT_FLOAT4_E2M1, (K, M * N))
        sc = tens(fq.DT_FLOAT8_E8M0, (K, -(-(M * N) // 64), 2))
    return dict(x=x, p1=p1, p2=p2, out=out, sc=sc)


def plan(p, clip=1.0, dmax=0.0):
    st, ws, ex = fq.fq_get_workspace_size(p["x"], p["p1"], p["p2"], clip, dmax, p["out"], p["sc"])
    if ex:
        fq.fq_executor_destroy(ex)
    return st, ws


@pytest.mark.parametrize("mode", ["int32", "int4", "fp4", "int8", "e4m3", "e5m2"])
def test_valid_plans_have_zero_workspace(mode):
    st, ws = plan(problem(mode=mode))
    assert (st, ws) == (OK, 0)


@pytest.mark.parametrize("mode,p2_empty,ws", [("int32", False, 256), ("int4", False, 256), ("fp4", False, 0),
                                              ("fp4", True, 0), ("int8", False, 0)])
def test_pipelined_kernel_plans_a_slice_counter(mode, p2_empty, ws):
    """At M = N = 256 with both transforms and int4 per-token codes the pipelined kernel
    hands out slices at run time from a counter in the workspace (256 bytes); the other
    256 x 256 plans keep a zero workspace."""
    assert plan(problem(40, 256, 256, mode=mode, p2_empty=p2_empty)) == (OK, ws)


@pytest.mark.parametrize("M,N,mode,kernel", [(64, 64, "int32", 2), (64, 128, "int4", 2), (128, 64, "int32", 2),
                                            (64, 128, "int8", 2), (128, 128, "int32", 2), (128, 128, "fp4", 2),
                                            (64, 128, "fp4", 2), (86, 128, "int4", 2), (128, 256, "fp4", 3),
                                            (112, 128, "int4", 2), (128, 128, "e4m3", 2), (128, 136, "int32", 3),
                                            (17, 24, "int32", 2), (86, 64, "int4", 2), (33, 40, "int8", 2),
                                            (3, 8, "int32", 2), (40, 120, "e5m2", 2), (17, 34, "int4", 1),
                                            (33, 30, "int4", 1), (129, 64, "int32", 3), (17, 32, "fp4", 2),
                                            (86, 128, "fp4", 2), (17, 48, "fp4", 1), (129, 32, "fp4", 3),
                                            (224, 128, "int4", 3), (256, 200, "e5m2", 3), (3, 256, "int8", 3),
                                            (200, 130, "int4", 1), (224, 48, "fp4", 1), (130, 34, "int4", 1),
                                            (256, 96, "fp4", 3)])
def test_automatic_kernel_by_shape(M, N, mode, kernel):
    """The one-wave-per-slice MFMA kernel takes per-token slices up to 128 x 128 (one wave
    per SIMD above 4096 elements, two passes over GEMM2 above 8192), padded to its sizes when
    N is a multiple of 8, and per-group ones up to 128 x 128 (one wave per SIMD above 8192),
    M padded when N is 32, 64 or 128.  Slices with a side above 128 run the two-sided 256 x 256
    kernel padded, when N is a multiple of 8 (per group: of 32).  Other shapes take the
    generic kernel."""
    st, ws, ex = fq.fq_get_workspace_size(*[problem(3, M, N, mode=mode)[k] for k in ("x", "p1", "p2")], 1.0, 0.0,
                                          problem(3, M, N, mode=mode)["out"], problem(3, M, N, mode=mode)["sc"])
    assert st == OK
    assert fq.fq_executor_kernel(ex) == kernel
    fq.fq_executor_destroy(ex)


def test_example_problem_from_page_plans():
    # fp16 x [16,16,16], P [16,16], out INT32 [16,16,2], scale [16], clip 1.0, dstTypeMax 0.0
    assert plan(problem(16, 16, 16, fq.DT_FLOAT16, "int32")) == (OK, 0)


@pytest.mark.parametrize("which", ["x", "p1", "p2", "out", "sc"])
def test_null_tensor_is_161001(which):
    p = problem()
    p[which] = None
    assert plan(p)[0] == NULLP
    p = problem()
    p[which] = tens(p[which].dtype, list(p[which].shape)[: p[which].ndim], data=0)
    assert plan(p)[0] == NULLP


def test_null_out_params_are_161001():
    p = problem()
    P = ctypes.byref
    ws = ctypes.c_uint64()
    ex = ctypes.c_void_p()
    assert fq.lib.fq_get_workspace_size(P(p["x"]), P(p["p1"]), P(p["p2"]), 1.0, 0.0, P(p["out"]),
                                        P(p["sc"]), None, P(ex)) == NULLP
    assert fq.lib.fq_get_workspace_size(P(p["x"]), P(p["p1"]), P(p["p2"]), 1.0, 0.0, P(p["out"]),
                                        P(p["sc"]), P(ws), None) == NULLP


def test_null_beats_invalid():
    p = problem()
    p["out"] = None
    assert plan(p, clip=5.0)[0] == NULLP


@pytest.mark.parametrize("clip", [0.0, -0.5, 1.0000001, 2.0, float("nan"), float("inf")])
def test_clip_ratio_range(clip):
    assert plan(problem(), clip=clip)[0] == INVAL


@pytest.mark.parametrize("clip", [1e-6, 0.5, 0.9, 1.0])
def test_clip_ratio_ok(clip):
    assert plan(problem(), clip=clip)[0] == OK


@pytest.mark.parametrize("K,M,N", [(0, 16, 16), (262145, 16, 16), (4, 0, 16), (4, 257, 16),
                                   (4, 16, 0), (4, 16, 264)])
def test_x_dimension_ranges(K, M, N):
    p = problem()
    p["x"] = tens(fq.DT_BFLOAT16, (K, M, N))
    assert plan(p)[0] == INVAL


def test_x_dimension_extremes_ok():
    assert plan(problem(262144, 1, 8))[0] == OK
    assert plan(problem(1, 256, 256))[0] == OK
    assert plan(problem(1, 1, 2, mode="fp4"))[0] == OK


def test_order_clip_before_dtype():
    # both clipRatio and the P1 dtype are wrong; either way 161002 (same class)
    p = problem()
    p["p1"] = tens(fq.DT_FLOAT16, (16, 16))
    assert plan(p, clip=0.0)[0] == INVAL


@pytest.mark.parametrize("bad", ["xdt", "p1dt", "p2dt", "p1shape", "p2shape", "xndim"])
def test_dtype_and_shape_rules(bad):
    p = problem()
    if bad == "xdt":
        p["x"] = tens(fq.DT_FLOAT32, (4, 16, 16))
    elif bad == "p1dt":
        p["p1"] = tens(fq.DT_FLOAT16, (16, 16))
    elif bad == "p2dt":
        p["p2"] = tens(fq.DT_FLOAT16, (16, 16))
    elif bad == "p1shape":
        p["p1"] = tens(fq.DT_BFLOAT16, (16, 8))
    elif bad == "p2shape":
        p["p2"] = tens(fq.DT_BFLOAT16, (8, 8))
    elif bad == "xndim":
        p["x"] = tens(fq.DT_BFLOAT16, (4, 256))
    assert plan(p)[0] == INVAL


def test_out_shape_rules():
    p = problem(N=12, mode="int32")  # N % 8 != 0
    p["out"] = tens(fq.DT_INT32, (4, 16, 1))
    assert plan(p)[0] == INVAL
    p = problem(N=16, mode="int32")
    p["out"] = tens(fq.DT_INT32, (4, 16, 4))
    assert plan(p)[0] == INVAL
    p = problem(M=4, N=6, mode="int4")  # INT4 needs N even and out == x's shape
    assert plan(p)[0] == OK
    p["out"] = tens(fq.DT_INT4, (4, 4, 5))
    assert plan(p)[0] == INVAL
    p = problem(M=4, N=5, mode="fp4")
    p["out"] = tens(fq.DT_FLOAT4_E2M1, (4, 20))
    assert plan(p)[0] == INVAL  # N odd
    p = problem(M=4, N=6, mode="fp4")
    p["out"] = tens(fq.DT_FLOAT4_E2M1, (4, 4, 6))
    assert plan(p)[0] == INVAL  # FLOAT4_E2M1 out is 2-D [K, M*N]


def test_scale_rules():
    p = problem(mode="int32")
    p["sc"] = tens(fq.DT_FLOAT8_E8M0, (4, 4, 2))
    assert plan(p)[0] == INVAL
    p = problem(mode="int32")
    p["sc"] = tens(fq.DT_FLOAT32, (4, 1))
    assert plan(p)[0] == INVAL
    p = problem(mode="fp4")
    p["sc"] = tens(fq.DT_FLOAT32, (4,))  # not the [K] FP32 habit in the per-group mode
    assert plan(p)[0] == INVAL
    p = problem(M=3, N=32, mode="fp4")  # 96 elements: ceilDiv(96, 64) = 2
    assert plan(p)[0] == OK
    p["sc"] = tens(fq.DT_FLOAT8_E8M0, (4, 1, 2))
    assert plan(p)[0] == INVAL


def test_p2_empty_only_for_per_group():
    assert plan(problem(mode="fp4", p2_empty=True))[0] == OK
    assert plan(problem(mode="int32", p2_empty=True))[0] == INVAL
    assert plan(problem(mode="int4", p2_empty=True))[0] == INVAL


@pytest.mark.parametrize("dmax,ok", [(0.0, True), (6.0, True), (8.0, True), (12.0, True), (5.99, False),
                                     (12.01, False), (-1.0, False), (3.0, False),
                                     (float("nan"), False)])
def test_dst_type_max_values(dmax, ok):
    for mode in ("fp4", "int32"):  # validated in every mode, used by fp4 only
        assert plan(problem(mode=mode), dmax=dmax)[0] == (OK if ok else INVAL)


def test_strided_inputs_get_a_workspace():
    # x with a unit innermost stride and 16-byte slice / row strides is read in place
    p = problem()
    p["x"] = tens(fq.DT_BFLOAT16, (4, 16, 16), (16, 64 * 16, 1))  # K and M axes swapped
    assert plan(p) == (OK, 0)
    p["x"] = tens(fq.DT_BFLOAT16, (4, 16, 16), (16 * 24, 24, 1))  # padded rows
    assert plan(p) == (OK, 0)
    # otherwise it is gathered into the workspace
    for strides in [(512, 32, 2), (16 * 17, 17, 1), (16 * 16 + 4, 16, 1)]:
        p["x"] = tens(fq.DT_BFLOAT16, (4, 16, 16), strides)
        st, ws = plan(p)
        assert st == OK and ws >= 4 * 16 * 16 * 2, strides
    # the 256-class kernel always reads a gathered x
    p = problem(K=2, M=256, N=256, mode="int4")
    p["x"] = tens(fq.DT_BFLOAT16, (2, 256, 256), (256 * 264, 264, 1))
    st, ws = plan(p)
    assert st == OK and ws >= 2 * 256 * 256 * 2
    p = problem()
    p["p2"] = tens(fq.DT_BFLOAT16, (16, 16), (1, 16))  # transposed view
    st, ws = plan(p)
    assert st == OK and ws >= 16 * 16 * 2


def test_strided_outputs():
    p = problem(mode="int4")
    p["out"] = tens(fq.DT_INT4, (4, 16, 16), (2 * 16 * 32, 32, 1))  # padded rows
    st, ws = plan(p)
    assert st == OK and ws >= 4 * 16 * 16 // 2
    p["out"] = tens(fq.DT_INT4, (4, 16, 16), (16 * 16, 16, 2))  # nibble-strided innermost
    assert plan(p)[0] == INVAL
    p["out"] = tens(fq.DT_INT4, (4, 16, 16), (16 * 17, 17, 1))  # odd row stride
    assert plan(p)[0] == INVAL


def test_negative_stride_rejected():
    p = problem()
    p["x"] = tens(fq.DT_BFLOAT16, (4, 16, 16), (256, -16, 1))
    assert plan(p)[0] == INVAL


def test_run_argument_checks_without_device():
    p = problem()
    st, ws, ex = fq.fq_get_workspace_size(p["x"], p["p1"], p["p2"], 1.0, 0.0, p["out"], p["sc"])
    assert st == OK
    assert fq.fq_run(0, 0, 0, 0) == NULLP  # NULL executor
    # a strided problem needs its workspace
    p2 = problem()
    p2["x"] = tens(fq.DT_BFLOAT16, (4, 16, 16), (512, 32, 2))
    st, ws2, ex2 = fq.fq_get_workspace_size(p2["x"], p2["p1"], p2["p2"], 1.0, 0.0, p2["out"], p2["sc"])
    assert st == OK and ws2 > 0
    assert fq.fq_executor_set_repeatable(ex2, True) == OK
    assert fq.fq_run(0, ws2, ex2, 0) == NULLP          # NULL workspace while needed
    assert fq.fq_run(DUMMY, ws2 - 1, ex2, 0) == INVAL  # too small
    fq.fq_executor_destroy(ex2)
    assert fq.fq_executor_set_repeatable(ex2, True) == INVAL  # released
    # single-use executor: released by fq_run even when it fails (here: no device).  The
    # dummy pointers must never reach a kernel, so this part runs only without a GPU.
    if _no_gpu():
        st = fq.fq_run(0, 0, ex, 0)
        assert st == fq.FQ_ERR_RUNTIME
        assert fq.fq_run(0, 0, ex, 0) == INVAL
        assert fq.fq_executor_kernel(ex) < 0
    else:
        fq.fq_executor_destroy(ex)


def test_run_no_alloc_argument_checks_without_device():
    """fq_run_no_alloc: NULL and dead executors, and a planned workspace above its 64 MiB
    scratch, are rejected before any HIP call; a rejected single-use executor is released."""
    assert fq.fq_run_no_alloc(0, 0) == NULLP
    p = problem()
    # a strided x of 262144 x 16 x 16 bf16 stages 128 MiB through the workspace
    p["x"] = tens(fq.DT_BFLOAT16, (262144, 16, 16), (512, 32, 2))
    p["out"] = tens(fq.DT_INT32, (262144, 16, 2))
    p["sc"] = tens(fq.DT_FLOAT32, (262144,))
    st, ws, ex = fq.fq_get_workspace_size(p["x"], p["p1"], p["p2"], 1.0, 0.0, p["out"], p["sc"])
    assert st == OK and ws > fq.NO_ALLOC_SCRATCH_BYTES
    assert fq.fq_run_no_alloc(ex, 0) == INVAL
    assert "exceeds" in fq.fq_last_error() and str(ws) in fq.fq_last_error()
    assert fq.fq_run_no_alloc(ex, 0) == INVAL  # released: no longer live
    assert fq.fq_executor_kernel(ex) < 0


def test_kernel_selection_api():
    st, ws, ex = fq.fq_get_workspace_size(*[problem()[k] for k in ("x", "p1", "p2")], 1.0, 0.0,
                                          problem()["out"], problem()["sc"])
    assert st == OK
    assert fq.fq_executor_kernel(ex) in (1, 2, 3)
    assert fq.fq_executor_set_kernel(ex, fq.KERNEL_GENERIC) == OK
    assert fq.fq_executor_kernel(ex) == fq.KERNEL_GENERIC
    assert fq.fq_executor_set_kernel(ex, 99) == INVAL
    assert fq.fq_executor_kernel(ex) == fq.KERNEL_GENERIC
    fq.fq_executor_destroy(ex)
    assert fq.fq_executor_set_kernel(0, 1) == NULLP


def test_status_strings():
    for s in (OK, NULLP, INVAL, fq.FQ_ERR_RUNTIME, 42):
        assert isinstance(fq.status_string(s), str) and fq.status_string(s)


def test_one_hip_runtime_per_process():
    """Importing the binding before torch must not leave two HIP runtimes mapped: torch's
    copy and the system one share a soname, and handles from one are invalid in the other."""
    code = ("import flatquant_transform_quant_amd, torch\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(paths))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"


# ---------------------------------------------------------------- fq_dequant arguments
# (every case is rejected before any HIP call, so no pointer is ever dereferenced)

def dq_args(mode="int32", K=4, M=16, N=16, dt=fq.DT_BFLOAT16):
    out = tens(dt, (K, M, N))
    if mode == "int32":
        return tens(fq.DT_INT32, (K, M, N // 8)), tens(fq.DT_FLOAT32, (K,)), out
    if mode == "int4":
        return tens(fq.DT_INT4, (K, M, N)), tens(fq.DT_FLOAT32, (K,)), out
    return tens(fq.DT_FLOAT4_E2M1, (K, M * N)), tens(fq.DT_FLOAT8_E8M0, (K, -(-(M * N) // 64), 2)), out


def test_dequant_null_is_161001():
    c, s, o = dq_args()
    assert fq.fq_dequant(None, s, o, 0) == NULLP
    assert fq.fq_dequant(c, None, o, 0) == NULLP
    assert fq.fq_dequant(c, s, None, 0) == NULLP
    assert fq.fq_dequant(c, s, tens(fq.DT_BFLOAT16, (4, 16, 16), data=0), 0) == NULLP


@pytest.mark.parametrize("case", ["out_dtype", "out_rank", "K0", "M257", "codes_shape", "codes_dtype",
                                  "scale_dtype", "scale_shape", "e8m0_shape", "strided_out",
                                  "strided_codes", "misaligned_out", "int32_N", "mixed_mode"])
def test_dequant_invalid_is_161002(case):
    c, s, o = dq_args("fp4" if case in ("e8m0_shape", "mixed_mode") else "int32")
    if case == "out_dtype":
        o = tens(fq.DT_FLOAT32, (4, 16, 16))
    elif case == "out_rank":
        o = tens(fq.DT_BFLOAT16, (4, 256))
    elif case == "K0":
        c, s, o = tens(fq.DT_INT32, (0, 16, 2)), tens(fq.DT_FLOAT32, (0,)), tens(fq.DT_BFLOAT16, (0, 16, 16))
    elif case == "M257":
        c, s, o = dq_args("int32", M=257)
    elif case == "codes_shape":
        c = tens(fq.DT_INT32, (4, 16, 4))
    elif case == "codes_dtype":
        c = tens(fq.DT_FLOAT32, (4, 16, 2))
    elif case == "scale_dtype":
        s = tens(fq.DT_FLOAT8_E8M0, (4,))
    elif case == "scale_shape":
        s = tens(fq.DT_FLOAT32, (5,))
    elif case == "e8m0_shape":
        s = tens(fq.DT_FLOAT8_E8M0, (4, 3, 2))
    elif case == "strided_out":
        o = tens(fq.DT_BFLOAT16, (4, 16, 16), (512, 32, 1))
    elif case == "strided_codes":
        c = tens(fq.DT_INT32, (4, 16, 2), (64, 4, 1))
    elif case == "misaligned_out":
        o = tens(fq.DT_BFLOAT16, (4, 16, 16), data=DUMMY + 2)
    elif case == "int32_N":
        c, s, o = tens(fq.DT_INT32, (4, 16, 1)), tens(fq.DT_FLOAT32, (4,)), tens(fq.DT_BFLOAT16, (4, 16, 12))
    elif case == "mixed_mode":
        s = tens(fq.DT_FLOAT32, (4,))
    assert fq.fq_dequant(c, s, o, 0) == INVAL


# ---------------------------------------------------------------- the V1 form
# ([FQV2] V1 还是 V2: V2 with dstTypeMax 0.0 behaves as V1)

@pytest.mark.parametrize("mode", ["int32", "int4", "fp4"])
@pytest.mark.parametrize("bad", [None, "clip", "dims", "p1", "out", "scale", "null"])
def test_v1_form_matches_v2_with_dst_type_max_zero(mode, bad):
    p = problem(mode=mode)
    clip = 1.0
    if bad == "clip":
        clip = 1.5
    elif bad == "dims":
        p["x"] = tens(fq.DT_BFLOAT16, (4, 300, 16))
    elif bad == "p1":
        p["p1"] = tens(fq.DT_FLOAT16, (16, 16))
    elif bad == "out":
        p["out"] = tens(fq.DT_INT32, (4, 16, 3))
    elif bad == "scale":
        p["sc"] = tens(fq.DT_FLOAT32, (5,))
    elif bad == "null":
        p["out"] = None
    st1, ws1, ex1 = fq.fq_v1_get_workspace_size(p["x"], p["p1"], p["p2"], clip, p["out"], p["sc"])
    st2, ws2, ex2 = fq.fq_get_workspace_size(p["x"], p["p1"], p["p2"], clip, 0.0, p["out"], p["sc"])
    for ex in (ex1, ex2):
        if ex:
            fq.fq_executor_destroy(ex)
    assert (st1, ws1) == (st2, ws2)
    assert (st1 == OK) == (bad is None)


# ---------------------------------------------------------------- fq_mx_gemm arguments
# (rejected before any HIP call)

def mx_args(T=4, O=8, H=256, cdt=fq.DT_BFLOAT16):
    G = -(-H // 64)
    return [tens(fq.DT_FLOAT4_E2M1, (T, H)), tens(fq.DT_FLOAT8_E8M0, (T, G, 2)), tens(fq.DT_FLOAT4_E2M1, (O, H)),
            tens(fq.DT_FLOAT8_E8M0, (O, G, 2)), tens(cdt, (T, O))]


@pytest.mark.parametrize("which", range(5))
def test_mx_gemm_null_is_161001(which):
    args = mx_args()
    args[which] = None
    assert fq.fq_mx_gemm(*args, 0) == NULLP


@pytest.mark.parametrize("case", ["H_not_128", "H_mismatch", "a_dtype", "scale_shape", "c_shape", "c_dtype",
                                  "strided_a", "misaligned_a", "too_big"])
def test_mx_gemm_invalid_is_161002(case):
    args = mx_args()
    if case == "H_not_128":
        args = mx_args(H=192)
    elif case == "H_mismatch":
        args[2] = tens(fq.DT_FLOAT4_E2M1, (8, 384))
    elif case == "a_dtype":
        args[0] = tens(fq.DT_INT4, (4, 256))
    elif case == "scale_shape":
        args[1] = tens(fq.DT_FLOAT8_E8M0, (4, 3, 2))
    elif case == "c_shape":
        args[4] = tens(fq.DT_BFLOAT16, (8, 4))
    elif case == "c_dtype":
        args[4] = tens(fq.DT_FLOAT16, (4, 8))
    elif case == "strided_a":
        args[0] = tens(fq.DT_FLOAT4_E2M1, (4, 256), (512, 1))
    elif case == "misaligned_a":
        args[0] = tens(fq.DT_FLOAT4_E2M1, (4, 256), data=DUMMY + 8)
    elif case == "too_big":
        args = mx_args(T=1 << 18, H=1 << 14)
    assert fq.fq_mx_gemm(*args, 0) == INVAL


# ---------------------------------------------------------------- 8-bit per-token outputs
# (dynamic per-row quantization of the dequant_swiglu_quant page, section 3.4)

@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
def test_8bit_outputs_shape_scale_and_p2_rules(mode):
    dt = fq.BYTE_MODES[mode]
    assert plan(problem(K=3, M=5, N=7, mode=mode)) == (OK, 0)  # any N: one code a byte
    p = problem(mode=mode)
    p["out"] = tens(dt, (4, 16 * 16))  # must be [K, M, N]
    assert plan(p)[0] == INVAL
    p = problem(mode=mode)
    p["out"] = tens(dt, (4, 16, 8))
    assert plan(p)[0] == INVAL
    p = problem(mode=mode)
    p["sc"] = tens(fq.DT_FLOAT8_E8M0, (4, 4, 2))  # per-token scales are FLOAT32 [K]
    assert plan(p)[0] == INVAL
    p = problem(mode=mode)
    p["sc"] = tens(fq.DT_FLOAT32, (5,))
    assert plan(p)[0] == INVAL
    assert plan(problem(mode=mode, p2_empty=True))[0] == INVAL  # [0, 0] P2 is per-group only
    assert plan(problem(mode=mode), clip=1.5)[0] == INVAL
    assert plan(problem(mode=mode), dmax=5.0)[0] == INVAL  # validated in every mode


@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
def test_8bit_strided_output_is_staged_in_the_workspace(mode):
    p = problem(K=4, M=16, N=16, mode=mode)
    p["out"] = tens(fq.BYTE_MODES[mode], (4, 16, 16), (16 * 32, 32, 1))  # padded rows
    st, ws = plan(p)
    assert st == OK and ws >= 4 * 16 * 16


def test_8bit_modes_pick_a_kernel_by_shape():
    # (48 x 40 runs padded to 64 x 64; N = 36 is not a multiple of 8)
    for M, N, want in [(64, 64, 2), (32, 128, 2), (256, 256, 3), (48, 40, 2), (48, 36, 1)]:
        p = problem(K=8, M=M, N=N, mode="int8")
        st, ws, ex = fq.fq_get_workspace_size(p["x"], p["p1"], p["p2"], 1.0, 0.0, p["out"], p["sc"])
        assert st == OK
        k = fq.lib.fq_executor_kernel(ex)
        fq.fq_executor_destroy(ex)
        assert k == want, (M, N, k)


@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
def test_dequant_8bit_codes_arguments(mode):
    """8-bit codes: [K, M, N] one byte a code with FLOAT32 [K] scales; other shapes, e8m0
    scales or a wrong scale count are rejected before any HIP call."""
    dt = fq.BYTE_MODES[mode]
    o = tens(fq.DT_BFLOAT16, (4, 16, 16))
    s = tens(fq.DT_FLOAT32, (4,))
    assert fq.fq_dequant(tens(dt, (4, 16, 8)), s, o, 0) == INVAL
    assert fq.fq_dequant(tens(dt, (4, 256)), s, o, 0) == INVAL
    assert fq.fq_dequant(tens(dt, (4, 16, 16)), tens(fq.DT_FLOAT8_E8M0, (4, 4, 2)), o, 0) == INVAL
    assert fq.fq_dequant(tens(dt, (4, 16, 16)), tens(fq.DT_FLOAT32, (3,)), o, 0) == INVAL
    assert fq.fq_dequant(tens(dt, (4, 16, 16), (512, 32, 1)), s, o, 0) == INVAL  # contiguous only
    assert fq.fq_dequant(None, s, o, 0) == NULLP


# ---------------------------------------------------------------- fq_int4_gemm arguments

def i4_args(T=32, O=16, H=256, cdt=fq.DT_BFLOAT16):
    return (tens(fq.DT_INT4, (T, H)), tens(fq.DT_FLOAT32, (T,)), tens(fq.DT_INT4, (O, H)),
            tens(fq.DT_FLOAT32, (O,)), tens(cdt, (T, O)))


def test_int4_gemm_arguments():
    """Rejected before any HIP call: NULLs, H not a multiple of 128, mismatched H, wrong
    scale shapes or dtypes, a C of another shape or dtype, e2m1 codes, strided operands."""
    a, sa, w, sw, c = i4_args()
    assert fq.fq_int4_gemm(None, sa, w, sw, c, 0) == NULLP
    assert fq.fq_int4_gemm(a, sa, w, sw, tens(fq.DT_BFLOAT16, (32, 16), data=0), 0) == NULLP
    bad = [
        (tens(fq.DT_INT4, (32, 192)), sa, tens(fq.DT_INT4, (16, 192)), sw, c),        # H % 128
        (a, sa, tens(fq.DT_INT4, (16, 384)), sw, c),                                   # H differs
        (a, tens(fq.DT_FLOAT32, (31,)), w, sw, c),                                     # scale count
        (a, sa, w, tens(fq.DT_FLOAT8_E8M0, (16,)), c),                                 # scale dtype
        (a, sa, w, sw, tens(fq.DT_FLOAT16, (32, 16))),                                 # C dtype
        (a, sa, w, sw, tens(fq.DT_BFLOAT16, (16, 32))),                                # C shape
        (tens(fq.DT_FLOAT4_E2M1, (32, 256)), sa, w, sw, c),                            # codes dtype
        (tens(fq.DT_INT4, (32, 256), (512, 1)), sa, w, sw, c),                         # strided
    ]
    for args in bad:
        assert fq.fq_int4_gemm(*args, 0) == INVAL


@pytest.mark.parametrize("M,N,mode,p2_empty,auto,accepts", [
    (256, 256, "fp4", True, 5, {1, 3, 5}),       # left-only E2M1: the streaming kernel
    (256, 256, "fp4", False, 3, {1, 3}),         # two-sided E2M1: the whole-workgroup kernel
    (256, 256, "int4", False, 4, {1, 3, 4}),     # two-sided per-token int4: the pipelined kernel
    (256, 256, "int8", False, 3, {1, 3}),
    (128, 256, "fp4", True, 3, {1, 3}),          # a side above 128: padded in the whole-workgroup kernel
    (224, 128, "int4", False, 3, {1, 3}),        # (the pipelined and streaming kernels need 256 x 256)
    (200, 48, "fp4", False, 1, {1}),             # per group padding needs N a multiple of 32
    (128, 128, "fp4", True, 2, {1, 2}),
])
def test_256_class_kernels_by_mode_and_transforms(M, N, mode, p2_empty, auto, accepts):
    """Which variants accept a plan (fq_executor_set_kernel returns success) and which one the
    automatic choice takes: the streaming kernel (5) only for 256 x 256 slices with an empty
    P2 and E2M1 codes, the pipelined one (4) only for 256 x 256 two-sided per-token int4,
    the whole-workgroup kernel (3) also for padded slices with a side above 128."""
    p = problem(3, M, N, mode=mode, p2_empty=p2_empty)
    st, ws, ex = fq.fq_get_workspace_size(p["x"], p["p1"], p["p2"], 1.0, 0.0, p["out"], p["sc"])
    assert st == OK
    try:
        assert fq.fq_executor_kernel(ex) == auto
        for k in range(1, 6):
            got = fq.fq_executor_set_kernel(ex, k)
            assert (got == OK) == (k in accepts), (k, got)
        assert fq.fq_executor_set_kernel(ex, 0) == OK and fq.fq_executor_kernel(ex) == auto
    finally:
        fq.fq_executor_destroy(ex)


def test_run_on_another_stream_records_the_workspace_on_it(monkeypatch):
    """The binding allocates a planned call's workspace (here the slice counter of the
    256 x 256 per-token kernel) on the planning thread's current stream.  Run on another
    stream, it must mark the workspace as in use there before the kernels are enqueued, or
    the caching allocator could hand it to the allocating stream while they still run
    (quantize() drops its executor, and so the workspace, as soon as it returns)."""
    import torch
    K, M, N = 4, 256, 256
    x = torch.zeros((K, M, N), dtype=torch.bfloat16)
    p1 = torch.zeros((M, M), dtype=torch.bfloat16)
    p2 = torch.zeros((N, N), dtype=torch.bfloat16)
    out, sc = fq.empty_outputs(K, M, N, "int4", device="cpu")
    ex = fq.Executor(x, p1, p2, out, sc, "int4", 0.95)
    assert ex.workspace_size > 0 and ex.workspace is not None
    events = []

    class Workspace:
        def data_ptr(self):
            return 0x20000

        def record_stream(self, s):
            events.append(("record_stream", s))

    class Stream:
        cuda_stream = 0x1234

    def fake_run(wsp, size, handle, stream):
        events.append(("fq_run", wsp, size, stream))
        return fq.FQ_SUCCESS

    side = Stream()
    ex.workspace = Workspace()
    monkeypatch.setattr(fq, "fq_run", fake_run)
    try:
        ex.run(stream=side)
        ex.run(stream=side)  # the allocator keeps the stream: no second record
    finally:
        ex.destroy()
    run = ("fq_run", 0x20000, ex.workspace_size, 0x1234)
    assert events == [("record_stream", side), run, run]
