"""fq_run_no_alloc (the second stage with the staging buffer taken from the library's own
device array) against fq_run with a caller-allocated workspace, through the C ABI: the same
bits on non-contiguous inputs and outputs that need staging, on two calls in a row, the second
with a smaller problem (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import flatquant_transform_quant_amd as fq
import synth
from gpu_util import DEV, fetch, say, to_dev

pytestmark = pytest.mark.gpu


def _strided_problem(w, K, mode):
    """x with its K and M axes swapped in memory, P1 / P2 transposed views, padded output
    rows and a strided scale vector: every tensor but P2's storage needs the workspace."""
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d, p2d = to_dev(x, w.dtype), to_dev(p1, w.dtype), to_dev(p2, w.dtype)
    x_s = xd.transpose(0, 1).contiguous().transpose(0, 1)
    p1_s = p1d.t().contiguous().t()
    p2_s = p2d.t().contiguous().t()
    return x_s, p1_s, p2_s


def _outputs(K, M, N, mode):
    if mode == "fp4":
        out_big = torch.zeros((K, M * N // 2 + 32), dtype=torch.uint8, device=DEV)
        out_s = out_big[:, : M * N // 2]
        sc_big = torch.zeros((K, -(-M * N // 64), 2 + 2), dtype=torch.uint8, device=DEV)
        sc_s = sc_big[:, :, 1:3]
    else:
        out_big = torch.zeros((K, M, N // 2 + 16), dtype=torch.uint8, device=DEV)
        out_s = out_big[:, :, : N // 2]
        sc_big = torch.zeros((K, 3), dtype=torch.float32, device=DEV)
        sc_s = sc_big[:, 1]
    return out_s, sc_s


def _plan(x, p1, p2, out, sc, mode, clip, dmax):
    K, M, N = x.shape
    st, ws, ex = fq.fq_get_workspace_size(fq.describe_input(x), fq.describe_input(p1), fq.describe_input(p2),
                                          clip, dmax, fq.describe_out(out, mode, K, M, N),
                                          fq.describe_scale(sc, mode))
    assert st == fq.FQ_SUCCESS and ws > 0
    return ws, ex


@pytest.mark.parametrize("key,mode", [("c2", "int4"), ("c3", "fp4"), ("c4", "int4")])
def test_no_alloc_equals_fq_run_twice_second_smaller(key, mode):
    w = synth.WORKLOADS[key]
    stream = torch.cuda.current_stream().cuda_stream
    for K in (48, 7):  # the second call is smaller: the array still holds the first's data
        x, p1, p2 = _strided_problem(w, K, mode)
        # reference: fq_run with a torch-allocated workspace
        out_r, sc_r = _outputs(K, w.M, w.N, mode)
        ws, ex = _plan(x, p1, p2, out_r, sc_r, mode, w.clip_ratio, w.dst_type_max)
        buf = torch.empty(ws, dtype=torch.uint8, device=DEV)
        assert fq.fq_run(buf.data_ptr(), ws, ex, stream) == fq.FQ_SUCCESS
        # the same problem through the entry point that allocates nothing
        out_n, sc_n = _outputs(K, w.M, w.N, mode)
        ws2, ex2 = _plan(x, p1, p2, out_n, sc_n, mode, w.clip_ratio, w.dst_type_max)
        assert ws2 == ws <= fq.NO_ALLOC_SCRATCH_BYTES
        say(f"[gpu] no-alloc {key} {mode} K={K}: workspace {ws} bytes")
        assert fq.fq_run_no_alloc(ex2, stream) == fq.FQ_SUCCESS, fq.fq_last_error()
        torch.cuda.synchronize()
        ref = fetch(out_r, sc_r, mode, K)
        got = fetch(out_n, sc_n, mode, K)
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_no_alloc_contiguous_problem_needs_no_scratch():
    w = synth.WORKLOADS["c2"]
    K = 16
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d, p2d = to_dev(x, w.dtype), to_dev(p1, w.dtype), to_dev(p2, w.dtype)
    out, sc = fq.empty_outputs(K, w.M, w.N, "int4", DEV)
    st, ws, ex = fq.fq_get_workspace_size(fq.describe_input(xd), fq.describe_input(p1d), fq.describe_input(p2d),
                                          w.clip_ratio, 0.0, fq.describe_out(out, "int4", K, w.M, w.N),
                                          fq.describe_scale(sc, "int4"))
    assert st == fq.FQ_SUCCESS and ws == 0
    assert fq.fq_run_no_alloc(ex, torch.cuda.current_stream().cuda_stream) == fq.FQ_SUCCESS
    out2, sc2 = fq.empty_outputs(K, w.M, w.N, "int4", DEV)
    fq.quantize(xd, p1d, p2d, out2, sc2, "int4", w.clip_ratio, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(sc, sc2)
