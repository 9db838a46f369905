"""GPU parity: libfq (through its C ABI) against the oracle, element by element.

Bar (the tolerance rule of oracle/compare.py): codes and e8m0 scales bit-exact except
where the oracle shows a rounding tie reachable within 1e-6 relative or within the fp32
summation error bound -- there one code step, at most ceil(1e-4 * elements) of them;
per-token fp32 scales within 1e-5 relative.
"""
import numpy as np
import pytest
import torch

import flatquant_transform_quant_amd as fq
import synth
from gpu_util import DEV, check, fetch, run_lib, say, supported_kernels, to_dev

pytestmark = pytest.mark.gpu

SMALL_K = {"c1": 64, "c2": 96, "c3": 40, "c4": 6, "c5": 6}


def _inputs(M, N, dt, K, seed, dist="gauss", frac=0.02, scale=20.0, two_sided=True):
    x = synth.gen_x(M, N, dt, dist, frac, scale, seed=seed, k0=0, k1=K)
    p1 = synth.gen_orthogonal(M, dt, seed, 2)
    p2 = synth.gen_orthogonal(N, dt, seed, 3) if two_sided else None
    return x, p1, p2


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_shapes_every_kernel(key):
    w = synth.WORKLOADS[key]
    K = SMALL_K[key]
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    p2d = to_dev(p2, w.dtype) if p2 is not None else None
    ks = supported_kernels(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max)
    assert fq.KERNEL_GENERIC in ks
    for k in ks:
        rep = check(x, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, kernel=k, label=key)
        assert rep["ok"], rep["errors"]


EDGE_PER_TOKEN = [  # (M, N, mode)
    (1, 8, "int32"), (2, 8, "int32"), (8, 8, "int32"), (16, 16, "int32"), (17, 24, "int32"),
    (31, 32, "int32"), (32, 32, "int32"), (33, 40, "int32"), (255, 16, "int32"), (16, 256, "int32"),
    (64, 64, "int32"), (128, 128, "int32"), (256, 256, "int32"),
    (1, 2, "int4"), (3, 2, "int4"), (17, 34, "int4"), (33, 30, "int4"), (64, 128, "int4"),
    (255, 254, "int4"), (256, 256, "int4"), (128, 256, "int4"),
]


@pytest.mark.parametrize("M,N,mode", EDGE_PER_TOKEN)
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_edge_shapes_per_token(M, N, mode, dt):
    K = 5 if M * N <= 64 * 64 else 3
    x, p1, p2 = _inputs(M, N, dt, K, seed=M * 1000 + N)
    xd, p1d, p2d = to_dev(x, dt), to_dev(p1, dt), to_dev(p2, dt)
    for k in supported_kernels(xd, p1d, p2d, mode, 0.9, 0.0):
        rep = check(x, p1, p2, dt, mode, 0.9, 0.0, kernel=k, label="edge")
        assert rep["ok"], rep["errors"]


EDGE_PER_GROUP = [  # (M, N, two_sided, dmax)
    (1, 2, True, 0.0), (3, 10, True, 0.0), (3, 32, True, 6.0), (5, 6, True, 8.0),
    (17, 18, True, 0.0), (16, 16, True, 0.0), (32, 32, False, 8.0), (64, 128, True, 0.0),
    (64, 128, False, 10.0), (128, 64, True, 12.0), (255, 254, True, 6.0), (256, 256, True, 0.0),
    (256, 256, False, 8.0), (1, 256, False, 0.0), (256, 2, False, 7.0),
]


@pytest.mark.parametrize("M,N,two_sided,dmax", EDGE_PER_GROUP)
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_edge_shapes_per_group(M, N, two_sided, dmax, dt):
    K = 5 if M * N <= 64 * 64 else 3
    x, p1, p2 = _inputs(M, N, dt, K, seed=M * 1000 + N + 7, dist="laplace", two_sided=two_sided)
    xd, p1d = to_dev(x, dt), to_dev(p1, dt)
    p2d = to_dev(p2, dt) if p2 is not None else None
    for k in supported_kernels(xd, p1d, p2d, "fp4", 1.0, dmax):
        rep = check(x, p1, p2, dt, "fp4", 1.0, dmax, kernel=k, label="edge")
        assert rep["ok"], rep["errors"]


def test_k_not_a_multiple_of_the_grid():
    w = synth.WORKLOADS["c2"]
    for K in (1, 7, 257, 1031):
        x, p1, p2 = synth.make_inputs(w, 0, K)
        rep = check(x, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, label="ragged K",
                    slices=sorted({0, K // 2, K - 1}))
        assert rep["ok"], rep["errors"]


@pytest.mark.parametrize("M,N,mode,kernel", [(16, 32, "int32", fq.KERNEL_MFMA_SMALL),
                                            (16, 32, "fp4", fq.KERNEL_MFMA_SMALL),
                                            (1, 8, "int4", fq.KERNEL_GENERIC)])
def test_largest_k(M, N, mode, kernel):
    """K at the library's limit (262144 slices): the persistent kernel's walk over slices and
    the per-slice offsets of codes and scales at the far end, compared with the oracle on
    sampled slices that include the first and the last."""
    K = 262144
    x = synth.gen_x(M, N, "bf16", "gauss", 0.01, 20.0, seed=5, k0=0, k1=K)
    p1, p2 = synth.gen_orthogonal(M, "bf16", 5, 2), synth.gen_orthogonal(N, "bf16", 5, 3)
    rng = np.random.default_rng(5)
    slices = sorted({0, 1, K // 2 - 1, K // 2, K - 2, K - 1, *rng.integers(0, K, 26).tolist()})
    rep = check(x, p1, p2, "bf16", mode, 1.0, 0.0, kernel=kernel, label="largest K", slices=slices)
    assert rep["ok"], rep["errors"]


@pytest.mark.parametrize("key", ["c4", "c5"])
def test_k_ragged_whole_workgroup_kernels(key):
    """M = N = 256 with K leaving some CUs two or three slices and others one: the slice
    loop's later passes, the chunk lookahead across slices and the loads past K."""
    w = synth.WORKLOADS[key]
    for K in (257, 515):
        x, p1, p2 = synth.make_inputs(w, 0, K)
        rep = check(x, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, label=f"{key} ragged K={K}",
                    slices=sorted({0, 1, 255, 256, 257 % K, K // 2, K - 2, K - 1}))
        assert rep["ok"], rep["errors"]


def test_zero_input_gives_zero_scale_and_codes():
    for mode, dmax in (("int32", 0.0), ("fp4", 0.0), ("fp4", 8.0)):
        x = np.zeros((4, 64, 64), np.uint16)
        p = synth.gen_orthogonal(64, "bf16", 0, 2)
        xd, pd = to_dev(x, "bf16"), to_dev(p, "bf16")
        for k in supported_kernels(xd, pd, pd, mode, 1.0, dmax):
            out, sc = run_lib(xd, pd, pd, mode, 1.0, dmax, k)
            packed, scale = fetch(out, sc, mode, 4)
            assert (packed == 0).all() and (scale == 0).all()


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_full_size_sampled(key):
    """The full configuration in the launch the benchmark times, checked on sampled slices
    (first, last, middle and random ones) that the oracle computes one by one."""
    w = synth.WORKLOADS[key]
    say(f"[gpu] generating {key} full size K={w.K}")
    x, p1, p2 = synth.make_inputs(w)
    rng = np.random.default_rng(0)
    n_rand = 12 if w.M * w.N <= 8192 else 4
    slices = sorted({0, 1, w.K // 2, w.K - 2, w.K - 1, *rng.integers(0, w.K, n_rand).tolist()})
    rep = check(x, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, label=f"{key} full",
                slices=slices)
    assert rep["ok"], rep["errors"]


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_deterministic_across_runs_and_streams(key):
    w = synth.WORKLOADS[key]
    K = 512 if w.M * w.N <= 8192 else 32
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    p2d = to_dev(p2, w.dtype) if p2 is not None else None
    for k in supported_kernels(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max):
        ref = fetch(*run_lib(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max, k), w.mode, K)
        for rep in range(2):
            got = fetch(*run_lib(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max, k), w.mode, K)
            assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])
        s = torch.cuda.Stream()
        out, sc = fq.empty_outputs(K, w.M, w.N, w.mode, DEV)
        with torch.cuda.stream(s):
            fq.quantize(xd, p1d, p2d, out, sc, w.mode, w.clip_ratio, w.dst_type_max, stream=s, kernel=k)
        s.synchronize()
        got = fetch(out, sc, w.mode, K)
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c5"])
def test_canary_guards_untouched(key):
    """Outputs placed between 4 KB guard bands: nothing outside them is written."""
    w = synth.WORKLOADS[key]
    K = 33
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    p2d = to_dev(p2, w.dtype) if p2 is not None else None
    G = 4096
    ref_out, ref_sc = fq.empty_outputs(K, w.M, w.N, w.mode, DEV)
    nb_out = ref_out.numel() * ref_out.element_size()
    nb_sc = ref_sc.numel() * ref_sc.element_size()
    for k in supported_kernels(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max):
        big_o = torch.full((G + nb_out + G,), 0xA5, dtype=torch.uint8, device=DEV)
        big_s = torch.full((G + nb_sc + G,), 0x5A, dtype=torch.uint8, device=DEV)
        out = big_o[G:G + nb_out].view(ref_out.dtype).reshape(ref_out.shape)
        sc = big_s[G:G + nb_sc].view(ref_sc.dtype).reshape(ref_sc.shape)
        fq.quantize(xd, p1d, p2d, out, sc, w.mode, w.clip_ratio, w.dst_type_max, kernel=k)
        torch.cuda.synchronize()
        bo, bs = big_o.cpu().numpy(), big_s.cpu().numpy()
        assert (bo[:G] == 0xA5).all() and (bo[G + nb_out:] == 0xA5).all()
        assert (bs[:G] == 0x5A).all() and (bs[G + nb_sc:] == 0x5A).all()


def test_non_contiguous_tensors():
    """Strided x (K and M axes swapped in memory), transposed-view P1/P2, padded rows in the
    int4 output and a strided scale: staged through the workspace, same codes."""
    w = synth.WORKLOADS["c2"]
    K, M, N = 24, w.M, w.N
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d, p2d = to_dev(x, w.dtype), to_dev(p1, w.dtype), to_dev(p2, w.dtype)
    ref_out, ref_sc = run_lib(xd, p1d, p2d, "int4", w.clip_ratio, 0.0)
    ref = fetch(ref_out, ref_sc, "int4", K)
    x_s = xd.transpose(0, 1).contiguous().transpose(0, 1)          # [K, M, N] with strides (N, K*N, 1)
    p1_s = p1d.t().contiguous().t()                                 # strides (1, M)
    p2_s = p2d.t().contiguous().t()
    out_big = torch.zeros((K, M, N // 2 + 16), dtype=torch.uint8, device=DEV)
    out_s = out_big[:, :, : N // 2]                                 # padded rows
    sc_big = torch.zeros((K, 3), dtype=torch.float32, device=DEV)
    sc_s = sc_big[:, 1]                                             # stride 3
    assert not x_s.is_contiguous() and not out_s.is_contiguous() and not sc_s.is_contiguous()
    ex = fq.Executor(x_s, p1_s, p2_s, out_s, sc_s, "int4", w.clip_ratio, 0.0, repeatable=False)
    assert ex.workspace_size > 0
    ex.run()
    torch.cuda.synchronize()
    got = fetch(out_s, sc_s, "int4", K)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    assert (out_big[:, :, N // 2:] == 0).all()


def test_int32_and_int4_layouts_are_byte_identical():
    w = synth.WORKLOADS["c2"]
    K = 16
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d, p2d = to_dev(x, w.dtype), to_dev(p1, w.dtype), to_dev(p2, w.dtype)
    a = fetch(*run_lib(xd, p1d, p2d, "int32", w.clip_ratio, 0.0), "int32", K)
    b = fetch(*run_lib(xd, p1d, p2d, "int4", w.clip_ratio, 0.0), "int4", K)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("key", ["c2", "c3", "c5"])
def test_v1_form_runs_like_v2_with_dst_type_max_zero(key):
    """[FQV2] V1 还是 V2: the V1 call (no dstTypeMax) gives what V2 gives with dstTypeMax 0.0."""
    w = synth.WORKLOADS[key]
    K = 16
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    p2d = to_dev(p2, w.dtype) if p2 is not None else torch.empty((0, 0), dtype=xd.dtype, device=DEV)
    ref = fetch(*run_lib(xd, p1d, p2d if p2 is not None else None, w.mode, w.clip_ratio, 0.0), w.mode, K)
    out, sc = fq.empty_outputs(K, w.M, w.N, w.mode, DEV)
    st, ws, ex = fq.fq_v1_get_workspace_size(fq.describe_input(xd), fq.describe_input(p1d), fq.describe_input(p2d),
                                             w.clip_ratio, fq.describe_out(out, w.mode, K, w.M, w.N),
                                             fq.describe_scale(sc, w.mode))
    assert st == fq.FQ_SUCCESS and ws == 0
    assert fq.fq_run(0, 0, ex, torch.cuda.current_stream().cuda_stream) == fq.FQ_SUCCESS
    torch.cuda.synchronize()
    got = fetch(out, sc, w.mode, K)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


@pytest.mark.parametrize("M,N,mode", [(64, 64, "int4"), (33, 40, "int32"), (64, 128, "fp4"), (256, 256, "int4"),
                                      (64, 64, "e4m3")])
def test_strided_x_in_place_or_gathered(M, N, mode):
    """x as a view with padded rows and padded slices (read in place by the generic and
    one-wave-per-slice kernels, gathered for the 256-class kernel), and with a non-unit
    innermost stride (always gathered): the codes and scales equal those of a contiguous x."""
    dt = "bf16"
    K = 9
    x, p1, p2 = _inputs(M, N, dt, K, seed=M * 7 + N)
    if mode == "int32" and N % 8:
        pytest.skip("INT32 needs N % 8 == 0")
    xd, p1d, p2d = to_dev(x, dt), to_dev(p1, dt), to_dev(p2, dt)
    ref = fetch(*run_lib(xd, p1d, p2d, mode, 0.9, 0.0), mode, K)
    big = torch.zeros((K + 1, M + 3, N + 8), dtype=xd.dtype, device=DEV)
    big[:K, :M, :N] = xd
    views = {"padded": big[:K, :M, :N],
             "innermost stride 2": torch.zeros((K, M, 2 * N), dtype=xd.dtype, device=DEV)}
    views["innermost stride 2"][:, :, 0::2] = xd
    views["innermost stride 2"] = views["innermost stride 2"][:, :, 0::2]
    for name, xv in views.items():
        assert not xv.is_contiguous()
        out, sc = fq.empty_outputs(K, M, N, mode, DEV)
        ex = fq.Executor(xv, p1d, p2d, out, sc, mode, 0.9, 0.0, repeatable=False)
        say(f"[gpu] strided x ({name}) {M}x{N} {mode}: kernel {ex.kernel}, workspace {ex.workspace_size}")
        ex.run()
        torch.cuda.synchronize()
        got = fetch(out, sc, mode, K)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), name
