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
import oracle
import synth
from oracle.compare import compare
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
    (32, 16, "int4"), (64, 16, "int32"), (128, 16, "int4"),  # N = 16 on the small MFMA kernel
    (128, 64, "int32"),  # with (64, 128): one wave per SIMD on the small MFMA kernel
    (86, 64, "int4"), (56, 64, "int32"), (40, 120, "int32"), (9, 8, "int4"),  # padded on it
    (112, 128, "int4"), (86, 128, "int32"), (100, 96, "int4"),  # two passes over GEMM2 on it
    (224, 128, "int32"), (129, 136, "int4"), (256, 200, "int4"),  # padded on the 256 x 256 kernel
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
    (128, 128, True, 0.0), (128, 128, False, 8.0),  # one wave per SIMD on the small MFMA kernel
    (86, 128, True, 0.0), (17, 32, False, 8.0), (33, 64, True, 12.0),  # M padded on it
    (224, 128, True, 0.0), (129, 160, True, 6.0), (256, 96, False, 8.0), (160, 256, False, 0.0),  # padded, 256 x 256
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
                                            (16, 16, "int4", fq.KERNEL_MFMA_SMALL),
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


@pytest.mark.parametrize("K", [1, 255, 256, 257, 700, 32768])
def test_pipelined_kernel_writes_every_slice(K):
    """The pipelined 256 x 256 kernel hands out slices at run time from a counter in the
    workspace (zeroed by the library before each launch): on two runs of one executor, with
    the workspace filled with 0xFF bytes first and the outputs with a marker before each
    run, every slice's scale and codes are written, and they equal those of the two-sided
    256-class kernel, which walks a fixed share of the slices per workgroup."""
    w = synth.WORKLOADS["c4"]
    say(f"[gpu] pipelined kernel, every slice, K={K}")
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d, p2d = to_dev(x, w.dtype), to_dev(p1, w.dtype), to_dev(p2, w.dtype)
    ref = fetch(*run_lib(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max, fq.KERNEL_MFMA_WIDE), w.mode, K)
    out, sc = fq.empty_outputs(K, w.M, w.N, w.mode, DEV)
    ex = fq.Executor(xd, p1d, p2d, out, sc, w.mode, w.clip_ratio, w.dst_type_max, kernel=fq.KERNEL_MFMA_WIDE_T)
    assert ex.kernel == fq.KERNEL_MFMA_WIDE_T and ex.workspace_size > 0
    ex.workspace.fill_(0xFF)
    for run in range(2):
        out.view(torch.uint8).fill_(0xEE)
        sc.fill_(float("nan"))
        ex.run()
        torch.cuda.synchronize()
        packed, scale = fetch(out, sc, w.mode, K)
        assert not np.isnan(scale).any(), f"run {run}: {int(np.isnan(scale).sum())} slices without a scale"
        unwritten = int((packed == 0xEE).all(axis=1).sum())
        assert unwritten == 0, f"run {run}: {unwritten} slices without codes"
        assert np.array_equal(packed, ref[0]) and np.array_equal(scale, ref[1]), f"run {run}"
    ex.destroy()


@pytest.mark.parametrize("M,N,mode,K", [(33, 40, "int4", 1031), (86, 64, "int32", 300), (17, 24, "int8", 517),
                                         (40, 120, "int4", 257), (3, 8, "int32", 700), (100, 16, "e4m3", 129),
                                         (112, 128, "int4", 300), (128, 128, "int8", 130), (86, 128, "e5m2", 77)])
def test_padded_shapes_on_the_small_kernel(M, N, mode, K):
    """Per-token slices of other sizes (M up to 128, N a multiple of 8 up to 128) run the
    one-wave-per-slice MFMA kernel padded to its next sizes: every slice against the oracle at
    a K that leaves a ragged last pass (a slice's codes need not be a multiple of 16 bytes),
    and nothing written outside the outputs (4 KB guard bands around them)."""
    say(f"[gpu] padded {M}x{N} {mode} K={K}")
    x, p1, p2 = _inputs(M, N, "bf16", K, seed=M * 1000 + N + 3)
    xd, p1d, p2d = to_dev(x, "bf16"), to_dev(p1, "bf16"), to_dev(p2, "bf16")
    assert fq.KERNEL_MFMA_SMALL in supported_kernels(xd, p1d, p2d, mode, 0.9, 0.0)
    rep = check(x, p1, p2, "bf16", mode, 0.9, 0.0, kernel=fq.KERNEL_MFMA_SMALL, label="padded")
    assert rep["ok"], rep["errors"]
    G = 4096
    ref_out, ref_sc = fq.empty_outputs(K, M, N, mode, DEV)
    nb_out = ref_out.numel() * ref_out.element_size()
    nb_sc = ref_sc.numel() * ref_sc.element_size()
    big_o = torch.full((G + nb_out + G,), 0xA5, dtype=torch.uint8, device=DEV)
    big_s = torch.full((G + nb_sc + G,), 0x5A, dtype=torch.uint8, device=DEV)
    out = big_o[G:G + nb_out].view(ref_out.dtype).reshape(ref_out.shape)
    sc = big_s[G:G + nb_sc].view(ref_sc.dtype).reshape(ref_sc.shape)
    fq.quantize(xd, p1d, p2d, out, sc, mode, 0.9, 0.0, kernel=fq.KERNEL_MFMA_SMALL)
    torch.cuda.synchronize()
    bo, bs = big_o.cpu().numpy(), big_s.cpu().numpy()
    assert (bo[:G] == 0xA5).all() and (bo[G + nb_out:] == 0xA5).all()
    assert (bs[:G] == 0x5A).all() and (bs[G + nb_sc:] == 0x5A).all()


@pytest.mark.parametrize("M,N,two_sided,dmax,K", [(86, 128, True, 0.0, 300), (33, 32, False, 8.0, 517),
                                                   (100, 64, True, 6.0, 257), (5, 128, False, 0.0, 1031)])
def test_padded_per_group_on_the_small_kernel(M, N, two_sided, dmax, K):
    """Per-group slices with M up to 128 and N of 32, 64 or 128 run the one-wave-per-slice
    MFMA kernel with M padded: every slice's codes and e8m0 bytes against the oracle (an odd
    count of groups ends with the zero pad byte: 33 x 32 has 33), and nothing written outside
    the outputs."""
    say(f"[gpu] padded per group {M}x{N} two_sided={two_sided} dmax={dmax} K={K}")
    x, p1, p2 = _inputs(M, N, "bf16", K, seed=M * 1000 + N + 11, dist="laplace", two_sided=two_sided)
    xd, p1d = to_dev(x, "bf16"), to_dev(p1, "bf16")
    p2d = to_dev(p2, "bf16") if p2 is not None else None
    assert fq.KERNEL_MFMA_SMALL in supported_kernels(xd, p1d, p2d, "fp4", 1.0, dmax)
    rep = check(x, p1, p2, "bf16", "fp4", 1.0, dmax, kernel=fq.KERNEL_MFMA_SMALL, label="padded per group")
    assert rep["ok"], rep["errors"]
    G = 4096
    ref_out, ref_sc = fq.empty_outputs(K, M, N, "fp4", DEV)
    nb_out, nb_sc = ref_out.numel(), ref_sc.numel()
    big_o = torch.full((G + nb_out + G,), 0xA5, dtype=torch.uint8, device=DEV)
    big_s = torch.full((G + nb_sc + G,), 0x5A, dtype=torch.uint8, device=DEV)
    out = big_o[G:G + nb_out].reshape(ref_out.shape)
    sc = big_s[G:G + nb_sc].reshape(ref_sc.shape)
    fq.quantize(xd, p1d, p2d, out, sc, "fp4", 1.0, dmax, kernel=fq.KERNEL_MFMA_SMALL)
    torch.cuda.synchronize()
    bo, bs = big_o.cpu().numpy(), big_s.cpu().numpy()
    assert (bo[:G] == 0xA5).all() and (bo[G + nb_out:] == 0xA5).all()
    assert (bs[:G] == 0x5A).all() and (bs[G + nb_sc:] == 0x5A).all()
    # (the pad byte itself: compared with the oracle's zero above through check())


@pytest.mark.parametrize("M,N,mode,two_sided,dmax,dt,K", [
    (224, 128, "int32", True, 0.0, "bf16", 300), (256, 200, "int4", True, 0.0, "f16", 263),
    (3, 256, "int32", True, 0.0, "bf16", 517), (129, 136, "int8", True, 0.0, "bf16", 77),
    (200, 248, "e4m3", True, 0.0, "f16", 40), (136, 256, "e5m2", True, 0.0, "bf16", 33),
    (224, 128, "fp4", True, 0.0, "bf16", 300), (129, 160, "fp4", True, 6.0, "f16", 77),
    (256, 96, "fp4", False, 8.0, "bf16", 257), (160, 256, "fp4", False, 10.0, "f16", 100),
])
def test_padded_shapes_on_the_wide_kernel(M, N, mode, two_sided, dmax, dt, K):
    """Slices with a side above 128 run the two-sided 256 x 256 MFMA kernel padded (an empty
    P2 as the identity): every slice against the oracle, at K past the grid (workgroups with
    one and two slices), and nothing written outside the outputs (4 KB guard bands).  129 x 160
    per group has an odd count of groups, so each slice ends with the zero pad byte."""
    clip = 1.0 if mode == "fp4" else 0.9
    say(f"[gpu] padded wide {M}x{N} {mode} two_sided={two_sided} dmax={dmax} {dt} K={K}")
    x, p1, p2 = _inputs(M, N, dt, K, seed=M * 1000 + N + 13, dist="laplace" if mode == "fp4" else "gauss",
                        two_sided=two_sided)
    xd, p1d = to_dev(x, dt), to_dev(p1, dt)
    p2d = to_dev(p2, dt) if p2 is not None else None
    ks = supported_kernels(xd, p1d, p2d, mode, clip, dmax)
    assert fq.KERNEL_MFMA_WIDE in ks and fq.KERNEL_MFMA_SMALL not in ks
    rep = check(x, p1, p2, dt, mode, clip, dmax, kernel=fq.KERNEL_MFMA_WIDE, label="padded wide")
    assert rep["ok"], rep["errors"]
    G = 4096
    ref_out, ref_sc = fq.empty_outputs(K, M, N, mode, DEV)
    nb_out = ref_out.numel() * ref_out.element_size()
    nb_sc = ref_sc.numel() * ref_sc.element_size()
    big_o = torch.full((G + nb_out + G,), 0xA5, dtype=torch.uint8, device=DEV)
    big_s = torch.full((G + nb_sc + G,), 0x5A, dtype=torch.uint8, device=DEV)
    out = big_o[G:G + nb_out].view(ref_out.dtype).reshape(ref_out.shape)
    sc = big_s[G:G + nb_sc].view(ref_sc.dtype).reshape(ref_sc.shape)
    fq.quantize(xd, p1d, p2d, out, sc, mode, clip, dmax, kernel=fq.KERNEL_MFMA_WIDE)
    torch.cuda.synchronize()
    bo, bs = big_o.cpu().numpy(), big_s.cpu().numpy()
    assert (bo[:G] == 0xA5).all() and (bo[G + nb_out:] == 0xA5).all()
    assert (bs[:G] == 0x5A).all() and (bs[G + nb_sc:] == 0x5A).all()
    # every output byte was written (the guard value survives nowhere inside the outputs
    # unless the codes themselves hold it: compare with the run into fresh buffers)
    o2, s2 = run_lib(xd, p1d, p2d, mode, clip, dmax, fq.KERNEL_MFMA_WIDE)
    assert np.array_equal(bo[G:G + nb_out], o2.contiguous().view(torch.uint8).reshape(-1).cpu().numpy())
    assert np.array_equal(bs[G:G + nb_sc], s2.contiguous().view(torch.uint8).reshape(-1).cpu().numpy())


def test_zero_input_gives_zero_scale_and_codes():
    for n, mode, dmax, two in ((64, "int32", 0.0, True), (64, "fp4", 0.0, True), (64, "fp4", 8.0, True),
                               (256, "fp4", 0.0, False), (256, "fp4", 8.0, False)):
        x = np.zeros((4, n, n), np.uint16)
        p = synth.gen_orthogonal(n, "bf16", 0, 2)
        xd, pd = to_dev(x, "bf16"), to_dev(p, "bf16")
        p2d = pd if two else None
        for k in supported_kernels(xd, pd, p2d, mode, 1.0, dmax):
            out, sc = run_lib(xd, pd, p2d, mode, 1.0, dmax, k)
            packed, scale = fetch(out, sc, mode, 4)
            assert (packed == 0).all() and (scale == 0).all(), (n, mode, dmax, two, k)


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_full_size_sampled(key):
    """The full configuration in the launch the benchmark times, checked on sampled slices
    (first, last, middle and random ones) that the oracle computes one by one."""
    w = synth.WORKLOADS[key]
    say(f"[gpu] generating {key} full size K={w.K}")
    x, p1, p2 = synth.make_inputs(w)
    rng = np.random.default_rng(0)
    # every CU's first and last slice of the persistent walk are among the 256-class samples
    n_rand = 12 if w.M * w.N <= 8192 else 64
    slices = sorted({0, 1, 255, 256, w.K // 2, w.K - 257, w.K - 256, w.K - 2, w.K - 1,
                     *rng.integers(0, w.K, n_rand).tolist()})
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


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
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


@pytest.mark.parametrize("M,N,mode,two_sided", [(64, 64, "int4", True), (33, 40, "int32", True),
                                                (64, 128, "fp4", True), (256, 256, "int4", True),
                                                (64, 64, "e4m3", True), (256, 256, "fp4", False)])
def test_strided_x_in_place_or_gathered(M, N, mode, two_sided):
    """x as a view with padded rows and padded slices (read in place by the generic and
    one-wave-per-slice kernels, gathered for the 256-class kernels), and with a non-unit
    innermost stride (always gathered): the codes and scales equal those of a contiguous x."""
    dt = "bf16"
    K = 9
    x, p1, p2 = _inputs(M, N, dt, K, seed=M * 7 + N, two_sided=two_sided)
    if mode == "int32" and N % 8:
        pytest.skip("INT32 needs N % 8 == 0")
    xd, p1d = to_dev(x, dt), to_dev(p1, dt)
    p2d = to_dev(p2, dt) if two_sided else None
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


@pytest.mark.parametrize("K", [1, 255, 256, 257, 700])
def test_streaming_left_only_kernel_writes_every_slice(K):
    """The streaming 256 x 256 left-only kernel (x through an LDS ring filled by DMA loads,
    nine chunks ahead, across slice boundaries and past K): outputs pre-filled with a marker,
    every slice compared with the oracle, on two runs of one executor."""
    w = synth.WORKLOADS["c5"]
    x, p1, _ = synth.make_inputs(w, 0, K)
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    out, sc = fq.empty_outputs(K, w.M, w.N, w.mode, DEV)
    ex = fq.Executor(xd, p1d, None, out, sc, w.mode, w.clip_ratio, w.dst_type_max, kernel=fq.KERNEL_MFMA_WIDE_L)
    assert ex.kernel == fq.KERNEL_MFMA_WIDE_L
    orc = oracle.run(x, p1, None, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, nthreads=8)
    try:
        for run in range(2):
            say(f"[gpu] streaming left-only kernel K={K} run {run}")
            out.view(torch.uint8).fill_(0xEE)
            sc.view(torch.uint8).fill_(0xEE)
            ex.run()
            torch.cuda.synchronize()
            packed, scale = fetch(out, sc, w.mode, K)
            rep = compare(orc, packed, scale)
            assert rep["ok"], rep["errors"]
    finally:
        ex.destroy()


@pytest.mark.parametrize("dt,dmax", [("f16", 6.0), ("bf16", 0.0)])
def test_streaming_left_only_kernel_other_dtype_and_rules(dt, dmax):
    """The streaming 256 x 256 left-only kernel on K = 257 slices (some workgroups take two)
    in fp16 with the V2 rule by division (dstTypeMax 6) and in bf16 with the V1 rule, every
    slice compared with the oracle."""
    K = 257
    x, p1, _ = _inputs(256, 256, dt, K, seed=11, dist="laplace", frac=0.01, scale=30.0, two_sided=False)
    rep = check(x, p1, None, dt, "fp4", 1.0, dmax, kernel=fq.KERNEL_MFMA_WIDE_L, label=f"streaming {dt} dmax={dmax}")
    assert rep["ok"], rep["errors"]


@pytest.mark.parametrize("M,N,K,mode,two_sided,dmax,kernel", [
    (256, 256, 40000, "int4", True, 0.0, fq.KERNEL_MFMA_WIDE_T),
    (256, 256, 40000, "fp4", True, 8.0, fq.KERNEL_MFMA_WIDE),
    (256, 256, 40000, "fp4", False, 8.0, fq.KERNEL_MFMA_WIDE_L),
    (128, 128, 262144, "int4", True, 0.0, fq.KERNEL_MFMA_SMALL)])
def test_kernels_past_four_gigabytes_of_x(M, N, K, mode, two_sided, dmax, kernel):
    """x spanning more than 4 GB (5.2 GB for 40000 slices of 256 x 256, 8.6 GB for 262144 of
    128 x 128: slice offsets pass 2^31 elements and 2^32 bytes), drawn on the device from a
    seeded normal distribution; the slices on both sides of those offsets and the last ones
    are compared with the oracle (their x copied back)."""
    dt = "bf16"
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    xd = torch.randn((K, M, N), generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    p1 = synth.gen_orthogonal(M, dt, 7, 2)
    p2 = synth.gen_orthogonal(N, dt, 7, 3) if two_sided else None
    p1d, p2d = to_dev(p1, dt), (to_dev(p2, dt) if two_sided else None)
    out, sc = fq.empty_outputs(K, M, N, mode, DEV)
    ex = fq.Executor(xd, p1d, p2d, out, sc, mode, 0.95 if mode == "int4" else 1.0, dmax, kernel=kernel)
    assert ex.kernel == kernel
    say(f"[gpu] K={K} 256x256 {mode} two_sided={two_sided} kernel {kernel}")
    try:
        ex.run()
        torch.cuda.synchronize()
    finally:
        ex.destroy()
    b31 = (1 << 31) // (M * N)  # the first slice at 2^31 elements (2^32 bytes)
    slices = sorted({0, 1, b31 - 1, b31, b31 + 1, K - 257, K - 256, K - 2, K - 1})
    xs = xd[slices].view(torch.int16).cpu().numpy().view(np.uint16)
    del xd
    packed, scale = fetch(out, sc, mode, K)
    orc = oracle.run(xs, p1, p2, dt, mode, 0.95 if mode == "int4" else 1.0, dmax, nthreads=8)
    rep = compare(orc, packed[slices], scale[slices])
    assert rep["ok"], rep["errors"]
    # the dequantized values of the same outputs (2 bytes an element: past 4 GB as well)
    vals = fq.dequantize(out, sc, mode, M, N, torch.bfloat16)
    torch.cuda.synchronize()
    got = vals[slices].view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.dequant(packed[slices], scale[slices], M, N, dt, mode)
    assert np.array_equal(got, want)
