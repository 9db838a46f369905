"""GPU parity of the per-token 8-bit codes (INT8, FP8 E4M3FN, FP8 E5M2: the dynamic per-row
quantization of the dequant_swiglu_quant page, section 3.4, on the transformed slice) with
the oracle, element by element, under the same rule as the 4-bit modes (oracle/compare.py):
codes equal except one step at a reachable rounding tie (at most ceil(1e-4 * elements)),
the sign of an FP8 zero free where y is within error of 0, scales within 1e-5 relative.
Every kernel that accepts the shape is run: the generic one always, the one-wave-per-slice
MFMA kernel for its shapes (M and N up to 128, N a multiple of 8), the whole-workgroup
MFMA kernel for M = N = 256."""
import numpy as np
import pytest

import flatquant_transform_quant_amd as fq
import synth
from gpu_util import check, fetch, run_lib, say, supported_kernels, to_dev

pytestmark = pytest.mark.gpu

MODES = ["int8", "e4m3", "e5m2"]
SHAPES = [(1, 1), (3, 5), (16, 32), (17, 24), (32, 32), (64, 64), (16, 128), (128, 32), (32, 128),
          (64, 128), (128, 64), (128, 128), (112, 128), (255, 254), (256, 256)]


def _inputs(M, N, dt, K, seed):
    x = synth.gen_x(M, N, dt, "gauss", 0.02, 30.0, seed=seed, k0=0, k1=K)
    return x, synth.gen_orthogonal(M, dt, seed, 2), synth.gen_orthogonal(N, dt, seed, 3)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_8bit_shapes_every_kernel(mode, dt):
    for i, (M, N) in enumerate(SHAPES):
        # (256 x 256: enough slices that the FP8 mismatch count, about 8e-5 of elements
        # against the 1e-4 cap, does not hinge on one slice)
        K = 6 if M * N <= 64 * 64 else (12 if M * N == 65536 else 3)
        x, p1, p2 = _inputs(M, N, dt, K, seed=M * 1000 + N)
        clip = 1.0 if i % 2 == 0 else 0.9
        xd, p1d, p2d = to_dev(x, dt), to_dev(p1, dt), to_dev(p2, dt)
        ks = supported_kernels(xd, p1d, p2d, mode, clip, 0.0)
        assert fq.KERNEL_GENERIC in ks and (fq.KERNEL_MFMA_WIDE in ks) == (M == N == 256)
        for k in ks:
            rep = check(x, p1, p2, dt, mode, clip, 0.0, kernel=k, label=f"8-bit {M}x{N}")
            assert rep["ok"], rep["errors"]


@pytest.mark.parametrize("clip", [127.0 / 127.4998, 127.0 / 127.5002, 0.5])
def test_int8_clamp_threshold_every_kernel(clip):
    """INT8 codes where 127/clipRatio sits just below 127.5 (the kernels then round without
    the clamp, so the largest |y / scale| must still give 127), just above it, and well
    above it (the clamp then bites on every slice's largest elements)."""
    for M, N in [(64, 64), (64, 128), (256, 256)]:
        x, p1, p2 = _inputs(M, N, "bf16", 5, seed=M + N)
        xd, p1d, p2d = to_dev(x, "bf16"), to_dev(p1, "bf16"), to_dev(p2, "bf16")
        for k in supported_kernels(xd, p1d, p2d, "int8", clip, 0.0):
            rep = check(x, p1, p2, "bf16", "int8", clip, 0.0, kernel=k, label=f"int8 clip {clip:.7f} {M}x{N}")
            assert rep["ok"], rep["errors"]


@pytest.mark.parametrize("mode", MODES)
def test_8bit_ragged_k(mode):
    w = synth.WORKLOADS["c2i8"]
    for K in (1, 7, 257, 1031):
        x, p1, p2 = synth.make_inputs(w, 0, K)
        rep = check(x, p1, p2, w.dtype, mode, 1.0, 0.0, label=f"8-bit ragged K={K}",
                    slices=sorted({0, K // 2, K - 1}))
        assert rep["ok"], rep["errors"]


@pytest.mark.parametrize("mode", MODES)
def test_8bit_whole_workgroup_kernel_ragged_k(mode):
    """M = N = 256 (the two-sided 256-class kernel) with K leaving some CUs two or three
    slices and others one, on the 256-class activation workload's distribution."""
    w = synth.WORKLOADS["c4"]
    for K in (257, 515):
        x, p1, p2 = synth.make_inputs(w, 0, K)
        rep = check(x, p1, p2, w.dtype, mode, 1.0, 0.0, kernel=fq.KERNEL_MFMA_WIDE, label=f"8-bit 256 K={K}",
                    slices=sorted({0, 1, 255, 256, 257 % K, K // 2, K - 2, K - 1}))
        assert rep["ok"], rep["errors"]


def test_8bit_zero_input_gives_zero_scale_and_zero_codes():
    for mode in MODES:
        x = np.zeros((4, 64, 64), np.uint16)
        p = synth.gen_orthogonal(64, "bf16", 0, 2)
        xd, pd = to_dev(x, "bf16"), to_dev(p, "bf16")
        for k in supported_kernels(xd, pd, pd, mode, 1.0, 0.0):
            out, sc = run_lib(xd, pd, pd, mode, 1.0, 0.0, k)
            packed, scale = fetch(out, sc, mode, 4)
            assert (scale == 0).all()
            assert ((packed & 0x7F) == 0).all() if mode != "int8" else (packed == 0).all()


@pytest.mark.parametrize("key", ["c2i8", "c2e4m3", "c2e5m2"])
def test_8bit_full_size_sampled(key):
    """The full 64 x 64 workload (K = 8192) in the launch the benchmark times, checked on
    sampled slices that the oracle computes one by one."""
    w = synth.WORKLOADS[key]
    say(f"[gpu] generating {key} full size K={w.K}")
    x, p1, p2 = synth.make_inputs(w)
    rng = np.random.default_rng(3)
    slices = sorted({0, 1, w.K // 2, w.K - 1, *rng.integers(0, w.K, 12).tolist()})
    rep = check(x, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, label=f"{key} full", slices=slices)
    assert rep["ok"], rep["errors"]


def _bf16_bits(v):
    f = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_next(bits, up):
    """The neighbouring bf16 value away from / towards zero for positive bits."""
    return (bits.astype(np.int32) + (1 if up else -1)).astype(np.uint16)


@pytest.mark.parametrize("mode", MODES)
def test_8bit_every_code_midpoint_and_neighbour_exact(mode):
    """Identity transforms and a slice whose largest value is max_val make scale = 1 and
    y / scale = x exactly, so each element's code is the encoding of a chosen value: every
    FP8 value (every integer for INT8), every midpoint between neighbours (an exact tie,
    which goes to the even code) and the bf16 values next to each midpoint, both signs.
    The codes must equal the oracle's bit for bit on every kernel."""
    import oracle

    qmax = oracle.qmax(mode)
    if mode == "int8":
        vals = np.arange(0, 128, dtype=np.float64)
        mids = np.arange(0, 127, dtype=np.float64) + 0.5
    else:
        top = 0x7E if mode == "e4m3" else 0x7B
        vals = np.array([oracle.fp8_value(c, mode) for c in range(top + 1)])
        mids = 0.5 * (vals[:-1] + vals[1:])
    mb = _bf16_bits(mids)
    assert np.array_equal(oracle.dt_to_float(mb, "bf16"), mids)  # the ties are bf16 values
    pos = np.concatenate([_bf16_bits(vals), mb, _bf16_next(mb, True), _bf16_next(mb[1:], False)])
    pos = pos[oracle.dt_to_float(pos, "bf16") <= qmax]
    allv = np.concatenate([pos, pos | 0x8000, _bf16_bits([qmax])])
    M = N = 64
    assert allv.size <= M * N
    x = np.zeros(M * N, np.uint16)
    x[: allv.size] = allv
    x = x.reshape(1, M, N)
    eye = _bf16_bits(np.eye(M))
    r = oracle.run(x, eye, eye, "bf16", mode, 1.0, ranges=False)
    assert r["scale"][0] == 1.0
    xd, pd = to_dev(x, "bf16"), to_dev(eye, "bf16")
    ks = supported_kernels(xd, pd, pd, mode, 1.0, 0.0)
    assert fq.KERNEL_MFMA_SMALL in ks
    for k in ks:
        out, sc = run_lib(xd, pd, pd, mode, 1.0, 0.0, k)
        packed, scale = fetch(out, sc, mode, 1)
        say(f"[gpu] {mode} exhaustive codes kernel={k}: {int((packed != r['packed']).sum())} differ")
        assert scale[0] == 1.0
        assert np.array_equal(packed, r["packed"]), np.nonzero(packed != r["packed"])[1][:8]
