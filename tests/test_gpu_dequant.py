"""GPU parity of fq_dequant (codes + scales -> values in x's dtype) with the oracle's
dequantization: bit-exact (NaN for NaN), on seeded random codes and scales that include
the special cases (zero, subnormal and overflowing scales; e8m0 bytes 0, 1, 254 and 255),
on the fast path (M*N a multiple of 32) and the per-byte path, and on the quantizer's own
outputs (a quantize -> dequantize round trip, whose RMS error against y is reported)."""
import numpy as np
import pytest
import torch

import flatquant_transform_quant_amd as fq
import oracle
import synth
from gpu_util import DEV, fetch, run_lib, say, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _random_codes(K, M, N, mode, rng):
    MN = M * N
    packed = rng.integers(0, 256, (K, MN // 2), dtype=np.uint8)
    if mode == "fp4":
        e8 = rng.integers(100, 160, (K, 2 * (-(-MN // 64))), dtype=np.uint8)  # ordinary scales
        flat = e8.reshape(-1)
        special = np.array([0, 1, 2, 126, 127, 253, 254, 255], np.uint8)
        flat[rng.integers(0, flat.size, 4 * special.size)] = np.repeat(special, 4)
        return packed, e8
    sc = np.abs(rng.standard_normal(K) * np.exp(rng.uniform(-25, 25, K))).astype(np.float32)
    special = np.array([0.0, 1e-45, 1.1e-38, 1.0, 7.0 / 3.0, 3.3e38], np.float32)
    sc[rng.integers(0, K, min(K, special.size))] = special[: min(K, special.size)]
    return packed, sc


def _to_device(packed, scale, K, M, N, mode):
    out, sc = fq.empty_outputs(K, M, N, mode, DEV)
    out.view(torch.uint8).copy_(torch.from_numpy(packed).reshape(out.view(torch.uint8).shape))
    if mode == "fp4":
        sc.copy_(torch.from_numpy(scale).reshape(sc.shape))
    else:
        sc.copy_(torch.from_numpy(scale))
    return out, sc


def _gpu_dequant(out, sc, mode, M, N, dt):
    v = fq.dequantize(out, sc, mode, M, N, tdtype(dt))
    torch.cuda.synchronize()
    return v.view(torch.int16).cpu().numpy().view(np.uint16)


def _assert_same(got, want, dt, label):
    g, w = oracle.dt_to_float(got, dt), oracle.dt_to_float(want, dt)
    nan = np.isnan(w)
    bad = (np.isnan(g) != nan) | ((got != want) & ~nan)
    say(f"[gpu]   {label}: {int(bad.sum())} of {bad.size} differ")
    assert not bad.any(), (label, np.argwhere(bad)[:5].tolist())


SHAPES = [(16, 16), (64, 64), (64, 128), (256, 256),      # M*N % 32 == 0: 32 codes a thread
          (1, 2), (5, 6), (3, 10), (33, 40), (255, 254)]  # per-byte path


@pytest.mark.parametrize("mode", ["int32", "int4", "fp4"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_dequant_random_codes_match_oracle(mode, dt):
    rng = np.random.default_rng(11)
    for M, N in SHAPES:
        if mode == "int32" and N % 8:
            continue
        for K in (1, 7, 300 if M * N <= 4096 else 20):
            say(f"[gpu] dequant {mode} {dt} K={K} M={M} N={N}")
            packed, scale = _random_codes(K, M, N, mode, rng)
            out, sc = _to_device(packed, scale, K, M, N, mode)
            got = _gpu_dequant(out, sc, mode, M, N, dt)
            _assert_same(got, oracle.dequant(packed, scale, M, N, dt, mode), dt, f"{mode} {dt} {K}x{M}x{N}")


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_round_trip_matches_oracle_and_reports_rms(key):
    """Quantize on the GPU, dequantize on the GPU, compare with the oracle's dequantization
    of the same codes; report the relative RMS error of the round trip against y."""
    w = synth.WORKLOADS[key]
    K = 64 if w.M * w.N <= 8192 else 8
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    p2d = to_dev(p2, w.dtype) if p2 is not None else None
    out, sc = run_lib(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max)
    packed, scale = fetch(out, sc, w.mode, K)
    got = _gpu_dequant(out, sc, w.mode, w.M, w.N, w.dtype)
    _assert_same(got, oracle.dequant(packed, scale, w.M, w.N, w.dtype, w.mode), w.dtype, f"{key} round trip")
    y = oracle.run(x[:4], p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, ranges=False,
                   want_y=True)["y"].reshape(4, -1).astype(np.float64)
    v = oracle.dt_to_float(got[:4], w.dtype).reshape(4, -1)
    rel = np.sqrt(((v - y) ** 2).sum() / (y ** 2).sum())
    say(f"[gpu]   {key}: relative RMS error of dequantize(quantize(y)) against y = {rel:.4f}")
    assert rel < 0.5  # a sanity bound; the figure itself is reported


def test_full_size_c2_round_trip():
    w = synth.WORKLOADS["c2"]
    say(f"[gpu] dequant full size {w.name}")
    x, p1, p2 = synth.make_inputs(w)
    out, sc = run_lib(to_dev(x, w.dtype), to_dev(p1, w.dtype), to_dev(p2, w.dtype), w.mode, w.clip_ratio,
                      w.dst_type_max)
    packed, scale = fetch(out, sc, w.mode, w.K)
    got = _gpu_dequant(out, sc, w.mode, w.M, w.N, w.dtype)
    _assert_same(got, oracle.dequant(packed, scale, w.M, w.N, w.dtype, w.mode), w.dtype, "c2 full")


def _valid_8bit_codes(K, MN, mode, rng):
    """Random codes the quantizer can write: INT8 -127..127, finite FP8 codes of both signs."""
    if mode == "int8":
        return rng.integers(-127, 128, (K, MN)).astype(np.int8).view(np.uint8)
    top = 0x7E if mode == "e4m3" else 0x7B
    mag = rng.integers(0, top + 1, (K, MN)).astype(np.uint8)
    return mag | (rng.integers(0, 2, (K, MN)).astype(np.uint8) << 7)


@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_dequant_8bit_codes_match_oracle(mode, dt):
    """Every shape (the 8-codes-a-lane path when M*N is a multiple of 8, a thread a code
    otherwise), the special scales, and every code at least once: bit-exact."""
    rng = np.random.default_rng(13)
    for M, N in [(16, 16), (64, 64), (256, 256), (1, 1), (3, 5), (7, 9), (33, 40)]:
        for K in (1, 7, 300 if M * N <= 4096 else 9):
            say(f"[gpu] dequant {mode} {dt} K={K} M={M} N={N}")
            codes = _valid_8bit_codes(K, M * N, mode, rng)
            sc = np.abs(rng.standard_normal(K) * np.exp(rng.uniform(-25, 25, K))).astype(np.float32)
            special = np.array([0.0, 1e-45, 1.1e-38, 1.0, 7.0 / 3.0, 3.3e38], np.float32)
            sc[rng.integers(0, K, min(K, special.size))] = special[: min(K, special.size)]
            out, scd = fq.empty_outputs(K, M, N, mode, DEV)
            out.view(torch.uint8).copy_(torch.from_numpy(codes).reshape(K, M, N))
            scd.copy_(torch.from_numpy(sc))
            got = _gpu_dequant(out, scd, mode, M, N, dt)
            _assert_same(got, oracle.dequant(codes, sc, M, N, dt, mode), dt, f"{mode} {dt} {K}x{M}x{N}")


@pytest.mark.parametrize("key", ["c2i8", "c2e4m3", "c2e5m2", "c4i8"])
def test_8bit_round_trip_matches_oracle_and_reports_rms(key):
    w = synth.WORKLOADS[key]
    K = 64 if w.M * w.N <= 8192 else 8
    x, p1, p2 = synth.make_inputs(w, 0, K)
    out, sc = run_lib(to_dev(x, w.dtype), to_dev(p1, w.dtype), to_dev(p2, w.dtype), w.mode, w.clip_ratio,
                      w.dst_type_max)
    packed, scale = fetch(out, sc, w.mode, K)
    got = _gpu_dequant(out, sc, w.mode, w.M, w.N, w.dtype)
    _assert_same(got, oracle.dequant(packed, scale, w.M, w.N, w.dtype, w.mode), w.dtype, f"{key} round trip")
    y = oracle.run(x[:4], p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, ranges=False,
                   want_y=True)["y"].reshape(4, -1).astype(np.float64)
    v = oracle.dt_to_float(got[:4], w.dtype).reshape(4, -1)
    rel = np.sqrt(((v - y) ** 2).sum() / (y ** 2).sum())
    say(f"[gpu]   {key}: relative RMS error of dequantize(quantize(y)) against y = {rel:.4f}")
    assert rel < 0.1
