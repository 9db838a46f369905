"""GPU parity of the int4 consumer GEMM with the oracle.  The integer dot product is exact
and the scaling is a fixed sequence of fp32 operations, so an fp32 C must equal the oracle's
bit for bit, and a bf16 C must be its round-to-nearest-even (torch's cast)."""
import numpy as np
import pytest
import torch

import flatquant_transform_quant_amd as fq
import oracle
import synth
from gpu_util import DEV, fetch, run_lib, say, to_dev

pytestmark = pytest.mark.gpu


def _rand(rows, H, rng):
    codes = rng.integers(0, 256, (rows, H // 2), dtype=np.uint8)
    sc = np.abs(rng.standard_normal(rows) * np.exp(rng.uniform(-8, 8, rows))).astype(np.float32)
    return codes, sc


def _check(C, want32, bf16, label):
    got = C.cpu()
    if bf16:
        want = torch.from_numpy(want32).to(torch.bfloat16)
        bad = (got.view(torch.int16) != want.view(torch.int16)).numpy()
    else:
        bad = got.numpy().view(np.uint32) != want32.view(np.uint32)
    say(f"[gpu]   {label}: {int(bad.sum())} of {bad.size} differ")
    assert not bad.any(), np.argwhere(bad)[:5].tolist()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_int4_gemm_random_operands(out_dtype):
    rng = np.random.default_rng(41)
    for T, O, H in [(1, 1, 128), (16, 16, 128), (128, 128, 256), (130, 200, 384), (257, 129, 1024),
                    (64, 300, 4096), (3, 2, 8192), (2048, 1030, 384), (768, 2048, 512)]:
        say(f"[gpu] int4_gemm T={T} O={O} H={H} {out_dtype}")
        a, sa = _rand(T, H, rng)
        w, sw = _rand(O, H, rng)
        C = fq.int4_gemm(torch.from_numpy(a).to(DEV), torch.from_numpy(sa).to(DEV), torch.from_numpy(w).to(DEV),
                         torch.from_numpy(sw).to(DEV), H, out_dtype)
        torch.cuda.synchronize()
        _check(C, oracle.int4_gemm(a, sa, w, sw, H), out_dtype == torch.bfloat16, f"{T}x{O}x{H}")


def test_int4_gemm_extreme_codes():
    """Every code -8: each product is 64 and the sum 64 H, the largest magnitude."""
    H = 8192
    a = np.full((256, H // 2), 0x88, np.uint8)
    s = np.ones(256, np.float32)
    C = fq.int4_gemm(torch.from_numpy(a).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(a).to(DEV),
                     torch.from_numpy(s).to(DEV), H, torch.float32)
    torch.cuda.synchronize()
    assert (C.cpu().numpy() == 64.0 * H).all()


def test_int4_gemm_consumes_the_quantizer_output():
    """A = the per-token int4 output of the quantizer (64 x 64 workload, K slices as T tokens,
    H = M*N) with its scales."""
    w_ = synth.WORKLOADS["c2"]
    K, H = 96, w_.M * w_.N
    x, p1, p2 = synth.make_inputs(w_, 0, K)
    out, sc = run_lib(to_dev(x, w_.dtype), to_dev(p1, w_.dtype), to_dev(p2, w_.dtype), w_.mode, w_.clip_ratio,
                      w_.dst_type_max)
    a, sa = fetch(out, sc, w_.mode, K)
    rng = np.random.default_rng(42)
    wc, ws = _rand(160, H, rng)
    C = fq.int4_gemm(out.view(torch.uint8).reshape(K, H // 2), sc, torch.from_numpy(wc).to(DEV),
                     torch.from_numpy(ws).to(DEV), H, torch.float32)
    torch.cuda.synchronize()
    _check(C, oracle.int4_gemm(a, sa, wc, ws, H), False, "c2 A")
