"""GPU parity of fq_mx_gemm (C = A . W^T over MXFP4 operands) with the oracle: the exact sum of
the dequantized products, within the bound any fp32 accumulation order reaches,
gamma(H) * sum|terms| (gamma(n) = n u / (1 - n u), u = 2^-24), plus half a unit in the last
place for a bf16 C.  Random operands (scales kept in the fp32 normal range) on ragged shapes,
and the quantizer's own MXFP4 output as A."""
import numpy as np
import pytest
import torch

import flatquant_transform_quant_amd as fq
import oracle
import synth
from gpu_util import DEV, fetch, run_lib, say, to_dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _rand(rows, H, rng):
    codes = rng.integers(0, 256, (rows, H // 2), dtype=np.uint8)
    e8 = rng.integers(110, 140, (rows, -(-H // 64), 2), dtype=np.uint8)
    return codes, e8


def _run(a, ae, w, we, H, out_dtype):
    C = fq.mx_gemm(torch.from_numpy(a).to(DEV), torch.from_numpy(ae).to(DEV), torch.from_numpy(w).to(DEV),
                   torch.from_numpy(we).to(DEV), H, out_dtype)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def _check(C, a, ae, w, we, H, bf16, label):
    S, Sabs = oracle.mx_gemm(a, ae.reshape(a.shape[0], -1), w, we.reshape(w.shape[0], -1), H)
    g = H * U / (1 - H * U)
    bound = g * Sabs + (2.0 ** -8 * (np.abs(S) + g * Sabs) if bf16 else 0)
    err = np.abs(C - S)
    ok = err <= bound * (1 + 1e-9)
    say(f"[gpu]   {label}: max |C - S| / bound {float((err / np.maximum(bound, 1e-300)).max()):.3f}, "
        f"outside {int((~ok).sum())} of {ok.size}")
    assert ok.all()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mx_gemm_random_operands(out_dtype):
    rng = np.random.default_rng(21)
    for T, O, H in [(1, 1, 128), (16, 16, 128), (128, 128, 256), (130, 200, 384), (257, 129, 1024),
                    (64, 300, 4096), (3, 2, 8192), (200, 64, 128),
                    (2048, 1030, 384), (768, 2048, 512)]:  # several 256 x 256 tiles, ragged / 8-XCD tile counts
        say(f"[gpu] mx_gemm T={T} O={O} H={H} {out_dtype}")
        a, ae = _rand(T, H, rng)
        w, we = _rand(O, H, rng)
        C = _run(a, ae, w, we, H, out_dtype)
        _check(C, a, ae, w, we, H, out_dtype == torch.bfloat16, f"{T}x{O}x{H}")


def test_mx_gemm_consumes_the_quantizer_output():
    """A = the fp4 output of the quantizer (c3 workload, K slices as T tokens, H = M*N)."""
    w_ = synth.WORKLOADS["c3"]
    K, H = 96, w_.M * w_.N
    x, p1, p2 = synth.make_inputs(w_, 0, K)
    out, sc = run_lib(to_dev(x, w_.dtype), to_dev(p1, w_.dtype), to_dev(p2, w_.dtype), "fp4", 1.0, 0.0)
    a, ae = fetch(out, sc, "fp4", K)
    rng = np.random.default_rng(22)
    wc, we = _rand(160, H, rng)
    say(f"[gpu] mx_gemm on the c3 quantizer output: T={K} O=160 H={H}")
    C = fq.mx_gemm(out, sc, torch.from_numpy(wc).to(DEV), torch.from_numpy(we).to(DEV), H, torch.float32)
    torch.cuda.synchronize()
    _check(C.cpu().numpy().astype(np.float64), a, ae.reshape(K, -1, 2), wc, we, H, False, "c3 A")
