"""Helpers for the GPU tests: move generator output to the device, call libfq through
its C ABI binding, bring the codes back, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import flatquant_transform_quant_amd as fq
import oracle
from oracle.compare import compare

DEV = torch.device("cuda:0")


def tdtype(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float16


def to_dev(a: np.ndarray, dt: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdtype(dt)).to(DEV)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def fetch(out: torch.Tensor, sc: torch.Tensor, mode: str, K: int):
    packed = out.contiguous().view(torch.uint8).reshape(K, -1).cpu().numpy()
    if mode == "fp4":
        scale = sc.contiguous().view(torch.uint8).reshape(K, -1).cpu().numpy()
    else:
        scale = sc.contiguous().cpu().numpy()
    return packed, scale


def run_lib(x_dev, p1_dev, p2_dev, mode, clip, dmax, kernel=fq.KERNEL_AUTO):
    K, M, N = x_dev.shape
    out, sc = fq.empty_outputs(K, M, N, mode, DEV)
    fq.quantize(x_dev, p1_dev, p2_dev, out, sc, mode, clip, dmax, kernel=kernel)
    torch.cuda.synchronize()
    return out, sc


def supported_kernels(x_dev, p1_dev, p2_dev, mode, clip, dmax):
    """The kernel variants that accept this problem."""
    K, M, N = x_dev.shape
    out, sc = fq.empty_outputs(K, M, N, mode, DEV)
    ks = []
    for k in (fq.KERNEL_GENERIC, fq.KERNEL_MFMA_SMALL, fq.KERNEL_MFMA_WIDE, fq.KERNEL_MFMA_WIDE_T, fq.KERNEL_MFMA_WIDE_L):
        try:
            ex = fq.Executor(x_dev, p1_dev, p2_dev, out, sc, mode, clip, dmax, kernel=k)
        except fq.FqError:
            continue
        ex.destroy()
        ks.append(k)
    return ks


def check(x, p1, p2, dt, mode, clip, dmax, kernel=fq.KERNEL_AUTO, label="", slices=None):
    """Run libfq on x [K, M, N] (host uint16) and compare the slices `slices` (default:
    all) with the oracle.  Returns the comparison report."""
    K = x.shape[0]
    say(f"[gpu] {label} K={K} M={x.shape[1]} N={x.shape[2]} {dt} {mode} clip={clip} dmax={dmax} "
        f"kernel={kernel} two_sided={p2 is not None}")
    xd, p1d = to_dev(x, dt), to_dev(p1, dt)
    p2d = to_dev(p2, dt) if p2 is not None else None
    out, sc = run_lib(xd, p1d, p2d, mode, clip, dmax, kernel)
    packed, scale = fetch(out, sc, mode, K)
    idx = np.arange(K) if slices is None else np.asarray(slices)
    orc = oracle.run(x[idx], p1, p2, dt, mode, clip, dmax, nthreads=8)
    rep = compare(orc, packed[idx], scale[idx])
    say(f"[gpu]   -> mismatches {rep['mismatch']} (cap {rep['mismatch_cap']}; outside the stated window "
        f"{rep['mismatch_out_of_window']}, cap {rep['out_of_window_cap']}), flagged {rep['flagged']}, "
        f"alt groups {rep['alt_groups']}, max scale rel {rep['max_scale_rel']:.2e}, scale ties "
        f"{rep.get('scale_ties', 0)} (cap {rep.get('scale_ties_cap', 0)}), ok={rep['ok']}")
    return rep
