"""Accuracy of the quantize -> dequantize round trip (CPU, oracle only).

The relative RMS error of dequantize(quantize(y)) against y (the check the APT-LLM page,
section 5.2, describes), for each workload with its random orthogonal transforms and with
identity transforms (then y = x).  The transforms exist to flatten outlier channels before
the quantizer sees them: with per-token int4 scales over a whole slice an outlier channel
sets the step for everything else, so the orthogonal transforms must lower the error on the
outlier workloads; per-group scales already confine an outlier to its 32-group, so the gain
there is smaller.  With 8-bit codes per token the same holds for INT8 (a uniform grid), while
FP8 carries an exponent per element, so an outlier no longer sets every element's step and
the transforms leave the error about where it was.  Run with -s to see the figures.
"""
import numpy as np
import pytest

import oracle
import synth


def _round_trip_rel_rms(w, x, p1, p2):
    r = oracle.run(x, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, ranges=False, want_y=True,
                   nthreads=8)
    sc = r["scale"] if w.mode != "fp4" else r["e8m0"]
    v = oracle.dt_to_float(oracle.dequant(r["packed"], sc, w.M, w.N, w.dtype, w.mode), w.dtype)
    v = v.reshape(len(x), -1)
    y = r["y"].reshape(len(x), -1).astype(np.float64)
    return float(np.sqrt(((v - y) ** 2).sum() / (y ** 2).sum()))


def _identity(n, dtype):
    p = np.zeros((n, n), np.uint16)
    np.fill_diagonal(p, 0x3F80 if dtype == "bf16" else 0x3C00)
    return p


# workload: (slices sampled, range of the ratio identity / orthogonal)
CASES = {"c2": (32, 2.0, 10.0), "c3": (32, 1.1, 10.0), "c4": (4, 2.0, 10.0), "c5": (4, 1.05, 10.0),
         "c2i8": (32, 3.0, 20.0), "c2e4m3": (32, 0.8, 1.25), "c2e5m2": (32, 0.8, 1.25)}


@pytest.mark.parametrize("key", sorted(CASES))
def test_orthogonal_transforms_lower_the_round_trip_error(key):
    w = synth.WORKLOADS[key]
    K, least, most = CASES[key]
    x, p1, p2 = synth.make_inputs(w, 0, K)
    orth = _round_trip_rel_rms(w, x, p1, p2)
    ident = _round_trip_rel_rms(w, x, _identity(w.M, w.dtype), _identity(w.N, w.dtype) if p2 is not None else None)
    print(f"\n{w.name}: relative RMS of dequantize(quantize(y)) - y: orthogonal {orth:.4f}, identity "
          f"{ident:.4f} (x{ident / orth:.2f})")
    assert orth < 0.25
    assert least <= ident / orth <= most
