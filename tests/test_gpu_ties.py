"""Bit-exact GPU checks of the int4 and E2M1 encoders and the e8m0 rules at their edge cases.

The comparator's tolerance lets a code move by one step where the oracle sees a rounding
tie, so random data cannot show a wrong tie rule.  Here the transforms are exact
(permutation matrices with signs, or the identity), so y is x permuted and sign-flipped,
and x is built so that y / scale (per token) or y * 2^(127 - e8m0) (per group) is exactly
a chosen value: every int4 tie n + 1/2 and the dtype values on either side of it, the
clamps at -8 and 7 (clipRatio below 7/7.5, down to 2^-23 where y * (1/scale) reaches
-5.9e7), -0, tiny scales whose reciprocal overflows fp32; every E2M1 decision point 0.25,
0.75, ..., 5 and its neighbours, values above 6, -0; group maxima exactly at powers of two
with dstTypeMax 8, at 6 * 2^k with dstTypeMax 6, at 7 * 2^k with dstTypeMax 7 and at
12 * 2^k with dstTypeMax 12 (the V2 rule's "no increment when the mantissa is zero"
branch) and one dtype step on either side of them; e8m0 codes 0 and the largest reachable
(252 in V1: a group maximum of 1.5 * 2^127 from P1 = 1.5 I).  Every kernel variant that
accepts the shape runs, in both dtypes, and the codes, e8m0 bytes and fp32 scales must equal
the oracle's bit for bit.  The hand-worked fixtures under tests/golden run the same way.
"""
import math

import numpy as np
import pytest

import flatquant_transform_quant_amd as fq
import oracle
import synth
from gpu_util import fetch, run_lib, say, supported_kernels, to_dev
from golden_io import keyed

pytestmark = pytest.mark.gpu

FRAC = {"bf16": 7, "f16": 10}
EMIN = {"bf16": -126, "f16": -14}
MAXV = {"bf16": 3.3895313892515355e38, "f16": 65504.0}


def rt(v, dt):
    return synth.round_to(np.asarray(v, dtype=np.float64), dt)


def val(bits, dt):
    return oracle.dt_to_float(bits, dt)


def representable(v, dt):
    v = np.asarray(v, dtype=np.float64)
    return np.isfinite(val(rt(v, dt), dt)) & (val(rt(v, dt), dt) == v)


def neighbours(v, dt):
    """The dtype values next to v (v > 0, representable or not) below and above."""
    e = max(math.floor(math.log2(v)), EMIN[dt])
    ulp = 2.0 ** (e - FRAC[dt])
    lo = math.floor(v / ulp) * ulp
    below = lo if lo < v else lo - ulp
    above = lo + ulp
    return below, above


def exact_transforms(M, N, dt, seed, two_sided=True):
    """A permutation with signs for P1 and P2 (exact in any precision)."""
    rng = np.random.default_rng(seed)
    p1 = np.eye(M)[rng.permutation(M)] * rng.choice([-1.0, 1.0], M)
    p2 = np.eye(N)[rng.permutation(N)] * rng.choice([-1.0, 1.0], N) if two_sided else None
    return rt(p1, dt), (rt(p2, dt) if p2 is not None else None)


def place(values, M, N, K, dt, seed):
    """Spread the value list over K slices of [M, N] (zeros elsewhere), as dtype bits."""
    flat = np.zeros(K * M * N)
    rng = np.random.default_rng(seed)
    v = np.asarray(values, dtype=np.float64)
    assert v.size <= flat.size
    flat[: v.size] = v
    bits = rt(flat, dt)
    neg0 = np.nonzero([(x == 0 and math.copysign(1.0, x) < 0) for x in flat])[0]
    bits[neg0] = 0x8000
    bits = bits.reshape(K, M * N)
    for k in range(K):
        bits[k] = bits[k][rng.permutation(M * N)]
    return bits.reshape(K, M, N)


def run_every_kernel(x, p1, p2, dt, mode, clip, dmax, label, expect_scale=None, must_have=()):
    """Every accepting kernel; codes, e8m0 and scales equal to the oracle's bit for bit."""
    K = x.shape[0]
    r = oracle.run(x, p1, p2, dt, mode, clip, dmax, ranges=False)
    o_scale = r["scale"] if mode != "fp4" else r["e8m0"]
    if expect_scale is not None:
        assert np.array_equal(o_scale, expect_scale), (o_scale, expect_scale)
    xd, p1d = to_dev(x, dt), to_dev(p1, dt)
    p2d = to_dev(p2, dt) if p2 is not None else None
    ks = supported_kernels(xd, p1d, p2d, mode, clip, dmax)
    for k in must_have:
        assert k in ks, (label, ks)
    for k in ks:
        out, sc = run_lib(xd, p1d, p2d, mode, clip, dmax, k)
        packed, scale = fetch(out, sc, mode, K)
        nd = int((packed != r["packed"]).sum())
        ns = int((np.asarray(scale).view(np.uint8) != np.asarray(o_scale).view(np.uint8)).sum())
        say(f"[gpu] {label} {dt} {mode} clip={clip} dmax={dmax} kernel={k}: {nd} code bytes, {ns} scale bytes differ")
        assert nd == 0 and ns == 0, (label, k, np.nonzero(packed != r["packed"])[1][:8])
    return ks


# ---------------------------------------------------------------- per token, int4

def int4_values(d, e, dt):
    """y values (scale 2^-e, max|q| = d) that hit every int4 tie, its dtype neighbours, the
    integers, the clamps and the signed zeros; plus +-d itself (the slice maximum)."""
    s = 2.0 ** -e
    qs = [d, -d, 0.0, -0.0]
    lim = min(d, 9.0)
    for n in np.arange(-9.0, 9.0):
        t = n + 0.5
        if abs(t) <= lim:
            qs.append(t)
        if abs(n) <= lim:
            qs.append(n)
    ys = [q * s for q in qs]
    for q in list(qs):
        if q != 0 and abs(q) != d and abs(q - round(q)) == 0.5:  # the neighbours of each tie
            b, a = neighbours(abs(q) * s, dt)
            ys += [math.copysign(b, q), math.copysign(a, q)]
    if d > 100:  # far beyond the clamps: -8 / 7 on every kernel
        for q in (10.0, 100.0, 1e4, 1e6, d / 2, d * 0.999):
            ys += [q * s, -q * s]
    ys += [2.0 ** (EMIN[dt] - FRAC[dt]), -(2.0 ** (EMIN[dt] - FRAC[dt]))]  # the smallest subnormals
    ys = np.asarray(ys, dtype=np.float64)
    ok = representable(ys, dt) & (np.abs(ys) <= d * s)
    return ys[ok]


# clipRatio -> d = fl32(7 / clipRatio), exact for these
CLIPS = {1.0: 7.0, 0.875: 8.0, 0.5: 14.0, 2.0 ** -23: 7.0 * 2.0 ** 23}
SHAPES_TOKEN = [(64, 64), (32, 128), (16, 16), (17, 24), (256, 256),
                (128, 128), (86, 128)]  # (two passes over GEMM2 on the small kernel, exact and padded)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("clip", list(CLIPS))
def test_int4_every_tie_clamp_and_zero_exact(dt, clip):
    d = CLIPS[clip]
    e = 0
    while d * 2.0 ** -e > MAXV[dt]:  # keep the slice maximum d * scale representable
        e += 1
    if dt == "f16" and d > 100:
        e = max(e, 10)
    ys = int4_values(d, e, dt)
    for M, N in SHAPES_TOKEN:
        K = 3
        x = place(ys, M, N, K, dt, seed=M + N)
        # every slice has its maximum d * 2^-e, so the scale is 2^-e exactly
        for k in range(K):
            x[k].reshape(-1)[0] = rt([d * 2.0 ** -e], dt)[0]
        p1, p2 = exact_transforms(M, N, dt, seed=M * 3 + N)
        mode = "int4" if N % 8 else "int32"
        ks = run_every_kernel(x, p1, p2, dt, mode, clip, 0.0, f"int4 ties {M}x{N}",
                              expect_scale=np.full(K, 2.0 ** -e, np.float32))
        if (M, N) in ((64, 64), (32, 128)):
            assert fq.KERNEL_MFMA_SMALL in ks
        if (M, N) == (256, 256):
            assert fq.KERNEL_MFMA_WIDE in ks


@pytest.mark.parametrize("case", ["subnormal y, clip 1", "normal y, clip 2^-30"])
def test_int4_tiny_scale_whose_reciprocal_overflows(case):
    """Slices whose scale is below 2^-128 (1 / scale is +inf in fp32), next to ordinary
    slices: the codes must still be those of y / scale.  With clipRatio 1 the slice maximum
    is 1.75 * 2^-128 (scale 2^-130) and the other values are ties and integers of it (fp32
    subnormals); with clipRatio 2^-30 (d = 7 * 2^30) the maximum is a normal 1.75 * 2^-100
    (scale 2^-132), every other value is normal or zero, and the zeros must stay 0 (0 * inf
    is NaN)."""
    dt = "bf16"
    sub = case.startswith("subnormal")
    clip = 1.0 if sub else 2.0 ** -30
    tiny_max = 1.75 * 2.0 ** -128 if sub else 1.75 * 2.0 ** -100
    for M, N in SHAPES_TOKEN:
        K = 4
        rng = np.random.default_rng(M + N)
        x = np.zeros((K, M, N))
        for k in range(K):
            if k % 2 == 1:   # an ordinary slice: maximum 7, scale 1 (clip 1) or 2^-30
                qs = rng.integers(-14, 15, size=M * N) / 2.0
                x[k] = (qs * (1.0 if sub else 2.0 ** 30)).reshape(M, N)
                x[k].reshape(-1)[0] = 7.0 * (1.0 if sub else 2.0 ** 30)
            elif sub:
                qs = rng.integers(-14, 15, size=M * N) / 2.0      # ties and integers in [-7, 7]
                x[k] = (qs * tiny_max / 7.0).reshape(M, N)
                x[k].reshape(-1)[0] = tiny_max
            else:
                mag = 2.0 ** rng.integers(-126, -100, size=M * N) * rng.choice([-1.0, 0.0, 1.0], M * N)
                x[k] = mag.reshape(M, N)
                x[k].reshape(-1)[0] = tiny_max
        xb = rt(x, dt)
        assert np.array_equal(val(xb, dt), x)
        p1, p2 = exact_transforms(M, N, dt, seed=M * 5 + N)
        mode = "int4" if N % 8 else "int32"
        want = [2.0 ** -130, 1.0] if sub else [2.0 ** -132, 1.0]
        run_every_kernel(xb, p1, p2, dt, mode, clip, 0.0, f"int4 tiny scale ({case}) {M}x{N}",
                         expect_scale=np.array(want * 2, np.float32))


# ---------------------------------------------------------------- per group, E2M1 + e8m0

E2M1_MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def group_values(v_max, dt, scale_exp):
    """31 values of one group (in units of 2^scale_exp) that hit the E2M1 decision points,
    their dtype neighbours, zeros and saturation, plus the group maximum v_max."""
    s = 2.0 ** scale_exp
    vals = []
    for m in E2M1_MIDS:
        vals += [m, -m]
        b, a = neighbours(m * s, dt)
        vals += [b / s, -a / s]
    vals += [-0.0, 0.0, 6.0, -6.0, 7.0, -7.5, 6.5, 0.125, -0.375]
    vals = [v for v in vals if abs(v) <= v_max]
    vals = np.asarray(vals[:31] + [v_max], dtype=np.float64) * s
    return vals


def build_groups(M, N, K, dt, groups):
    """groups: list of (v_max, scale_exp) -- one 32-group each, cycled over the K slices'
    groups.  Returns x bits [K, M, N]; a group is 32 consecutive elements of the flattened
    slice, so with the identity transforms each group's y is its x."""
    G = M * N // 32
    x = np.zeros((K, G, 32))
    i = 0
    for k in range(K):
        for g in range(G):
            vmax, se = groups[i % len(groups)]
            i += 1
            gv = group_values(vmax, dt, se)
            ok = representable(gv, dt) & np.isfinite(gv)
            gv = np.where(ok, gv, 0.0)
            x[k, g, : gv.size] = gv
    bits = rt(x.reshape(K, -1), dt)
    negz = (x.reshape(K, -1) == 0) & np.signbit(x.reshape(K, -1))
    bits[negz] = 0x8000
    return bits.reshape(K, M, N)


SHAPES_GROUP = [(64, 64, True), (64, 128, True), (16, 16, True), (256, 256, True), (256, 256, False),
                (32, 32, False)]


def _group_plan(dt, dmax):
    """Group maxima that pin the e8m0 rule: for V1 values in [4, 8) * 2^j (and 6 * 2^j);
    for V2 the exact dmax * 2^j (mantissa of S zero: no increment) and the dtype values
    just below and above it (increment), over a spread of exponents."""
    js = [-20, -5, -1, 0, 1, 3, 10] if dt == "f16" else [-120, -60, -5, 0, 3, 40, 120]
    js = [j for j in js if not (dt == "f16" and (j < -8 or j > 10))]
    plan = []
    for j in js:
        if dmax == 0.0:
            plan += [(4.0, j), (6.0, j), (7.5, j), (5.0, j)]
        else:
            b, a = neighbours(dmax, dt)
            plan += [(dmax, j), (b, j), (a, j)]
    return plan


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("dmax", [0.0, 6.0, 7.0, 8.0, 12.0])
def test_e2m1_every_decision_point_and_e8m0_rule_exact(dt, dmax):
    plan = _group_plan(dt, dmax)
    for M, N, two in SHAPES_GROUP:
        K = 2
        x = build_groups(M, N, K, dt, plan)
        eye1 = rt(np.eye(M), dt)
        eye2 = rt(np.eye(N), dt) if two else None
        ks = run_every_kernel(x, eye1, eye2, dt, "fp4", 1.0, dmax, f"e2m1 ties {M}x{N} two_sided={two}")
        if (M, N) in ((64, 64), (64, 128)):
            assert fq.KERNEL_MFMA_SMALL in ks
        if (M, N) == (256, 256):
            assert fq.KERNEL_MFMA_WIDE in ks
            assert (fq.KERNEL_MFMA_WIDE_L in ks) == (not two)
        # the plan reached both branches of the V2 rule
        r = oracle.run(x, eye1, eye2, dt, "fp4", 1.0, dmax, ranges=False)
        if dmax > 0:
            G = M * N // 32
            amax = np.abs(val(x, dt).reshape(K, G, 32)).max(axis=2)
            exact = amax / dmax == 2.0 ** np.floor(np.log2(amax / dmax))
            assert exact.any() and (~exact).any()
        assert r["e8m0"].max() > 0


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_e2m1_permuted_transforms_exact(dt):
    """The same decision-point groups through permutation-with-sign transforms: y is a
    shuffled, sign-flipped x, so groups mix -- every code and e8m0 byte still exact."""
    plan = _group_plan(dt, 0.0)
    for M, N, two in SHAPES_GROUP:
        x = build_groups(M, N, 2, dt, plan)
        p1, p2 = exact_transforms(M, N, dt, seed=M + 7 * N, two_sided=two)
        run_every_kernel(x, p1, p2, dt, "fp4", 1.0, 0.0, f"e2m1 permuted {M}x{N} two_sided={two}")


@pytest.mark.parametrize("dmax", [0.0, 6.0])
def test_e8m0_extreme_codes(dmax):
    """The smallest and largest e8m0 codes.  Code 0: group maxima 4, 6 and 7.5 times 2^-127
    (V1 gives floor(log2) - 2 + 127 = 0; the scale is the subnormal 2^-127) and 3 * 2^-127
    (below that: clamped to 0), with the other elements 2 .. 6 times 2^-127 (fp32 normal).
    The largest: P1 = 1.5 I and a bf16 group maximum of 2^127, so y's maximum is 1.5 * 2^127
    -- V1 gives 252, V2 with dstTypeMax 6 gives S = 2^125 exactly, no increment, 252 -- and
    the bf16 value one step above 2^127 (V2: S's mantissa is non-zero, 253).  A code of 254
    needs a group maximum of at least 2^129 (V1) or 6 * 2^127 (V2), beyond fp32's range."""
    dt = "bf16"
    M = N = 64
    G = M * N // 32
    mids = np.array([2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, -2.5, -3.5, -5.0, -6.0, -2.0, 0.0])
    for what in ("smallest", "largest"):
        x = np.zeros((2, G, 32))
        for k in range(2):
            for g in range(G):
                if what == "smallest":
                    vm = [4.0, 6.0, 7.5, 3.0][g % 4]
                    gv = np.concatenate([[vm], mids[np.abs(mids) <= vm]]) * 2.0 ** -127
                else:
                    top = 2.0 ** 127 * (1.0 if g % 2 == 0 else 1.0 + 2.0 ** -7)
                    gv = np.concatenate([[top], mids * 2.0 ** 124])
                x[k, g, : gv.size] = gv
        xb = rt(x.reshape(2, M, N), dt)
        assert np.array_equal(val(xb, dt), x.reshape(2, M, N))
        p1 = rt((1.0 if what == "smallest" else 1.5) * np.eye(M), dt)
        p2 = rt(np.eye(N), dt)
        r = oracle.run(xb, p1, p2, dt, "fp4", 1.0, dmax, ranges=False)
        e8 = r["e8m0"][:, :G]
        if what == "smallest":
            assert e8.max() == 0 if dmax == 0.0 else True
        else:
            assert (e8[:, 0::2] == 252).all()
            assert (e8[:, 1::2] == (252 if dmax == 0.0 else 253)).all()
        run_every_kernel(xb, p1, p2, dt, "fp4", 1.0, dmax, f"e8m0 {what}")


# ---------------------------------------------------------------- the hand-worked fixtures

def test_worked_pertoken_fixture_every_kernel():
    """tests/golden/worked_pertoken.txt (clipRatio 0.875, scale 0.5, ties to even and the
    clamp worked by hand), tiled over 64 x 64 and 256 x 256 slices with identity transforms:
    each copy of the 12 values must give the fixture's codes on every kernel."""
    k = keyed("worked_pertoken.txt")
    clip = float(k["clip"][0])
    xs = np.array([float(v) for v in k["x"]])
    codes = np.array([int(v) for v in k["codes"]])
    for M, N in ((64, 64), (256, 256), (2, 6)):
        n = M * N // 12 * 12
        x = np.zeros((1, M * N))
        x[0, :n] = np.tile(xs, n // 12)
        xb = rt(x.reshape(1, M, N), "bf16")
        eye1, eye2 = rt(np.eye(M), "bf16"), rt(np.eye(N), "bf16")
        mode = "int32" if N % 8 == 0 else "int4"
        xd, p1d, p2d = to_dev(xb, "bf16"), to_dev(eye1, "bf16"), to_dev(eye2, "bf16")
        for kern in supported_kernels(xd, p1d, p2d, mode, clip, 0.0):
            out, sc = run_lib(xd, p1d, p2d, mode, clip, 0.0, kern)
            packed, scale = fetch(out, sc, mode, 1)
            nib = np.stack([packed[0] & 0xF, packed[0] >> 4], axis=1).reshape(-1)[:n].astype(np.int16)
            nib = np.where(nib >= 8, nib - 16, nib)
            say(f"[gpu] worked per-token fixture {M}x{N} kernel={kern}")
            assert scale[0] == float(k["scale"][0])
            assert np.array_equal(nib, np.tile(codes, n // 12))


def test_worked_pergroup_fixture_every_kernel():
    """tests/golden/worked_pergroup.txt: group A (V1) and group B at every listed dstTypeMax,
    repeated over every 32-group of 64 x 64 and 256 x 256 slices (identity transforms, left-only
    too): the fixture's codes and e8m0 bytes on every kernel."""
    k = keyed("worked_pergroup.txt")
    xa = np.array([float(v) for v in k["xA"]])
    hexes = lambda key: np.array([int(v, 16) for v in k[key]], dtype=np.uint8)
    cases = [(xa, 0.0, hexes("codesA"), int(k["e8m0A_v1"][0]))]
    for key, dmax in (("e8m0B_v1", 0.0), ("e8m0B_v2_6", 6.0), ("e8m0B_v2_8", 8.0), ("e8m0B_v2_10", 10.0)):
        cases.append((2 * xa, dmax, hexes("codesB_v2_10") if dmax == 10.0 else hexes("codesA"), int(k[key][0])))
    for xv, dmax, want_codes, want_e8 in cases:
        for M, N, two in ((64, 64, True), (256, 256, True), (256, 256, False), (1, 32, True)):
            G = M * N // 32
            x = np.tile(xv, G).reshape(1, M, N)
            xb = rt(x, "bf16")
            xb.reshape(-1)[np.nonzero((x.reshape(-1) == 0) & np.signbit(x.reshape(-1)))[0]] = 0x8000
            eye1 = rt(np.eye(M), "bf16")
            eye2 = rt(np.eye(N), "bf16") if two else None
            xd, p1d = to_dev(xb, "bf16"), to_dev(eye1, "bf16")
            p2d = to_dev(eye2, "bf16") if two else None
            for kern in supported_kernels(xd, p1d, p2d, "fp4", 1.0, dmax):
                out, sc = run_lib(xd, p1d, p2d, "fp4", 1.0, dmax, kern)
                packed, e8 = fetch(out, sc, "fp4", 1)
                nib = np.stack([packed[0] & 0xF, packed[0] >> 4], axis=1).reshape(-1)
                say(f"[gpu] worked per-group fixture dmax={dmax} {M}x{N} two_sided={two} kernel={kern}")
                assert (e8[0, :G] == want_e8).all()
                assert np.array_equal(nib, np.tile(want_codes, G))
