"""Pins of the oracle's 16-bit decoding, of its fp16 transform path and of the reachable code
ranges it reports (CPU only).

The reachable ranges are what the comparator relies on where a GPU result may differ from
the oracle's: they must contain every code some fp32 summation order can give (checked by
brute force over every order on tiny inputs), they must flag an intermediate sum that sits
exactly on a rounding midpoint of the activation dtype (constructed inputs, the two codes
it can reach computed here from the two neighbouring dtype values), and they must collapse
to one code where every sum is far from every boundary.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore")

FRAC = {"bf16": 7, "f16": 10}  # fraction bits of the activation dtypes


def rt(vals, dt):
    return synth.round_to(np.asarray(vals, dtype=np.float64), dt)


def val(bits, dt):
    return oracle.dt_to_float(bits, dt)


def to_dt(v, dt):
    """RNE of float64 values to the dtype through fp32 with numpy / torch casts."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if dt == "f16":
        return f.astype(np.float16).astype(np.float64)
    return torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------- 16-bit decoding

def test_f16_decoding_every_bit_pattern():
    """The oracle's fp16 decoder (normal, subnormal, zero, infinity, NaN, both signs) against
    numpy's float16 -> float64 conversion on all 65536 bit patterns."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode16(b, "f16")
    want = b.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))  # -0 keeps its sign
    # the subnormal step and the largest finite value
    assert got[1] == 2.0 ** -24 and got[0x7BFF] == 65504.0 and got[0x0400] == 2.0 ** -14


def test_bf16_decoding_every_bit_pattern():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode16(b, "bf16")
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))


def test_every_finite_f16_value_passes_the_identity_transform_exactly():
    """Through the whole path: with P1 = P2 = I the oracle's y is x itself, for every finite
    fp16 bit pattern (a decoding mistake anywhere in the path shows here)."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = b[~np.isnan(b.view(np.float16)) & ~np.isinf(b.view(np.float16))]
    n = 64
    S = -(-fin.size // (n * n))
    x = np.zeros(S * n * n, np.uint16)
    x[: fin.size] = fin
    x = x.reshape(S, n, n)
    eye = rt(np.eye(n), "f16")
    r = oracle.run(x, eye, eye, "f16", "fp4", want_y=True, want_t=True, ranges=False)
    want = x.view(np.float16).astype(np.float64)
    assert np.array_equal(r["y"].astype(np.float64), want)
    # T = RNE(x . I) is x again, up to the sign of zero (a sum that starts at +0)
    tb = r["t"].reshape(-1)
    xb = x.reshape(-1)
    nz = (xb & 0x7FFF) != 0
    assert np.array_equal(tb[nz], xb[nz]) and ((tb[~nz] & 0x7FFF) == 0).all()


# ---------------------------------------------------------------- fp16 transform path

def _gen_small_exact(rng, M, N):
    x = rng.integers(-4, 5, size=(1, M, N)).astype(np.float64)
    p1 = rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=(M, M))
    p2 = rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=(N, N))
    return x, p1, p2


@pytest.mark.parametrize("M,N", [(1, 2), (2, 2), (3, 4), (4, 8), (8, 8), (5, 6)])
def test_kronecker_closed_form_f16(M, N):
    """vec_row(P1 x P2) = (P1 kron P2^T) vec_row(x) in fp16, on inputs whose intermediate is
    exact in fp16 (so every reading of the intermediate precision agrees)."""
    rng = np.random.default_rng(M * 100 + N + 1)
    for _ in range(5):
        x, p1, p2 = _gen_small_exact(rng, M, N)
        r = oracle.run(rt(x, "f16"), rt(p1, "f16"), rt(p2, "f16"), "f16", "fp4", want_y=True, ranges=False)
        want = (np.kron(p1, p2.T) @ x.reshape(-1)).reshape(M, N)
        assert np.array_equal(r["y"][0].astype(np.float64), want)
        r2 = oracle.run(rt(x, "f16"), rt(p1, "f16"), None, "f16", "fp4", want_y=True, ranges=False)
        assert np.array_equal(r2["y"][0].astype(np.float64), p1 @ x[0])


def test_transform_order_p2_first_then_p1_f16():
    """A non-exact intermediate makes the order observable in fp16 too: T = RNE_f16(fl32(x P2))
    first (numpy's float32 and float16 casts), then y = fl32(P1 T)."""
    rng = np.random.default_rng(21)
    for M, N in ((4, 4), (3, 6), (8, 16)):
        xb = rt(rng.standard_normal((1, M, N)), "f16")
        p1b, p2b = rt(rng.standard_normal((M, M)), "f16"), rt(rng.standard_normal((N, N)), "f16")
        r = oracle.run(xb, p1b, p2b, "f16", "int32" if N % 8 == 0 else "fp4", want_y=True, want_t=True,
                       ranges=False)
        X, P1, P2 = (b.view(np.float16).astype(np.float64) for b in (xb[0], p1b, p2b))
        T = (X @ P2).astype(np.float32).astype(np.float16)
        assert np.array_equal(r["t"][0], T.view(np.uint16))
        assert np.array_equal(r["y"][0], (P1 @ T.astype(np.float64)).astype(np.float32))


# ---------------------------------------------------------------- reachable ranges

def _midpoint_case(dt, boundary, p, big, ncols):
    """x [1, 2, ncols], P1 = diag(p, 1), P2 = I + E[1, 0]: T[0, 0] = x[0, 0] + x[0, 1] is the
    midpoint between the two dtype neighbours lo_t < boundary / p < hi_t, so y[0, 0] = p T[0, 0]
    reaches boundary from either side depending on how T is rounded; y[1, 0] = big sets the
    scale.  Returns the inputs and (lo_t, hi_t)."""
    t_star = boundary / p
    e = math.floor(math.log2(t_star))
    ulp = 2.0 ** (e - FRAC[dt])
    lo_t = math.floor(t_star / ulp) * ulp
    hi_t = lo_t + ulp
    assert lo_t < t_star < hi_t
    x = np.zeros((1, 2, ncols))
    x[0, 0, 0], x[0, 0, 1] = lo_t, ulp / 2
    x[0, 1, 0] = big
    p2 = np.eye(ncols)
    p2[1, 0] = 1.0
    p1 = np.diag([p, 1.0])
    xb, p1b, p2b = rt(x, dt), rt(p1, dt), rt(p2, dt)
    assert np.array_equal(val(xb, dt), x) and np.array_equal(val(p1b, dt), p1)  # all exact
    return xb, p1b, p2b, lo_t, hi_t


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_t_midpoint_flags_both_int4_codes(dt):
    """An x . P2 sum exactly on a dtype midpoint: the oracle rounds it half to even, and the
    y it feeds can land on either side of the int4 boundary 1.5 -- both codes must be
    reachable, and no other element may be flagged."""
    p = 0.6875
    xb, p1b, p2b, lo_t, hi_t = _midpoint_case(dt, 1.5, p, 7.0, 8)
    r = oracle.run(xb, p1b, p2b, dt, "int32", clip_ratio=1.0, want_y=True)
    assert r["scale"][0] == 1.0  # max|y| = 7, d = 7
    t_rne = to_dt(lo_t + (hi_t - lo_t) / 2, dt)[()]
    assert t_rne in (lo_t, hi_t)
    code = lambda q: int(round(q))  # Python rounds half to even; these q are not ties
    assert r["lvl"][0, 0] == code(p * t_rne)
    alts = sorted({code(p * lo_t), code(p * hi_t)})
    assert alts == [1, 2]
    assert (r["lo"][0, 0], r["hi"][0, 0]) == (1, 2)
    assert r["ns_tie"][0, 0] == 0  # not a tie of the code itself: the intermediate's
    rest = np.arange(1, 16)
    assert (r["lo"][0, rest] == r["hi"][0, rest]).all()
    # the scale is set by an exact element: its interval is the stated window only
    assert abs(r["scale_lo"][0] - 1.0) <= 1e-5 and abs(r["scale_hi"][0] - 1.0) <= 1e-5


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_t_midpoint_flags_both_e2m1_codes(dt):
    """The same for E2M1 at its decision point 1.25 (between 1.0 and 1.5), group max 4.5
    (e8m0 127, scale 1, far from a power of two)."""
    p = 0.6875
    xb, p1b, p2b, lo_t, hi_t = _midpoint_case(dt, 1.25, p, 4.5, 2)
    r = oracle.run(xb, p1b, p2b, dt, "fp4", dst_type_max=0.0)
    assert r["e8m0"][0, 0] == 127 and r["g_lo"][0, 0] == r["g_hi"][0, 0] == 127
    t_rne = to_dt(lo_t + (hi_t - lo_t) / 2, dt)[()]
    idx = lambda v: oracle.e2m1_code(v) & 7
    assert r["lvl"][0, 0] == idx(p * t_rne)
    assert sorted({idx(p * lo_t), idx(p * hi_t)}) == [2, 3]
    assert (r["lo"][0, 0], r["hi"][0, 0]) == (2, 3)
    assert r["ns_tie"][0, 0] == 0
    assert r["lo"][0, 2] == r["hi"][0, 2] == 6  # 4.5 -> 4, far from 5
    assert r["lo"][0, 1] == r["hi"][0, 1] == 0


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_t_midpoint_on_the_largest_element_widens_the_scale_interval(dt):
    """When the sum on a midpoint is the slice's largest element, the scale itself is
    ambiguous: the reachable interval must hold the scales of both roundings."""
    p = 0.6875
    xb, p1b, p2b, lo_t, hi_t = _midpoint_case(dt, 1.5, p, 0.25, 8)  # y[0, 0] is now the max
    r = oracle.run(xb, p1b, p2b, dt, "int32", clip_ratio=1.0)
    d = np.float32(7.0)
    for t in (lo_t, hi_t):
        s = np.float32(np.float32(p * t) / d)
        assert r["scale_lo"][0] <= s <= r["scale_hi"][0]
    # wider than the 1e-5 scale tolerance by far: one dtype step of the largest element
    assert r["scale_hi"][0] / r["scale_lo"][0] - 1 > 5e-4


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["int32", "fp4"])
def test_far_from_every_boundary_gives_one_code(dt, mode):
    """Every x . P2 sum exact and far from a dtype midpoint, every y exact and far from a code
    boundary, every group maximum far from a power of two: each element has a single
    reachable code, each group a single e8m0 code, the scale a tight interval."""
    rng = np.random.default_rng(7)
    M = N = 16
    P2 = np.eye(N) + 0.5 * np.roll(np.eye(N), 1, axis=1)          # T[m, n] = x[m, n] + x[m, n-1] / 2
    P1 = np.eye(M)[rng.permutation(M)] * rng.choice([-1.0, 1.0], M)
    if mode == "int32":
        x = 2.0 * rng.integers(-2, 3, size=(1, M, N))               # T integers in [-6, 6]
        x[0, 0, :] = 0.0
        x[0, 0, 4], x[0, 0, 5] = 6.0, 4.0                           # T[0, 5] = 7: the largest, scale 1
    else:
        x = 2.0 * rng.integers(-1, 2, size=(1, M, N))               # T integers in [-3, 3]
        x[0, :, 0] = 2.0
        x[0, :, 1] = 2.0                                            # T[m, 1] = 3: every group's max is 3
    r = oracle.run(rt(x, dt), rt(P1, dt), rt(P2, dt), dt, mode, clip_ratio=1.0, want_y=True)
    y = r["y"][0].astype(np.float64)
    assert np.array_equal(y, P1 @ (x[0] @ P2))  # exact
    assert (r["lo"] == r["hi"]).all() and (r["ns_tie"] == 0).all()
    if mode == "int32":
        # within the 1e-5 scale tolerance: only the fp32 accumulation bound remains
        assert r["scale"][0] == 1.0 and abs(r["scale_hi"][0] / r["scale_lo"][0] - 1) < 1e-5
    else:
        assert (r["e8m0"][0, :8] == 126).all() and (r["g_lo"] == r["g_hi"]).all()
        # no alternative scale: the alternative pass is the primary one
        assert (r["g_alt"] == r["e8m0"][:, :r["g_alt"].shape[1]]).all()
        assert (r["alt_lvl"] == r["lvl"]).all() and (r["alt_lo"] == r["lo"]).all() and (r["alt_hi"] == r["hi"]).all()


def _fp32_sums_every_order(terms):
    """Every value an fp32 sum of `terms` (exact fp32 products) can take over all orders of
    sequential accumulation and both pairings of 4 terms."""
    terms = [np.float32(t) for t in terms]
    out = set()
    for perm in itertools.permutations(terms):
        acc = np.float32(0.0)
        for t in perm:
            acc = np.float32(acc + t)
        out.add(float(acc))
        if len(perm) == 4:
            out.add(float(np.float32(np.float32(perm[0] + perm[1]) + np.float32(perm[2] + perm[3]))))
    return out


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_reachable_range_holds_every_summation_order(dt):
    """Brute force on 3 x 3 blocks with terms of widely spread magnitudes: every combination
    of fp32 summation orders of the x . P2 sums of a column and of the P1 . T sum, with T
    rounded to the dtype in between, gives an int4 code inside the oracle's reachable range;
    the oracle's own code is that of the correctly rounded sums.  (Random terms rarely reach
    two codes; the cancellation case below is built to.)  A fourth row and column hold one
    exact element, larger than every other, that fixes the scale."""
    rng = np.random.default_rng(3 if dt == "bf16" else 4)
    n = 3
    multi = checked = 0

    def spread(shape):
        return rng.choice([-1.0, 1.0], shape) * 2.0 ** rng.uniform(-3, 4, shape)

    for trial in range(60):
        x = np.zeros((1, n + 1, n + 1))
        x[0, :n, :n] = spread((n, n))
        p2 = np.zeros((n + 1, n + 1))
        p2[:n, :n] = spread((n, n))
        p1 = np.zeros((n + 1, n + 1))
        p1[:n, :n] = spread((n, n))
        p1[n, n] = p2[n, n] = 1.0
        Xb, P1b, P2b = rt(x[0, :n, :n], dt), rt(p1, dt), rt(p2, dt)
        X = np.zeros((n + 1, n + 1))
        X[:n, :n] = val(Xb, dt)
        P1, P2 = val(P1b, dt), val(P2b, dt)
        ymax = np.abs(P1 @ (X @ P2)).max()
        X[n, n] = val(rt(2.0 ** math.ceil(math.log2(ymax * 1.5)) * 1.75, dt), dt)  # > every other |y|
        xb = rt(X[None], dt)
        if dt == "f16" and not np.isfinite(val(xb, dt)).all():
            continue
        r = oracle.run(xb, P1b, P2b, dt, "int32", clip_ratio=1.0)
        scale = np.float32(r["scale"][0])
        assert scale == np.float32(np.float32(X[n, n]) / np.float32(7.0))
        for i in range(n):
            for col in range(n):
                t_sets = [sorted({to_dt(s, dt)[()] for s in _fp32_sums_every_order(X[m, :] * P2[:, col])})
                          for m in range(n + 1)]
                codes = set()
                for ts in itertools.product(*t_sets):
                    for yv in _fp32_sums_every_order([P1[i, m] * ts[m] for m in range(n + 1)]):
                        codes.add(oracle.int4_code(float(np.float32(np.float32(yv) / scale))))
                # the correctly rounded path: T = RNE_dt(fl32(exact)), y = fl32(exact P1 . T)
                t_ok = to_dt(X @ P2[:, col], dt)
                q_ok = np.float32(np.float32(P1[i] @ t_ok) / scale)
                f = i * (n + 1) + col
                assert r["lvl"][0, f] == oracle.int4_code(float(q_ok))
                lo, hi = int(r["lo"][0, f]), int(r["hi"][0, f])
                assert all(lo <= c <= hi for c in codes), (trial, i, col, codes, lo, hi)
                checked += 1
    assert checked > 400, checked


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_cancellation_reaches_two_codes_in_fp32_and_is_flagged(dt):
    """y[0, 0] = B - B + v with B = 2^20 (2^15 in fp16) and v just above the int4 boundary
    0.5 (scale 1): summed in the order (B - B) + v it is v (code 1), in the order (B + v) - B
    the fp32 sum drops v's low bits and lands on the tie 0.5 (code 0).  Brute force over every
    order gives both codes, and the oracle must report exactly that range, with the code of
    the correctly rounded sum as its own."""
    B = 2.0 ** 20 if dt == "bf16" else 2.0 ** 15
    v = 0.5 + 2.0 ** -(FRAC[dt] + 1)  # the dtype value next above 0.5
    x = np.zeros((1, 4, 2))
    x[0, 0, 0] = x[0, 1, 0] = B
    x[0, 2, 0] = v
    x[0, 3, 1] = 7.0                         # y[3, 1] = 7: scale 1
    p1 = np.zeros((4, 4))
    p1[0, :3] = [1.0, -1.0, 1.0]
    p1[3, 3] = 1.0
    xb, p1b, p2b = rt(x, dt), rt(p1, dt), rt(np.eye(2), dt)
    assert np.array_equal(val(xb, dt), x)
    r = oracle.run(xb, p1b, p2b, dt, "int32", clip_ratio=1.0)
    assert r["scale"][0] == 1.0
    codes = {oracle.int4_code(float(np.float32(s))) for s in _fp32_sums_every_order([B, -B, v])}
    assert codes == {0, 1}
    assert r["lvl"][0, 0] == 1 and (r["lo"][0, 0], r["hi"][0, 0]) == (0, 1)
    assert (r["lo"][0, 1:] == r["hi"][0, 1:]).all()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_order_that_loses_three_fp32_steps_is_flagged(dt):
    """T[0, 0] = 1 + (half a dtype step) + six terms of 2^-24 (half an fp32 step at 1): the
    exact sum lies 3 fp32 steps above the dtype midpoint 1 + ulp/2, so the correctly rounded T
    is the dtype value above.  Summed from 1 upwards every 2^-24 is a tie that rounds back to
    even, and the fp32 sum is the midpoint itself, which rounds half to even to 1.0: one order
    gives the other T, and with it the other int4 code.  Brute force over every order
    confirms both; the oracle's range must contain both.  The fp32 error bound gamma_8 times
    the terms' magnitude is about 4.2 fp32 steps here and the error is 3 steps, so a bound
    of half the size (2.1 steps) would miss that order."""
    half_dt = 2.0 ** -(FRAC[dt] + 1)
    lo_t, hi_t, mid = 1.0, 1.0 + 2 * half_dt, 1.0 + half_dt
    p = 1.4921875 if dt == "bf16" else 1.4990234375  # p lo_t < 1.5 < p hi_t
    terms = [lo_t, half_dt] + [2.0 ** -24] * 6
    sums = _fp32_sums_every_order(terms)
    assert min(sums) == mid and max(sums) == mid + 3 * 2.0 ** -23
    assert sorted({float(to_dt(s, dt)) for s in sums}) == [lo_t, hi_t]
    x = np.zeros((1, 2, 8))
    x[0, 0, :] = terms
    x[0, 1, 0] = 7.0                        # y[1, 0] = 7: scale 1
    p2 = np.eye(8)
    p2[1:, 0] = 1.0                         # T[0, 0] = sum of row 0
    p1 = np.diag([p, 1.0])
    xb, p1b, p2b = rt(x, dt), rt(p1, dt), rt(p2, dt)
    assert np.array_equal(val(xb, dt), x) and np.array_equal(val(p1b, dt), p1)
    r = oracle.run(xb, p1b, p2b, dt, "int32", clip_ratio=1.0)
    assert r["scale"][0] == 1.0
    assert p * lo_t < 1.5 < p * hi_t
    assert r["lvl"][0, 0] == 2 and (r["lo"][0, 0], r["hi"][0, 0]) == (1, 2)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_long_sum_that_ties_down_at_every_step_is_flagged(dt):
    """y[0, 0] = sum over 256 rows of T[m, 0] (P1's first row all ones, P2 = I), per group:
    the terms 1.25, -2^-19 and -2^-22 form m' = 1.25 - 18 fp32 steps (even), and 253 terms of
    half an fp32 step follow.  The group's maximum y[0, 1] = 3 is far from a power of two, so
    its e8m0 scale (0.5) is certain and y[0, 0] / 0.5 sits near the E2M1 decision point 2.5.
    The exact sum is 1.25 + 108.5 steps (code of 3.0); summed from m' upwards every half step
    is a tie that rounds back to even and the fp32 sum stays m' (code of 2.0).  Both points
    lie outside the 1e-6 tie window, so only the fp32 error bound of GEMM2 can reach the
    lower code: gamma_256 times the terms' magnitude is 160 steps here, half of it (80) would
    not reach below the decision point."""
    step = 2.0 ** -23
    head = [1.25, -(2.0 ** -19), -(2.0 ** -22)]
    tail = [2.0 ** -24] * 253
    acc = np.float32(0.0)
    for t in head + tail:  # one order: m' first, then the ties
        acc = np.float32(acc + np.float32(t))
    assert float(acc) == 1.25 - 18 * step
    exact = sum(head) + sum(tail)
    assert exact == 1.25 + 108.5 * step
    assert abs(float(acc) - 1.25) > 1e-6 * 1.25 and abs(exact - 1.25) > 1e-6 * 1.25  # outside the tie window
    M, N = 256, 32
    x = np.zeros((1, M, N))
    x[0, :, 0] = head + tail
    x[0, 1, 1] = 3.0                        # y[0, 1] = 3: group 0's maximum, e8m0 code 126
    p1 = np.zeros((M, M))
    p1[0, :] = 1.0
    xb, p1b, p2b = rt(x, dt), rt(p1, dt), rt(np.eye(N), dt)
    assert np.array_equal(val(xb, dt), x)
    r = oracle.run(xb, p1b, p2b, dt, "fp4", dst_type_max=0.0)
    assert r["e8m0"][0, 0] == 126
    code = lambda v: [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0].index(v)
    assert r["lvl"][0, 0] == code(3.0) and (r["lo"][0, 0], r["hi"][0, 0]) == (code(2.0), code(3.0))
    assert r["ns_tie"][0, 0] == 0  # not flagged by the tie window


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_group_max_next_to_a_power_of_two_reaches_both_e8m0_codes(dt):
    """y[0, 0] = 2^1 + 2^0 + ... + 2^-21 = 4 - 2^-21 (P1's first row all ones over x's
    column of powers of two: every term and every partial sum exact), the maximum of its
    group, lies within reach of 4 (V1: e8m0 code 126 below 4, 127 at 4); y[0, 1] = 1.  The
    oracle's code is 126, the reachable range 126 .. 127 with 127 as the alternative, and the
    codes under both scales are those of y / 2^(code - 127): the maximum saturates to 6 under
    126 and rounds to 4 under 127; y[0, 1] gives 2 and 1."""
    M, N = 32, 32
    x = np.zeros((1, M, N))
    x[0, :23, 0] = [2.0 ** (1 - m) for m in range(23)]
    x[0, 0, 1] = 1.0
    p1 = np.zeros((M, M))
    p1[0, :] = 1.0
    xb, p1b, p2b = rt(x, dt), rt(p1, dt), rt(np.eye(N), dt)
    assert np.array_equal(val(xb, dt), x)
    assert sum(x[0, :, 0]) == 4.0 - 2.0 ** -21
    r = oracle.run(xb, p1b, p2b, dt, "fp4", dst_type_max=0.0, want_y=True)
    assert r["y"][0, 0, 0] == np.float32(4.0 - 2.0 ** -21) and r["y"][0, 0, 1] == 1.0
    assert r["e8m0"][0, 0] == 126
    assert (r["g_lo"][0, 0], r["g_hi"][0, 0], r["g_alt"][0, 0]) == (126, 127, 127)
    code = lambda v: [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0].index(v)
    assert r["lvl"][0, 0] == code(6.0) and r["alt_lvl"][0, 0] == code(4.0)
    assert r["lvl"][0, 1] == code(2.0) and r["alt_lvl"][0, 1] == code(1.0)
    assert (r["lo"][0, :2] == r["hi"][0, :2]).all() and (r["alt_lo"][0, :2] == r["alt_hi"][0, :2]).all()
