"""Pins of the oracle to what the pages and mathematics fix (CPU only).

Each test ties one part of the oracle to something other than itself: values printed on
the pages (fixtures under tests/golden), an independent library routine, a brute-force
search, a closed form or an invariant.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import keyed, rows

pytestmark = pytest.mark.filterwarnings("ignore")


def bf16(vals):
    return synth.round_to(np.asarray(vals, dtype=np.float64), "bf16")


def f32_of_bits(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- E2M1 encoder


def test_e2m1_magnitudes_match_page_table():
    mags = [float(v) for v in keyed("e2m1_table.txt")["magnitudes"]]
    assert mags == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for code in range(16):
        v = oracle.e2m1_value(code)
        assert abs(v) == mags[code & 7]
        assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0)
        # decode -> encode round trip over all 16 codes (-0 keeps its sign bit)
        assert oracle.e2m1_code(v) == code


def test_e2m1_decision_points_from_page():
    for r in rows("e2m1_table.txt")[1:]:
        p, below, above, at = (float(t) for t in r)
        lo = np.nextafter(p, 0.0)
        hi = np.nextafter(p, np.inf)
        assert oracle.e2m1_value(oracle.e2m1_code(lo)) == below
        assert oracle.e2m1_value(oracle.e2m1_code(hi)) == above
        assert oracle.e2m1_value(oracle.e2m1_code(p)) == at
        assert oracle.e2m1_value(oracle.e2m1_code(-p)) == -at


def _e2m1_by_format_rounding(v):
    """E2M1 as a binary float format: 1 mantissa bit, exponents 0..2, subnormal quantum
    0.5; round half to even with numpy's rint at the binade's quantum, saturate at 6."""
    a = abs(v)
    if a < 2.0:
        q = 0.5
    elif a < 4.0:
        q = 1.0
    else:
        q = 2.0
    r = float(np.rint(a / q)) * q
    r = min(r, 6.0)
    return math.copysign(r, v)


def test_e2m1_dense_sweep_against_format_rounding():
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    vals = list(np.linspace(-9, 9, 20001))
    for p in pts:
        for s in (-1, 1):
            x = s * p
            vals += [x, np.nextafter(x, -np.inf), np.nextafter(x, np.inf)]
            vals += list(x + np.arange(-4, 5) * 2.0 ** -20)
    for v in vals:
        v = float(v)
        got = oracle.e2m1_value(oracle.e2m1_code(v))
        want = _e2m1_by_format_rounding(v)
        assert got == want, (v, got, want)


# ---------------------------------------------------------------- int4 encoder


def test_int4_rne_examples_from_page():
    for inp, exp in rows("rne_examples.txt"):
        assert oracle.int4_code(float(inp)) == int(float(exp))


def test_int4_clamp_range_from_page():
    k = keyed("int4_range.txt")
    b, lo, hi = int(k["bits"][0]), int(k["min"][0]), int(k["max"][0])
    assert (lo, hi) == (-(2 ** (b - 1)), 2 ** (b - 1) - 1)
    assert oracle.int4_code(-100.0) == lo and oracle.int4_code(100.0) == hi
    assert oracle.int4_code(-8.5) == -8 and oracle.int4_code(7.5) == 7
    assert oracle.int4_code(-8.49) == -8 and oracle.int4_code(6.51) == 7


def test_int4_brute_force_nearest_even():
    codes = np.arange(-8, 8)
    grid = list(np.linspace(-9.5, 8.5, 7201))
    for n in range(-9, 9):
        t = n + 0.5
        grid += [t, float(np.nextafter(np.float32(t), np.float32(-np.inf))),
                 float(np.nextafter(np.float32(t), np.float32(np.inf)))]
    for q in grid:
        q32 = float(np.float32(q))
        d = np.abs(codes - q32)
        best = codes[d == d.min()]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert oracle.int4_code(q32) == want, q32


# ---------------------------------------------------------------- dtype rounding


def test_round_f32_matches_numpy_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        rng.standard_normal(2000) * 1e-42])
    for x in v:
        assert oracle.round_f32(float(x)) == float(np.float32(x))


def test_round_f16_matches_numpy_cast():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
                        (np.arange(-3000, 3000) + 0.5) * 2.0 ** -24])  # subnormal ties
    for x in v:
        want = float(np.float16(x))
        got = oracle.round_dt(float(x), "f16")
        assert got == want or (math.isinf(got) and math.isinf(want)), x


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    ties = (np.arange(1, 2000, dtype=np.float32) * 2 ** 7 + 2 ** 6).view(np.float32)  # exact ties
    v = np.concatenate([v, ties[np.isfinite(ties)]])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    for x, w in zip(v, want):
        assert oracle.round_dt(float(x), "bf16") == w, x


# ---------------------------------------------------------------- e8m0 scales


def test_e8m0_v1_invariant_scaled_max_in_4_8():
    rng = np.random.default_rng(4)
    amax = np.float32(np.abs(rng.standard_normal(20000)) * 10.0 ** rng.integers(-30, 30, 20000))
    for a in amax:
        if a == 0:
            continue
        c = oracle.e8m0_v1(float(a))
        assert 0 <= c <= 254
        r = float(a) * 2.0 ** (127 - c)  # scale 2^(c-127) is a power of two by construction
        assert 4.0 <= r < 8.0, (a, c)


def test_e8m0_v2_invariant_scaled_max_in_half_dmax_dmax():
    rng = np.random.default_rng(5)
    amax = np.float32(np.abs(rng.standard_normal(20000)) * 10.0 ** rng.integers(-30, 30, 20000))
    for dmax in (6.0, 7.5, 8.0, 10.0, 12.0):
        for a in amax:
            c = oracle.e8m0_v2(float(a), dmax)
            S = float(np.float32(np.float32(a) / np.float32(dmax)))
            if S < 2.0 ** -126:
                continue
            r = float(a) * 2.0 ** (127 - c)
            assert dmax / 2 < r <= dmax * (1 + 2.0 ** -23), (a, dmax, c)


def test_e8m0_v2_bits_and_frexp_agree():
    rng = np.random.default_rng(6)
    vals = list(np.float32(np.abs(rng.standard_normal(50000)) * 10.0 ** rng.integers(-44, 38, 50000)))
    vals += [np.float32(2.0 ** e) for e in range(-140, 128)]
    vals += [np.nextafter(np.float32(2.0 ** e), np.float32(0)) for e in range(-120, 128)]
    vals += [np.float32(0.0), np.float32(1e-45), np.float32(3.4e38)]
    for dmax in (6.0, 8.0, 11.0, 12.0):
        for a in vals:
            assert oracle.e8m0_v2(float(a), dmax, "bits") == oracle.e8m0_v2(float(a), dmax, "frexp"), a


def test_v2_dmax8_equals_v1_except_powers_of_two():
    """With dstTypeMax = 8: S = amax/8 is exact, so V2's ceil exponent equals V1's
    floor(log2 amax) - 2 unless amax is a power of two, where it is one less."""
    rng = np.random.default_rng(7)
    vals = list(np.float32(np.abs(rng.standard_normal(20000)) * 10.0 ** rng.integers(-20, 20, 20000)))
    vals += [np.float32(2.0 ** e) for e in range(-60, 60)]
    for a in vals:
        if a == 0:
            continue
        v1 = oracle.e8m0_v1(float(a))
        v2 = oracle.e8m0_v2(float(a), 8.0)
        m, _ = math.frexp(float(a))
        assert v2 == (v1 - 1 if m == 0.5 else v1), a


# ---------------------------------------------------------------- transform


def _gen_small_exact(rng, M, N):
    x = rng.integers(-4, 5, size=(1, M, N)).astype(np.float64)
    p1 = rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=(M, M))
    p2 = rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=(N, N))
    return x, p1, p2


@pytest.mark.parametrize("M,N", [(1, 2), (2, 2), (3, 4), (4, 8), (8, 8), (5, 6)])
def test_kronecker_closed_form(M, N):
    """vec_row(P1 x P2) = (P1 kron P2^T) vec_row(x), with inputs whose intermediate is
    exact in bf16, so every reading of the intermediate precision agrees."""
    rng = np.random.default_rng(M * 100 + N)
    for _ in range(5):
        x, p1, p2 = _gen_small_exact(rng, M, N)
        r = oracle.run(bf16(x), bf16(p1), bf16(p2), "bf16", "fp4", want_y=True, ranges=False)
        want = (np.kron(p1, p2.T) @ x.reshape(-1)).reshape(M, N)
        assert np.array_equal(r["y"][0].astype(np.float64), want)
        # left-only equals the two-sided transform with P2 = I
        r2 = oracle.run(bf16(x), bf16(p1), None, "bf16", "fp4", want_y=True, ranges=False)
        assert np.array_equal(r2["y"][0].astype(np.float64), p1 @ x[0])


def test_transform_order_p2_first_then_p1():
    """A non-exact intermediate makes the order observable: T = RNE(x P2) first."""
    rng = np.random.default_rng(11)
    M, N = 4, 4
    x = rng.standard_normal((1, M, N))
    p1 = rng.standard_normal((M, M))
    p2 = rng.standard_normal((N, N))
    xb, p1b, p2b = bf16(x), bf16(p1), bf16(p2)
    r = oracle.run(xb, p1b, p2b, "bf16", "int32", want_y=True, want_t=True, ranges=False)
    X, P1, P2 = (f32_of_bits(a).astype(np.float64) for a in (xb[0], p1b, p2b))
    T = torch.from_numpy((X @ P2).astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(f32_of_bits(r["t"][0]).astype(np.float64), T)
    assert np.array_equal(r["y"][0], (P1 @ T).astype(np.float32))


def test_identity_permutation_sign_transforms_are_exact():
    rng = np.random.default_rng(12)
    M, N = 16, 32
    x = synth.gen_x(M, N, "bf16", "gauss", 0.05, 20.0, seed=3, k0=0, k1=2)
    for trial in range(3):
        pm = np.eye(M)[rng.permutation(M)] * rng.choice([-1.0, 1.0], size=M)
        pn = np.eye(N)[rng.permutation(N)] * rng.choice([-1.0, 1.0], size=N)
        r = oracle.run(x, bf16(pm), bf16(pn), "bf16", "int32", want_y=True)
        X = f32_of_bits(x).astype(np.float64)
        want = np.einsum("im,kmn,nj->kij", pm, X, pn)
        assert np.array_equal(r["y"].astype(np.float64), want)
        # the transform is exact, so no code is ambiguous through the intermediate
        assert (r["zsign"] == 0).all()


# ---------------------------------------------------------------- per-token mode


def test_worked_pertoken_example():
    k = keyed("worked_pertoken.txt")
    clip = float(k["clip"][0])
    x = np.array([float(v) for v in k["x"]]).reshape(1, 2, 6)
    r = oracle.run(bf16(x), bf16(np.eye(2)), bf16(np.eye(6)), "bf16", "int32", clip_ratio=clip)
    assert r["scale"][0] == float(k["scale"][0])
    codes = [int(v) for v in k["codes"]]
    assert list(r["lvl"][0]) == codes
    packed = r["packed"][0]
    nib = [(b >> s) & 0xF for b in packed for s in (0, 4)]
    assert nib == [c & 0xF for c in codes]


@pytest.mark.parametrize("cfg", ["c1", "c2"])
def test_pertoken_invariants(cfg):
    w = synth.WORKLOADS[cfg]
    x, p1, p2 = synth.make_inputs(w, 0, 8)
    r = oracle.run(x, p1, p2, w.dtype, w.mode, w.clip_ratio, want_y=True)
    y = r["y"].reshape(8, -1).astype(np.float64)
    amax = np.abs(y).max(axis=1)
    s = r["scale"].astype(np.float64)
    d = float(np.float32(7.0 / w.clip_ratio))
    assert np.all(np.abs(s * d - amax) <= amax * 2.0 ** -23)  # one fp32 rounding
    c = r["lvl"].astype(np.float64)
    unclamped = (c > -8) & (c < 7)
    assert np.all(np.abs(y - c * s[:, None])[unclamped] <= (s[:, None] * 0.5 * (1 + 1e-6)).repeat(
        y.shape[1], 1)[unclamped])
    assert c.min() >= -8 and c.max() <= 7


def test_pertoken_clip_below_one_reaches_minus_eight():
    """clipRatio < 7/7.5 lets |q| exceed 7.5, so the int4 range's -8 is used."""
    w = synth.WORKLOADS["c2"]
    x, p1, p2 = synth.make_inputs(w, 0, 64)
    r = oracle.run(x, p1, p2, w.dtype, w.mode, w.clip_ratio, ranges=False)
    assert (r["lvl"] == -8).any()
    r1 = oracle.run(x, p1, p2, w.dtype, w.mode, 1.0, ranges=False)
    assert not (r1["lvl"] == -8).any()


def test_pertoken_zero_slice():
    x = np.zeros((2, 4, 8), np.uint16)
    r = oracle.run(x, bf16(np.eye(4)), bf16(np.eye(8)), "bf16", "int32")
    assert (r["scale"] == 0).all() and (r["packed"] == 0).all()
    assert (r["lo"] == 0).all() and (r["hi"] == 0).all()


# ---------------------------------------------------------------- per-group mode


def _hexes(vals):
    return [int(v, 16) for v in vals]


def test_worked_pergroup_examples():
    k = keyed("worked_pergroup.txt")
    xa = np.array([float(v) for v in k["xA"]]).reshape(1, 1, 32)
    one = bf16(np.ones((1, 1)))
    eye = bf16(np.eye(32))

    def codes(r):
        return [(b >> s) & 0xF for b in r["packed"][0] for s in (0, 4)]

    ra = oracle.run(bf16(xa), one, eye, "bf16", "fp4", dst_type_max=0.0)
    assert ra["e8m0"][0, 0] == int(k["e8m0A_v1"][0])
    assert codes(ra) == _hexes(k["codesA"])
    xb = bf16(2 * xa)
    for key, dmax in (("e8m0B_v1", 0.0), ("e8m0B_v2_6", 6.0), ("e8m0B_v2_8", 8.0),
                      ("e8m0B_v2_10", 10.0)):
        rb = oracle.run(xb, one, eye, "bf16", "fp4", dst_type_max=dmax)
        assert rb["e8m0"][0, 0] == int(k[key][0]), key
        if dmax in (0.0, 6.0, 8.0):
            assert codes(rb) == _hexes(k["codesA"]), key
        else:
            assert codes(rb) == _hexes(k["codesB_v2_10"])
    # left-only gives the same with an identity P1
    rl = oracle.run(bf16(xa), one, None, "bf16", "fp4")
    assert codes(rl) == _hexes(k["codesA"])


@pytest.mark.parametrize("dmax,lo,hi", [(0.0, 4.0, 8.0), (6.0, 3.0, 6.0), (8.0, 4.0, 8.0),
                                        (10.0, 5.0, 10.0), (12.0, 6.0, 12.0)])
def test_pergroup_scale_invariants(dmax, lo, hi):
    w = synth.WORKLOADS["c3"]
    x, p1, p2 = synth.make_inputs(w, 0, 4)
    r = oracle.run(x, p1, p2, w.dtype, "fp4", dst_type_max=dmax, want_y=True, ranges=False)
    y = r["y"].reshape(4, -1, 32).astype(np.float64)
    amax = np.abs(y).max(axis=2)
    code = r["e8m0"][:, : amax.shape[1]].astype(np.int64)
    scaled = amax * 2.0 ** (127 - code)
    if dmax == 0.0:
        assert np.all((scaled >= lo) & (scaled < hi))
    else:
        assert np.all((scaled > lo) & (scaled <= hi * (1 + 2.0 ** -23)))


def test_v1_and_v2_at_6_differ_and_v2_at_0_is_v1():
    """dstTypeMax 0.0 behaves as V1 (floor exponent); 6.0 is the V2 ceil path and gives a
    different scale for most groups."""
    w = synth.WORKLOADS["c3"]
    x, p1, p2 = synth.make_inputs(w, 0, 4)
    r0 = oracle.run(x, p1, p2, w.dtype, "fp4", dst_type_max=0.0, want_y=True, ranges=False)
    r6 = oracle.run(x, p1, p2, w.dtype, "fp4", dst_type_max=6.0, ranges=False)
    y = r0["y"].reshape(4, -1, 32)
    amax = np.abs(y).max(axis=2)
    v1 = np.vectorize(lambda a: oracle.e8m0_v1(float(a)))(amax)
    assert np.array_equal(r0["e8m0"][:, : amax.shape[1]], v1)
    # V1 puts the group max in [4, 8) of the scale, V2 at 6 in (3, 6]: they differ exactly
    # for the groups whose V1-scaled max exceeds 6
    G = amax.shape[1]
    scaled_v1 = amax.astype(np.float64) * 2.0 ** (127 - r0["e8m0"][:, :G].astype(np.int64))
    differ = r6["e8m0"][:, :G] != r0["e8m0"][:, :G]
    assert np.array_equal(differ, scaled_v1 > 6.0)
    assert differ.any() and not differ.all()


def test_partial_group_and_pad_slot():
    """M*N = 30: one partial group; 96: three groups, so the [.., 2] pair has a pad slot."""
    rng = np.random.default_rng(13)
    for M, N in ((3, 10), (3, 32), (1, 2)):
        x = bf16(rng.standard_normal((2, M, N)) * 3)
        r = oracle.run(x, bf16(np.eye(M)), bf16(np.eye(N)), "bf16", "fp4", want_y=True)
        MN = M * N
        G, GS = -(-MN // 32), 2 * (-(-MN // 64))
        assert r["e8m0"].shape == (2, GS)
        if GS > G:
            assert (r["e8m0"][:, G:] == 0).all()
        for s in range(2):
            for g in range(G):
                a = np.abs(r["y"][s].reshape(-1)[32 * g:32 * g + 32]).max()
                assert r["e8m0"][s, g] == oracle.e8m0_v1(float(a))


# ---------------------------------------------------------------- layouts


def test_example_shapes_from_page():
    k = keyed("example_shapes.txt")
    K, M, N = (int(v) for v in k["x"][1:])
    out_shape = tuple(int(v) for v in k["out"][1:])
    assert out_shape == (K, M, N // 8)
    assert tuple(int(v) for v in k["quantScale"][1:]) == (K,)
    x = synth.gen_x(M, N, "f16", "gauss", 0.0, 1.0, 0, 0, K)
    p = synth.gen_orthogonal(M, "f16", 0, 2)
    r = oracle.run(x, p, synth.gen_orthogonal(N, "f16", 0, 3), "f16", "int32",
                   clip_ratio=float(k["clipRatio"][0]), ranges=False)
    # INT32 [K, M, N/8] holds 8 codes per little-endian word, low nibble first, which is
    # byte for byte the INT4 [K, M, N] layout (2 per byte, low nibble first)
    words = r["packed"].reshape(-1).view("<i4").reshape(out_shape)
    lv = r["lvl"].reshape(K, M, N)
    for i in range(8):
        nib = ((words.astype(np.int64) >> (4 * i)) & 0xF)
        assert np.array_equal(np.where(nib >= 8, nib - 16, nib), lv[:, :, i::8])
    assert r["scale"].shape == (K,)


# ---------------------------------------------------------------- dequantization
# Pins of oracle.dequant against independent routines: numpy's IEEE fp32 arithmetic and
# ldexp, numpy's fp32 -> fp16 cast and torch's fp32 -> bf16 cast (both round to nearest
# even), and the E2M1 magnitudes the ModelOpt page prints (section 6.1, tests/golden).


def _to_dt_bits(v32, dtype):
    v32 = np.asarray(v32, dtype=np.float32)
    if dtype == "bf16":
        return torch.from_numpy(v32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return v32.astype(np.float16).view(np.uint16)


def _same_bits(got, want, dtype):
    """Equal bits, NaN for NaN (any payload)."""
    g = oracle.dt_to_float(got, dtype)
    w = oracle.dt_to_float(want, dtype)
    nan = np.isnan(w)
    assert np.array_equal(np.isnan(g), nan)
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_dequant_per_group_every_code_and_e8m0(dtype):
    # one slice of 32 * 256 elements: group g = e8m0 byte g, element j of a group = code j % 16
    M, N = 256, 32
    codes = np.tile(np.arange(16, dtype=np.uint8), 2 * 256)            # [256 * 32]
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    e8 = np.zeros((1, 2 * (-(-M * N // 64))), np.uint8)
    e8[0, :256] = np.arange(256, dtype=np.uint8)
    got = oracle.dequant(packed, e8, M, N, dtype, "fp4").reshape(-1)
    page = np.array([float(v) for v in keyed("e2m1_table.txt")["magnitudes"]])
    mag = page[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    e = np.repeat(np.arange(256), 32)
    with np.errstate(over="ignore"):
        v32 = np.ldexp(mag, e - 127).astype(np.float32)              # exact, or inf
    v32[e == 255] = np.nan
    _same_bits(got, _to_dt_bits(v32, dtype), dtype)
    assert (got[(codes == 8) & (e < 255)] == 0x8000).all()  # -0 keeps its sign


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_dequant_per_token_every_code_against_fp32_product(dtype):
    rng = np.random.default_rng(7)
    scales = np.concatenate([
        np.array([0.0, 1e-45, 1.2e-38, 2.0 ** -20, 0.125, 1.0, 7.0 / 3.0, 1e4, 9362.0, 3e37, 3.3e38],
                 np.float32),
        (rng.standard_normal(53) * np.exp(rng.uniform(-30, 30, 53))).astype(np.float32).__abs__()])
    S, M, N = scales.size, 2, 8
    codes = np.tile(np.arange(16, dtype=np.uint8), S).reshape(S, 16)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    got = oracle.dequant(packed, scales, M, N, dtype, "int4").reshape(S, 16)
    q = np.where(codes >= 8, codes.astype(np.int32) - 16, codes.astype(np.int32)).astype(np.float32)
    with np.errstate(over="ignore"):
        v32 = q * scales[:, None]                                     # IEEE fp32 product
    _same_bits(got.reshape(-1), _to_dt_bits(v32, dtype).reshape(-1), dtype)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_dequant_round_trip_error_bound(mode):
    # |value - y| is at most half the quantization step (the codes are nearest), plus the
    # output dtype's half unit in the last place
    w = synth.WORKLOADS["c2"]
    x, p1, p2 = synth.make_inputs(w, 0, 6)
    r = oracle.run(x, p1, p2, w.dtype, mode, clip_ratio=1.0, dst_type_max=0.0, ranges=False, want_y=True)
    M, N = w.M, w.N
    scale = r["scale"] if mode == "int4" else r["e8m0"]
    v = oracle.dt_to_float(oracle.dequant(r["packed"], scale, M, N, "bf16", mode), "bf16").reshape(6, -1)
    y = r["y"].reshape(6, -1).astype(np.float64)
    half_ulp = np.abs(v) * 2.0 ** -8
    if mode == "int4":
        step = r["scale"].astype(np.float64)[:, None]
        assert (np.abs(v - y) <= 0.5 * step * (1 + 1e-6) + half_ulp).all()
    else:
        # E2M1 spacing at |y|'s level: 0.5 below 2, 1 in [2, 4), 2 at and above 4 (x 2^(e-127));
        # values beyond 6 * 2^(e-127) saturate (V1 makes the group max land in [4, 8))
        e = np.repeat(r["e8m0"][:, : (M * N) // 32].astype(np.float64), 32, axis=1)
        unit = np.ldexp(1.0, (e - 127).astype(int))
        a = np.abs(y) / unit
        spacing = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0)) * unit
        sat = np.maximum(np.abs(y) - 6 * unit, 0)
        assert (np.abs(v - y) <= 0.5 * spacing * (1 + 1e-6) + sat + half_ulp).all()


# ---------------------------------------------------------------- MXFP4 consumer GEMM

def _mx_random(rows, H, rng, lo=100, hi=150):
    codes = rng.integers(0, 256, (rows, H // 2), dtype=np.uint8)
    e8 = rng.integers(lo, hi, (rows, 2 * (-(-H // 64))), dtype=np.uint8)
    return codes, e8


def _mx_decode(codes, e8, H):
    page = np.array([float(v) for v in keyed("e2m1_table.txt")["magnitudes"]])
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], H)
    val = page[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return np.ldexp(val, np.repeat(e8[:, : H // 32].astype(int) - 127, 32, axis=1))


def test_mx_gemm_against_numpy_matmul():
    rng = np.random.default_rng(3)
    T, O, H = 5, 7, 256
    a, ae = _mx_random(T, H, rng)
    w, we = _mx_random(O, H, rng)
    c, cabs = oracle.mx_gemm(a, ae, w, we, H)
    A, W = _mx_decode(a, ae, H), _mx_decode(w, we, H)
    assert np.allclose(c, A @ W.T, rtol=1e-12, atol=0)
    assert np.allclose(cabs, np.abs(A) @ np.abs(W).T, rtol=1e-12, atol=0)


def test_mx_gemm_one_hot_weights_select_activations():
    rng = np.random.default_rng(4)
    T, H = 6, 128
    a, ae = _mx_random(T, H, rng)
    O = 8
    cols = rng.integers(0, H, O)
    w = np.zeros((O, H // 2), np.uint8)
    for o, j in enumerate(cols):
        w[o, j // 2] |= np.uint8(0x2 << (4 * (j % 2)))     # E2M1 code 2 = 1.0
    we = np.full((O, 2 * (-(-H // 64))), 127, np.uint8)     # 2^0
    c, _ = oracle.mx_gemm(a, ae, w, we, H)
    A = _mx_decode(a, ae, H)
    assert np.array_equal(c, A[:, cols])


def test_mx_gemm_weight_scale_step_doubles_exactly():
    rng = np.random.default_rng(5)
    a, ae = _mx_random(4, 512, rng)
    w, we = _mx_random(3, 512, rng)
    c1, _ = oracle.mx_gemm(a, ae, w, we, 512)
    c2, _ = oracle.mx_gemm(a, ae, w, we + 1, 512)
    assert np.array_equal(c2, 2 * c1)


# ---------------------------------------------------------------- per-token 8-bit modes
# (the dequant_swiglu_quant page, section 3.4: dynamic per-row quantization with max_val
# 127 / 448 / 57344; section 6.1: round half to even)

FP8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def test_int8_rne_examples_and_symmetric_clamp_from_page():
    assert [oracle.int8_code(v) for v in (2.5, 3.5, -2.5, -3.5, 0.5, 1.5)] == [2, 4, -2, -4, 0, 2]
    assert oracle.int8_code(127.4) == 127 and oracle.int8_code(-127.4) == -127
    # clamp(round(.), -max_val, max_val): -127.6 rounds to -128, which the clamp takes to -127
    assert oracle.int8_code(-127.6) == -127 and oracle.int8_code(-1e9) == -127 and oracle.int8_code(1e9) == 127


def test_qmax_values_from_page():
    assert [oracle.qmax(m) for m in ("int4", "int8", "e4m3", "e5m2")] == [7.0, 127.0, 448.0, 57344.0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_value_table(fmt):
    vals = np.array([oracle.fp8_value(c, fmt) for c in range(128)])
    top = 0x7E if fmt == "e4m3" else 0x7B
    # the page's max_val is the largest finite value; the smallest subnormal and 1.0
    assert vals[top] == oracle.qmax(fmt)
    assert vals[1] == (2.0 ** -9 if fmt == "e4m3" else 2.0 ** -16)
    assert oracle.fp8_code(1.0, fmt) == (0x38 if fmt == "e4m3" else 0x3C)
    assert np.all(np.diff(vals[: top + 1]) > 0)  # values grow with the code
    # the same table as torch's float8 dtype decodes it
    codes = torch.arange(top + 1, dtype=torch.uint8).view(FP8_TORCH[fmt]).to(torch.float64).numpy()
    assert np.array_equal(codes, vals[: top + 1])
    assert oracle.fp8_value(0x80 | 0x38, fmt) == -vals[0x38]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_encoder_against_torch_conversion(fmt):
    """Every FP8 value, every midpoint between neighbours and one fp32 step either side of
    it, and random values over the whole range, both signs: the oracle's nearest-value
    search equals torch's float32 -> float8 conversion (round half to even) inside
    +-max_val; beyond it the oracle saturates."""
    top = 0x7E if fmt == "e4m3" else 0x7B
    v = np.array([oracle.fp8_value(c, fmt) for c in range(top + 1)])
    mids = 0.5 * (v[:-1] + v[1:])
    pts = [v, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
           np.nextafter(mids.astype(np.float32), np.float32(0))]
    rng = np.random.default_rng(5)
    pts.append(np.exp(rng.uniform(np.log(v[1] / 4), np.log(v[top]), 20000)))
    a = np.concatenate([np.asarray(p, dtype=np.float32) for p in pts])
    a = np.concatenate([a, -a, np.float32([0.0, -0.0])])
    a = a[np.abs(a) <= v[top]]
    want = torch.from_numpy(a).to(FP8_TORCH[fmt]).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_code(float(q), fmt) for q in a], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(a[i]), int(got[i]), int(want[i])) for i in bad[:5]]
    assert oracle.fp8_code(1e30, fmt) == top and oracle.fp8_code(-1e30, fmt) == 0x80 | top


@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
@pytest.mark.parametrize("clip", [1.0, 0.9])
def test_pertoken_8bit_invariants(mode, clip):
    """scale = amax / fl32(max_val / clip) within one fp32 rounding; the largest element
    maps to the largest level; every unclipped code dequantizes to within half a step of y
    (int8: scale/2; FP8: half the spacing of the neighbouring values at that magnitude);
    levels grow with y; the reachable interval holds the oracle's own level."""
    w = synth.WORKLOADS["c2"]
    x, p1, p2 = synth.make_inputs(w, 0, 6)
    r = oracle.run(x, p1, p2, w.dtype, mode, clip, want_y=True)
    S = x.shape[0]
    y = r["y"].reshape(S, -1).astype(np.float64)
    amax = np.abs(y).max(axis=1)
    s = r["scale"].astype(np.float64)
    d = float(np.float32(oracle.qmax(mode) / clip))
    assert np.all(np.abs(s * d - amax) <= amax * 2.0 ** -23)
    lvl = r["lvl"].astype(np.int64)
    codes = r["packed"].reshape(S, -1)
    top = 127 if mode == "int8" else (0x7E if mode == "e4m3" else 0x7B)
    assert np.abs(lvl).max() <= top
    if clip == 1.0:
        i = np.argmax(np.abs(y), axis=1)
        assert np.all(np.abs(lvl[np.arange(S), i]) == top)
    if mode == "int8":
        val = lvl.astype(np.float64)
        half = np.full_like(val, 0.5)
    else:
        table = np.array([oracle.fp8_value(c, mode) for c in range(top + 1)])
        mag = table[np.abs(lvl)]
        val = np.where(lvl < 0, -mag, mag)
        up = table[np.minimum(np.abs(lvl) + 1, top)] - mag
        dn = mag - table[np.maximum(np.abs(lvl) - 1, 0)]
        half = 0.5 * np.maximum(up, dn)
        assert np.array_equal(codes & 0x7F, np.abs(lvl))
    q = y / s[:, None]
    inside = np.abs(q) <= top * (1 - 1e-6) if mode == "int8" else np.abs(q) <= table[top] * (1 - 1e-6)
    err = np.abs(q - val)
    assert np.all(err[inside] <= half[inside] * (1 + 1e-5) + 1e-6)
    order = np.argsort(y, axis=1)
    assert np.all(np.diff(np.take_along_axis(lvl, order, axis=1), axis=1) >= 0)
    assert np.all(r["lo"] <= r["lvl"]) and np.all(r["lvl"] <= r["hi"])


def test_pertoken_8bit_zero_slice_and_sign_of_fp8_zero():
    x = np.zeros((1, 4, 8), np.uint16)
    for mode in ("int8", "e4m3", "e5m2"):
        r = oracle.run(x, bf16(np.eye(4)), bf16(np.eye(8)), "bf16", mode)
        assert (r["scale"] == 0).all() and (r["packed"] == 0).all()
        assert r["packed"].shape == (1, 32)
    # a tiny negative value keeps its sign in FP8 (code 0x80), not in INT8
    assert oracle.fp8_code(-1e-30, "e4m3") == 0x80 and oracle.int8_code(-1e-30) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
def test_dequant_8bit_every_code_against_fp32_product(mode, dtype):
    """Every code the quantizer can write (INT8 -127..127; every finite FP8 code, both signs)
    times fp32 scales from subnormal to overflowing: the oracle's values equal numpy's fp32
    product of the code's value (torch's float8 decoding for FP8) and the scale, cast to the
    dtype."""
    rng = np.random.default_rng(9)
    scales = np.concatenate([
        np.array([0.0, 1e-45, 1.2e-38, 2.0 ** -20, 0.125, 1.0, 7.0 / 3.0, 1e4, 3e37, 3.3e38], np.float32),
        np.abs(rng.standard_normal(20) * np.exp(rng.uniform(-30, 30, 20))).astype(np.float32)])
    if mode == "int8":
        codes = np.arange(-127, 128).astype(np.int8).view(np.uint8)
        q = codes.view(np.int8).astype(np.float32)
    else:
        top = 0x7E if mode == "e4m3" else 0x7B
        codes = np.concatenate([np.arange(top + 1), 0x80 | np.arange(top + 1)]).astype(np.uint8)
        q = torch.from_numpy(codes).view(FP8_TORCH[mode]).to(torch.float32).numpy()
    S, MN = scales.size, codes.size
    got = oracle.dequant(np.tile(codes, (S, 1)), scales, 1, MN, dtype, mode).reshape(S, MN)
    with np.errstate(over="ignore"):
        v32 = q[None, :] * scales[:, None]  # IEEE fp32 product
    _same_bits(got.reshape(-1), _to_dt_bits(v32, dtype).reshape(-1), dtype)


@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
def test_dequant_8bit_round_trip_within_half_a_step(mode):
    """dequantize(quantize(y)) is within half a code step of y (times the scale), plus half
    an output ulp, for every element (clip 1: nothing saturates)."""
    w = synth.WORKLOADS["c2i8"]
    x, p1, p2 = synth.make_inputs(w, 0, 4)
    r = oracle.run(x, p1, p2, w.dtype, mode, 1.0, want_y=True, ranges=False)
    v = oracle.dt_to_float(oracle.dequant(r["packed"], r["scale"], w.M, w.N, w.dtype, mode), w.dtype)
    y = r["y"].reshape(4, -1).astype(np.float64)
    v = v.reshape(4, -1)
    s = r["scale"].astype(np.float64)[:, None]
    if mode == "int8":
        step = np.full_like(y, 1.0)
    else:
        top = 0x7E if mode == "e4m3" else 0x7B
        table = np.array([oracle.fp8_value(c, mode) for c in range(top + 1)])
        q = np.minimum(np.abs(y / s), table[top])
        idx = np.clip(np.searchsorted(table, q), 1, top)
        step = table[idx] - table[idx - 1]
    bound = 0.5 * step * s * (1 + 1e-5) + np.abs(v) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(v - y) <= bound)


# ---------------------------------------------------------------- int4 consumer GEMM

def _int4_values(codes: np.ndarray) -> np.ndarray:
    lo, hi = (codes & 15).astype(np.int64), (codes >> 4).astype(np.int64)
    v = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    v[:, 0::2], v[:, 1::2] = np.where(lo >= 8, lo - 16, lo), np.where(hi >= 8, hi - 16, hi)
    return v


def test_int4_gemm_integer_part_against_numpy_matmul():
    """With unit scales C is fl32 of the exact integer dot product: numpy's int64 matmul of
    the decoded codes (|acc| < 2^24, so the fp32 value is exact)."""
    rng = np.random.default_rng(31)
    T, O, H = 19, 23, 384
    a = rng.integers(0, 256, (T, H // 2), dtype=np.uint8)
    w = rng.integers(0, 256, (O, H // 2), dtype=np.uint8)
    c = oracle.int4_gemm(a, np.ones(T, np.float32), w, np.ones(O, np.float32), H)
    ref = _int4_values(a) @ _int4_values(w).T
    assert np.array_equal(c.astype(np.int64), ref)
    # the extremes: every product -8 * -8 = 64
    full = np.full((1, H // 2), 0x88, np.uint8)
    assert oracle.int4_gemm(full, np.ones(1, np.float32), full, np.ones(1, np.float32), H)[0, 0] == 64 * H


def test_int4_gemm_scales_apply_as_one_fp32_factor():
    """Power-of-two scales are exact: C = acc * sa * sw exactly; with general scales C is
    fl32(acc * fl32(sa * sw)) (numpy's fp32 arithmetic on the same operands)."""
    rng = np.random.default_rng(32)
    T, O, H = 7, 9, 256
    a = rng.integers(0, 256, (T, H // 2), dtype=np.uint8)
    w = rng.integers(0, 256, (O, H // 2), dtype=np.uint8)
    acc = _int4_values(a) @ _int4_values(w).T
    sa = np.float32(2.0) ** rng.integers(-20, 20, T).astype(np.float32)
    sw = np.float32(2.0) ** rng.integers(-20, 20, O).astype(np.float32)
    c = oracle.int4_gemm(a, sa, w, sw, H)
    assert np.array_equal(c.astype(np.float64), acc * sa[:, None].astype(np.float64) * sw[None, :])
    sa = np.abs(rng.standard_normal(T)).astype(np.float32)
    sw = np.abs(rng.standard_normal(O)).astype(np.float32)
    c = oracle.int4_gemm(a, sa, w, sw, H)
    want = acc.astype(np.float32) * (sa[:, None] * sw[None, :])
    assert np.array_equal(c, want)


@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
def test_worked_8bit_examples(mode):
    """The hand-worked codes of tests/golden/worked_8bit.txt (scale exactly 1)."""
    k = keyed("worked_8bit.txt")
    M, N = (int(v) for v in k[f"{mode}_shape"])
    xv = np.array([float(v) for v in k[f"{mode}_x"]])
    x = bf16(xv).reshape(1, M, N)
    assert np.array_equal(oracle.dt_to_float(x, "bf16").reshape(-1), xv)  # exact in bf16
    r = oracle.run(x, bf16(np.eye(M)), bf16(np.eye(N)), "bf16", mode, 1.0)
    assert r["scale"][0] == 1.0
    if mode == "int8":
        want = np.array([int(v) for v in k["int8_codes"]]).astype(np.int8).view(np.uint8)
    else:
        want = np.array([int(v, 16) for v in k[f"{mode}_codes"]], np.uint8)
    assert r["packed"][0].tolist() == want.tolist()
