"""The comparator accepts what the tolerance rule allows and rejects the rest (CPU only)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import compare, unpack_nibbles


def _repack(codes):
    codes = codes.astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _pertoken(K=8):
    w = synth.WORKLOADS["c2"]
    x, p1, p2 = synth.make_inputs(w, 0, K)
    return oracle.run(x, p1, p2, w.dtype, w.mode, w.clip_ratio)


def _pergroup():
    w = synth.WORKLOADS["c3"]
    x, p1, p2 = synth.make_inputs(w, 0, 8)
    return oracle.run(x, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max)


def test_identical_passes():
    r = _pertoken()
    assert compare(r, r["packed"], r["scale"])["ok"]
    g = _pergroup()
    assert compare(g, g["packed"], g["e8m0"])["ok"]


def test_unflagged_code_change_fails():
    r = _pertoken()
    codes = unpack_nibbles(r["packed"], r["M"] * r["N"])
    s, f = np.argwhere(r["lo"] == r["hi"])[0]
    codes[s, f] = (codes[s, f] + 1) & 0xF
    assert not compare(r, _repack(codes), r["scale"])["ok"]


def test_flagged_one_step_passes_two_steps_fail():
    r = _pertoken()
    codes = unpack_nibbles(r["packed"], r["M"] * r["N"])
    idx = np.argwhere((r["hi"] > r["lvl"]))
    assert len(idx) > 0
    s, f = idx[0]
    c1 = codes.copy()
    c1[s, f] = (c1[s, f] + 1) & 0xF
    rep = compare(r, _repack(c1), r["scale"])
    assert rep["ok"] and rep["mismatch"] == 1
    c2 = codes.copy()
    c2[s, f] = (c2[s, f] + 2) & 0xF
    assert not compare(r, _repack(c2), r["scale"])["ok"]


def test_mismatch_cap():
    r = _pertoken()
    codes = unpack_nibbles(r["packed"], r["M"] * r["N"])
    idx = np.argwhere((r["hi"] > r["lvl"]))
    cap = int(np.ceil(1e-4 * codes.size))
    if len(idx) <= cap:
        # force the situation on a copy: mark more elements reachable
        r = dict(r)
        r["hi"] = np.minimum(r["lvl"] + 1, 7).astype(np.int8)
        idx = np.argwhere(r["hi"] > r["lvl"])
    c = codes.copy()
    for s, f in idx[: cap + 1]:
        c[s, f] = (c[s, f] + 1) & 0xF
    rep = compare(r, _repack(c), r["scale"])
    assert not rep["ok"] and rep["mismatch"] == cap + 1


def test_scale_tolerance():
    r = _pertoken(64)
    ok = r["scale"] * np.float32(1 + 5e-6)
    assert compare(r, r["packed"], ok)["ok"]
    # beyond 1e-5 and beyond the reachable interval: rejected
    lo, hi = r["scale_lo"].astype(np.float64), r["scale_hi"].astype(np.float64)
    out = np.maximum(hi * (1 + 1e-6), r["scale"] * (1 + 2e-5)).astype(np.float32)
    rep = compare(r, r["packed"], out)
    assert not rep["ok"] and rep.get("scale_fail") == r["S"]
    # beyond 1e-5 but inside the reachable interval of a slice whose intermediate rounding
    # is ambiguous: accepted and counted
    sc = r["scale"].astype(np.float64)
    dev = np.maximum(hi - sc, sc - lo) / sc
    s = int(np.argmax(dev))
    assert dev[s] > 1.5e-5
    g = r["scale"].copy()
    g[s] = np.float32(hi[s] if hi[s] - sc[s] >= sc[s] - lo[s] else lo[s])
    rep = compare(r, r["packed"], g)
    assert rep["ok"] and rep["scale_ties"] == 1


def test_scale_interval_is_tight_without_intermediate_ties():
    """With P2 = I the intermediate is exact: the reachable scale interval is then set by
    the fp32 summation bound of the second product alone and stays within 1e-5."""
    w = synth.WORKLOADS["c2"]
    x, p1, _ = synth.make_inputs(w, 0, 8)
    eye = synth.round_to(np.eye(w.N), "bf16")
    r = oracle.run(x, p1, eye, w.dtype, w.mode, w.clip_ratio)
    width = (r["scale_hi"].astype(np.float64) - r["scale_lo"]) / r["scale"]
    assert width.max() < 2e-5


def test_e8m0_change_and_pad():
    g = _pergroup()
    e = g["e8m0"].copy()
    e[0, 0] += 1
    assert not compare(g, g["packed"], e)["ok"]
    # a group whose scale is reachable both ways accepts the alternative with its codes
    r = dict(g)
    r["g_alt"] = r["g_alt"].copy()
    r["g_hi"] = r["g_hi"].copy()
    r["g_alt"][0, 0] = r["e8m0"][0, 0] + 1
    r["g_hi"][0, 0] = r["e8m0"][0, 0] + 1
    r["alt_lvl"] = r["alt_lvl"].copy()
    r["alt_lo"] = r["alt_lo"].copy()
    r["alt_hi"] = r["alt_hi"].copy()
    r["alt_lvl"][0, :32] = r["lvl"][0, :32]
    r["alt_lo"][0, :32] = r["lvl"][0, :32]
    r["alt_hi"][0, :32] = r["lvl"][0, :32]
    e = g["e8m0"].copy()
    e[0, 0] += 1
    rep = compare(r, g["packed"], e)
    assert rep["ok"] and rep["alt_groups"] == 1


def test_pad_slot_must_be_zero():
    rng = np.random.default_rng(0)
    x = synth.round_to(rng.standard_normal((2, 3, 32)), "bf16")
    eye3 = synth.round_to(np.eye(3), "bf16")
    eye32 = synth.round_to(np.eye(32), "bf16")
    g = oracle.run(x, eye3, eye32, "bf16", "fp4")
    assert compare(g, g["packed"], g["e8m0"])["ok"]
    e = g["e8m0"].copy()
    e[1, 3] = 1
    assert not compare(g, g["packed"], e)["ok"]


def test_zero_sign_rule():
    rng = np.random.default_rng(1)
    x = synth.round_to(rng.standard_normal((1, 2, 32)) * 4, "bf16")
    x[0, 0, 5] = 0x0000  # an exact zero in the input: y = 0 exactly, either sign allowed
    x[0, 0, 7] = synth.round_to(np.array([-1e-3]), "bf16")[0]  # rounds to -0, sign fixed
    eye2 = synth.round_to(np.eye(2), "bf16")
    eye32 = synth.round_to(np.eye(32), "bf16")
    g = oracle.run(x, eye2, eye32, "bf16", "fp4")
    codes = unpack_nibbles(g["packed"], 64)
    assert codes[0, 7] == 0x8
    c = codes.copy()
    c[0, 5] ^= 0x8
    assert compare(g, _repack(c), g["e8m0"])["ok"]
    c = codes.copy()
    c[0, 7] ^= 0x8
    assert not compare(g, _repack(c), g["e8m0"])["ok"]


def _byte_mode(mode, K=6):
    w = synth.WORKLOADS["c2i8"]
    x, p1, p2 = synth.make_inputs(w, 0, K)
    return oracle.run(x, p1, p2, w.dtype, mode, 1.0)


def _level_to_code(level, mode):
    level = np.asarray(level, np.int16)
    if mode == "int8":
        return level.astype(np.int8).view(np.uint8)
    return np.where(level < 0, 0x80 | (-level), level).astype(np.uint8)


@pytest.mark.parametrize("mode", ["int8", "e4m3", "e5m2"])
def test_byte_codes_rule(mode):
    """8-bit codes: identical passes; a change of an element whose reachable range is one
    level fails; a change to the far end of the widest reachable range passes (two or more
    levels away where the range allows it); a change outside the range fails; a changed
    scale fails."""
    r = _byte_mode(mode)
    assert compare(r, r["packed"], r["scale"])["ok"]
    one = np.argwhere(r["lo"] == r["hi"])
    s, f = one[len(one) // 2]
    g = r["packed"].copy()
    g[s, f] = _level_to_code(int(r["lvl"][s, f]) + 1, mode)
    assert not compare(r, g, r["scale"])["ok"]
    span = r["hi"].astype(int) - r["lo"].astype(int)
    wide = np.argwhere(span == span.max())
    assert span.max() >= 1
    s, f = wide[0]
    lv = int(r["lvl"][s, f])
    # the end of the reachable range farthest from the oracle's level
    target = int(r["lo"][s, f]) if lv - int(r["lo"][s, f]) >= int(r["hi"][s, f]) - lv else int(r["hi"][s, f])
    g = r["packed"].copy()
    g[s, f] = _level_to_code(target, mode)
    rep = compare(r, g, r["scale"])
    assert rep["ok"] and rep["mismatch"] == 1, rep["errors"]
    g[s, f] = _level_to_code(int(r["hi"][s, f]) + 1, mode)
    assert not compare(r, g, r["scale"])["ok"]
    assert not compare(r, r["packed"], r["scale"] * np.float32(1.001))["ok"]


def test_out_of_window_cap():
    """Differences at elements the oracle flags only through the fp32 error bound (not a tie
    within 1e-6) are allowed up to ceil(1e-5 * elements) for the 4-bit codes; one more fails."""
    r = _pertoken(8)
    codes = unpack_nibbles(r["packed"], r["M"] * r["N"])
    idx = np.argwhere((r["hi"] > r["lvl"]) & (r["ns_tie"] == 0))
    cap = int(np.ceil(1e-5 * codes.size))
    assert len(idx) > cap
    for n, want_ok in ((cap, True), (cap + 1, False)):
        c = codes.copy()
        for s, f in idx[:n]:
            c[s, f] = (c[s, f] + 1) & 0xF
        rep = compare(r, _repack(c), r["scale"])
        assert rep["ok"] == want_ok and rep["mismatch_out_of_window"] == n and rep["out_of_window_cap"] == cap


def test_scale_ties_cap():
    """Scales outside 1e-5 but inside the reachable interval are allowed on at most
    max(1, ceil(0.02 * slices)) slices."""
    r = _pertoken(64)
    sc = r["scale"].astype(np.float64)
    lo, hi = r["scale_lo"].astype(np.float64), r["scale_hi"].astype(np.float64)
    dev = np.maximum(hi - sc, sc - lo) / sc
    wide = np.nonzero(dev > 1.5e-5)[0]
    cap = max(1, int(np.ceil(0.02 * 64)))
    if len(wide) <= cap:
        # widen more slices' intervals on a copy, as an ambiguous intermediate would
        r = dict(r)
        r["scale_hi"] = (r["scale"] * np.float32(1 + 1e-3)).astype(np.float32)
        hi = r["scale_hi"].astype(np.float64)
        wide = np.arange(64)
    for n, want_ok in ((cap, True), (cap + 1, False)):
        g = r["scale"].copy()
        for s in wide[:n]:
            g[s] = np.float32(hi[s] if hi[s] - sc[s] >= sc[s] - lo[s] else lo[s])
        rep = compare(r, r["packed"], g)
        assert rep["ok"] == want_ok and rep["scale_ties"] == n
