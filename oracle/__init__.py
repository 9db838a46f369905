"""ORACLE -- TEST INFRASTRUCTURE ONLY.

Python access to the scalar C oracle in ``fq_oracle.c`` (see its header for what it
computes and which passage of the operator's page each step follows).  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import this package; the GPU
library never does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfqoracle.so")

F16, BF16 = 1, 2
PER_TOKEN, PER_GROUP = 0, 1
# per-token code formats (one byte a code except int4)
QFMT = {"int32": 0, "int4": 0, "int8": 1, "e4m3": 2, "e5m2": 3}
PER_TOKEN_MODES = tuple(QFMT)
_DT = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}


class Params(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("M", ctypes.c_int64),
                ("N", ctypes.c_int64), ("two_sided", ctypes.c_int32), ("qfmt", ctypes.c_int32),
                ("clip_ratio", ctypes.c_double), ("dst_type_max", ctypes.c_double)]


_OUT_FIELDS = ["packed", "scale", "e8m0", "y", "t", "lvl", "lo", "hi", "zsign", "ns_tie",
               "alt_lvl", "alt_lo", "alt_hi", "alt_zsign", "g_lo", "g_hi", "g_alt", "scale_lo",
               "scale_hi"]


class Out(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _OUT_FIELDS]


_lib = None


def build(verbose: bool = False) -> str:
    """Compile fq_oracle.c with gcc: -O2, IEEE arithmetic (no fast-math, no contraction)."""
    src = os.path.join(_HERE, "fq_oracle.c")
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-frounding-math", src, "-o", LIB_PATH + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        p = ctypes.c_void_p
        L.fqo_run.argtypes = [ctypes.POINTER(Params), p, p, p, ctypes.c_int64, ctypes.POINTER(Out),
                              ctypes.c_int]
        L.fqo_run.restype = ctypes.c_int
        L.fqo_int4_code.argtypes = [ctypes.c_float]
        L.fqo_int4_code.restype = ctypes.c_int
        L.fqo_int8_code.argtypes = [ctypes.c_float]
        L.fqo_int8_code.restype = ctypes.c_int
        L.fqo_fp8_code.argtypes = [ctypes.c_double, ctypes.c_int]
        L.fqo_fp8_code.restype = ctypes.c_int
        L.fqo_fp8_value.argtypes = [ctypes.c_int, ctypes.c_int]
        L.fqo_fp8_value.restype = ctypes.c_double
        L.fqo_qmax.argtypes = [ctypes.c_int]
        L.fqo_qmax.restype = ctypes.c_double
        L.fqo_e2m1_code.argtypes = [ctypes.c_double]
        L.fqo_e2m1_code.restype = ctypes.c_int
        L.fqo_e2m1_value.argtypes = [ctypes.c_int]
        L.fqo_e2m1_value.restype = ctypes.c_double
        for fn in ("fqo_e8m0_v2_bits", "fqo_e8m0_v2_frexp"):
            getattr(L, fn).argtypes = [ctypes.c_float, ctypes.c_float]
            getattr(L, fn).restype = ctypes.c_int
        L.fqo_e8m0_v1.argtypes = [ctypes.c_float]
        L.fqo_e8m0_v1.restype = ctypes.c_int
        for fn in ("fqo_round_f32", "fqo_round_bf16", "fqo_round_f16"):
            getattr(L, fn).argtypes = [ctypes.c_double]
            getattr(L, fn).restype = ctypes.c_double
        L.fqo_dequant.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                  p, p, p]
        L.fqo_dequant.restype = ctypes.c_int
        L.fqo_dequant8.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   p, p, p]
        L.fqo_dequant8.restype = ctypes.c_int
        L.fqo_int4_gemm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, p, p, p, p, p]
        L.fqo_int4_gemm.restype = ctypes.c_int
        L.fqo_decode16.argtypes = [p, ctypes.c_int64, ctypes.c_int, p]
        L.fqo_decode16.restype = ctypes.c_int
        L.fqo_mx_gemm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, p, p, p, p, p, p]
        L.fqo_mx_gemm.restype = ctypes.c_int
        _lib = L
    return _lib


# ---- scalar encoders, exposed for the pins -------------------------------------------

def int4_code(q: float) -> int:
    return lib().fqo_int4_code(q)


def int8_code(q: float) -> int:
    return lib().fqo_int8_code(q)


def fp8_code(q: float, fmt: str) -> int:
    """FP8 code (sign bit 7) of q, fmt "e4m3" or "e5m2"."""
    return lib().fqo_fp8_code(q, QFMT[fmt])


def fp8_value(code: int, fmt: str) -> float:
    return lib().fqo_fp8_value(code, QFMT[fmt])


def qmax(mode: str) -> float:
    """max_val of a per-token mode: 7 (int4), 127, 448, 57344."""
    return lib().fqo_qmax(QFMT[mode])


def code_bytes(M: int, N: int, mode: str) -> int:
    """Bytes of codes per slice: M*N/2 for the 4-bit modes, M*N for the 8-bit ones."""
    return M * N if mode in ("int8", "e4m3", "e5m2") else M * N // 2


def e2m1_code(v: float) -> int:
    return lib().fqo_e2m1_code(v)


def e2m1_value(code: int) -> float:
    return lib().fqo_e2m1_value(code)


def e8m0_v1(amax: float) -> int:
    return lib().fqo_e8m0_v1(amax)


def e8m0_v2(amax: float, dmax: float, how: str = "bits") -> int:
    fn = lib().fqo_e8m0_v2_bits if how == "bits" else lib().fqo_e8m0_v2_frexp
    return fn(amax, dmax)


def decode16(bits, dtype: str) -> np.ndarray:
    """The oracle's own decoding of 16-bit dtype bits to float64 (fqo_decode16)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, np.float64)
    if lib().fqo_decode16(b.ctypes.data, b.size, _DT[dtype], out.ctypes.data) != 0:
        raise ValueError("fqo_decode16 rejected the dtype")
    return out


def round_f32(v: float) -> float:
    return lib().fqo_round_f32(v)


def round_dt(v: float, dtype: str) -> float:
    return (lib().fqo_round_bf16 if _DT[dtype] == BF16 else lib().fqo_round_f16)(v)


# ---- the batch entry ---------------------------------------------------------------

def out_shapes(M: int, N: int, mode: str):
    """Per-slice byte/element counts of the packed outputs."""
    MN = M * N
    G = -(-MN // 32)
    GS = 2 * (-(-MN // 64))
    return MN, G, GS


def run(x: np.ndarray, p1: np.ndarray, p2: np.ndarray | None, dtype: str, mode: str,
        clip_ratio: float = 1.0, dst_type_max: float = 0.0, ranges: bool = True,
        want_y: bool = False, want_t: bool = False, nthreads: int = 1) -> dict:
    """Oracle outputs for x [S, M, N] (uint16 dtype bits) and P1 [M, M], P2 [N, N] or None.

    mode: "int32" / "int4" (per-token int4), "int8" / "e4m3" / "e5m2" (per-token 8-bit
    codes) or "fp4" (per-group-32 E2M1).  Returns a dict of numpy arrays; "packed" is
    [S, M*N/2] bytes (low nibble first) for the 4-bit modes, [S, M*N] for the 8-bit ones.  With ranges=True the
    per-element reachable-level data used by the comparator is included.
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    S, M, N = x.shape
    p1 = np.ascontiguousarray(p1, dtype=np.uint16)
    assert p1.shape == (M, M)
    if p2 is not None:
        p2 = np.ascontiguousarray(p2, dtype=np.uint16)
        assert p2.shape == (N, N)
    per_token = mode in PER_TOKEN_MODES
    MN, G, GS = out_shapes(M, N, mode)
    prm = Params(_DT[dtype], PER_TOKEN if per_token else PER_GROUP, M, N, 1 if p2 is not None else 0,
                 QFMT.get(mode, 0), float(clip_ratio), float(dst_type_max))
    res: dict = {}

    def alloc(name, shape, dt):
        a = np.zeros(shape, dtype=dt)
        res[name] = a
        return a.ctypes.data

    o = Out()
    o.packed = alloc("packed", (S, code_bytes(M, N, mode)), np.uint8)
    if per_token:
        o.scale = alloc("scale", (S,), np.float32)
    else:
        o.e8m0 = alloc("e8m0", (S, GS), np.uint8)
    if want_y:
        o.y = alloc("y", (S, M, N), np.float32)
    if want_t:
        o.t = alloc("t", (S, M, N), np.uint16)
    o.lvl = alloc("lvl", (S, MN), np.int8)
    o.ns_tie = alloc("ns_tie", (S, MN), np.uint8)
    if ranges:
        o.lo = alloc("lo", (S, MN), np.int8)
        o.hi = alloc("hi", (S, MN), np.int8)
        o.zsign = alloc("zsign", (S, MN), np.uint8)
        if per_token:
            o.scale_lo = alloc("scale_lo", (S,), np.float32)
            o.scale_hi = alloc("scale_hi", (S,), np.float32)
        else:
            o.alt_lvl = alloc("alt_lvl", (S, MN), np.int8)
            o.alt_lo = alloc("alt_lo", (S, MN), np.int8)
            o.alt_hi = alloc("alt_hi", (S, MN), np.int8)
            o.alt_zsign = alloc("alt_zsign", (S, MN), np.uint8)
            o.g_lo = alloc("g_lo", (S, G), np.uint8)
            o.g_hi = alloc("g_hi", (S, G), np.uint8)
            o.g_alt = alloc("g_alt", (S, G), np.uint8)
    rc = lib().fqo_run(ctypes.byref(prm), x.ctypes.data, p1.ctypes.data,
                       p2.ctypes.data if p2 is not None else None, S, ctypes.byref(o), int(nthreads))
    if rc != 0:
        raise ValueError(f"fqo_run failed ({rc})")
    res["mode"] = mode
    res["M"], res["N"], res["S"] = M, N, S
    return res


def run_codes_only(x, p1, p2, dtype, mode, clip_ratio=1.0, dst_type_max=0.0, nthreads=1):
    """Codes and scales only (what the operator outputs), for timing the oracle."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    S, M, N = x.shape
    per_token = mode in PER_TOKEN_MODES
    MN, G, GS = out_shapes(M, N, mode)
    prm = Params(_DT[dtype], PER_TOKEN if per_token else PER_GROUP, M, N, 1 if p2 is not None else 0,
                 QFMT.get(mode, 0), float(clip_ratio), float(dst_type_max))
    packed = np.zeros((S, code_bytes(M, N, mode)), np.uint8)
    sc = np.zeros((S,), np.float32) if per_token else np.zeros((S, GS), np.uint8)
    o = Out()
    o.packed = packed.ctypes.data
    if per_token:
        o.scale = sc.ctypes.data
    else:
        o.e8m0 = sc.ctypes.data
    p1 = np.ascontiguousarray(p1, dtype=np.uint16)
    p2c = np.ascontiguousarray(p2, dtype=np.uint16) if p2 is not None else None
    rc = lib().fqo_run(ctypes.byref(prm), x.ctypes.data, p1.ctypes.data,
                       p2c.ctypes.data if p2c is not None else None, S, ctypes.byref(o), int(nthreads))
    if rc != 0:
        raise ValueError(f"fqo_run failed ({rc})")
    return packed, sc


def dequant(packed: np.ndarray, scale: np.ndarray, M: int, N: int, dtype: str, mode: str) -> np.ndarray:
    """Values of the codes (uint16 bits of the output dtype, [S, M, N]): q * scale per
    token, E2M1 value * 2^(e8m0 - 127) per group (see fqo_dequant in fq_oracle.c).

    packed: [S, M*N/2] bytes as the quantizer writes them (low nibble first), [S, M*N] for
    the 8-bit codes; scale: fp32 [S] per token ("int32" / "int4" / "int8" / "e4m3" / "e5m2"),
    e8m0 bytes [S, 2*ceil(M*N/64)] per group ("fp4")."""
    S = packed.shape[0]
    if mode in ("int8", "e4m3", "e5m2"):  # one byte a code, fp32 scales [S]
        codes = np.ascontiguousarray(packed, dtype=np.uint8).reshape(S, M * N)
        scale = np.ascontiguousarray(scale, dtype=np.float32).reshape(S)
        out = np.empty((S, M, N), np.uint16)
        st = lib().fqo_dequant8(_DT[dtype], QFMT[mode], S, M, N, codes.ctypes.data, scale.ctypes.data,
                                out.ctypes.data)
        if st != 0:
            raise ValueError(f"fqo_dequant8 rejected the arguments ({st})")
        return out
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(S, M * N // 2)
    if mode in ("int32", "int4"):
        scale = np.ascontiguousarray(scale, dtype=np.float32).reshape(S)
        m = PER_TOKEN
    elif mode == "fp4":
        scale = np.ascontiguousarray(scale, dtype=np.uint8).reshape(S, -1)
        m = PER_GROUP
    else:
        raise ValueError(f"unknown mode {mode!r}")
    out = np.empty((S, M, N), np.uint16)
    st = lib().fqo_dequant(_DT[dtype], m, S, M, N, packed.ctypes.data, scale.ctypes.data, out.ctypes.data)
    if st != 0:
        raise ValueError(f"fqo_dequant rejected the arguments ({st})")
    return out


def dt_to_float(bits: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of 16-bit dtype bits (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if _DT[dtype] == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def mx_gemm(a: np.ndarray, a_e8: np.ndarray, w: np.ndarray, w_e8: np.ndarray, H: int):
    """C [T, O] = dequant(a) . dequant(w)^T in double, and sum|terms| [T, O] (see
    fqo_mx_gemm).  a [T, H/2] and w [O, H/2] are E2M1 code bytes (low nibble first); a_e8
    and w_e8 the e8m0 bytes [rows, 2*ceil(H/64)]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    a_e8 = np.ascontiguousarray(a_e8, dtype=np.uint8).reshape(a.shape[0], -1)
    w_e8 = np.ascontiguousarray(w_e8, dtype=np.uint8).reshape(w.shape[0], -1)
    T, O = a.shape[0], w.shape[0]
    c = np.empty((T, O), np.float64)
    cabs = np.empty((T, O), np.float64)
    st = lib().fqo_mx_gemm(T, O, H, a.ctypes.data, a_e8.ctypes.data, w.ctypes.data, w_e8.ctypes.data,
                           c.ctypes.data, cabs.ctypes.data)
    if st != 0:
        raise ValueError(f"fqo_mx_gemm rejected the arguments ({st})")
    return c, cabs


def int4_gemm(a: np.ndarray, sa: np.ndarray, w: np.ndarray, sw: np.ndarray, H: int) -> np.ndarray:
    """C [T, O] fp32 = fl32(fl32(acc) * fl32(sa[t] * sw[o])), acc the exact int4 dot product
    (see fqo_int4_gemm).  a [T, H/2], w [O, H/2] int4 code bytes (low nibble first); sa [T],
    sw [O] fp32."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    T, O = a.shape[0], w.shape[0]
    c = np.empty((T, O), np.float32)
    st = lib().fqo_int4_gemm(T, O, H, a.ctypes.data, sa.ctypes.data, w.ctypes.data, sw.ctypes.data, c.ctypes.data)
    if st != 0:
        raise ValueError(f"fqo_int4_gemm rejected the arguments ({st})")
    return c
