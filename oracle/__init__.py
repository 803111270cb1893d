"""The oracle: plain double-precision CPU implementation (``tqref.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
CPU-baseline leg of ``bench.py``; never by the product package. It shares no
code with the GPU path. This module only builds and marshals; all arithmetic
of the method lives in ``tqref.c`` (and in ``stats.py`` for the statistics the
pages report).

Parity pins for every oracle function are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tqref.c")
# TQ_SANITIZE=1: a separate build with AddressSanitizer and UBSan
_SAN = os.environ.get("TQ_SANITIZE") == "1"
_LIB = (os.path.join(os.path.dirname(_HERE), "_build", "san", "liboracle_san.so") if _SAN
        else os.path.join(_HERE, "liboracle.so"))
_lib = None

CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-std=gnu11", "-Wall"] + (["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]
                                    if _SAN else [])


def build(force: bool = False) -> str:
    """Compile ``tqref.c`` into ``liboracle.so`` (gcc, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Quantizer(C.Structure):
    _fields_ = [("d", C.c_int), ("bits", C.c_int), ("m", C.c_int),
                ("cent", C.POINTER(C.c_float)), ("bnd", C.POINTER(C.c_float)),
                ("diag", C.POINTER(C.c_uint32)), ("S", C.POINTER(C.c_uint16))]


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(_LIB)
        dp, fp = C.POINTER(C.c_double), C.POINTER(C.c_float)
        u32p, u16p = C.POINTER(C.c_uint32), C.POINTER(C.c_uint16)
        qp = C.POINTER(_Quantizer)
        L.tqref_codebook_law.argtypes = [C.c_int, C.c_int, C.c_int, dp, fp, fp, dp, dp]
        L.tqref_codebook_law.restype = C.c_int
        L.tqref_sphere_moments.argtypes = [C.c_int, C.c_double, C.c_double, dp]
        L.tqref_sphere_moments.restype = None
        L.tqref_quantize.argtypes = [qp, dp, C.c_int64, u32p, u32p, u16p, u16p, dp, dp]
        L.tqref_quantize.restype = None
        L.tqref_sketch.argtypes = [qp, dp, u32p, C.c_int64, u32p, u16p, dp]
        L.tqref_sketch.restype = None
        L.tqref_scores.argtypes = [qp, u32p, u32p, u16p, u16p, C.c_int64, dp, C.c_int64, dp]
        L.tqref_scores.restype = None
        L.tqref_dequantize.argtypes = [qp, u32p, u32p, u16p, u16p, C.c_int64, C.c_int, dp]
        L.tqref_dequantize.restype = None
        L.tqref_decode_attn.argtypes = [qp, qp, u32p, u32p, u16p, u16p, u32p, u16p,
                                        C.c_int64, C.c_int64, C.c_int, dp, C.c_double, dp]
        L.tqref_decode_attn.restype = None
        L.tqref_half_to_double.argtypes = [C.c_uint16]
        L.tqref_half_to_double.restype = C.c_double
        L.tqref_double_to_half.argtypes = [C.c_double]
        L.tqref_double_to_half.restype = C.c_uint16
        L.tqref_max_threads.restype = C.c_int
        L.tqref_set_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(C.POINTER(ct))


def max_threads() -> int:
    return lib().tqref_max_threads()


def set_threads(n: int) -> None:
    lib().tqref_set_threads(int(n))


# ------------------------------------------------------------------ codebook

@dataclass
class Codebook:
    d: int
    bits: int
    c_exact: np.ndarray      # float64 [L]
    centroids: np.ndarray    # float32 [L], fp16-representable
    boundaries: np.ndarray   # float32 [L-1]
    dist_exact: float
    dist_stored: float
    iters: int


LAW_GAUSSIAN, LAW_SPHERE = 0, 1


def codebook(d: int, bits: int, law: int = LAW_GAUSSIAN) -> Codebook:
    """Lloyd-Max codebook for N(0, 1/d) (law 0) or the exact coordinate law of
    a random unit vector in R^d (law 1, a Beta law of Y^2)."""
    L = 1 << bits
    ce = np.zeros(L, np.float64)
    cs = np.zeros(L, np.float32)
    ts = np.zeros(max(L - 1, 1), np.float32)
    de = C.c_double()
    ds = C.c_double()
    it = lib().tqref_codebook_law(d, bits, law, _p(ce, C.c_double), _p(cs, C.c_float), _p(ts, C.c_float),
                                  C.byref(de), C.byref(ds))
    if it < 0:
        raise RuntimeError(f"oracle codebook failed (d={d}, bits={bits}, law={law}): {it}")
    return Codebook(d, bits, ce, cs, ts[:L - 1], de.value, ds.value, it)


def sphere_moments(d: int, a: float, b: float) -> np.ndarray:
    """(mass, first, second moment) of the exact coordinate law over (a, b]."""
    m = np.zeros(3, np.float64)
    lib().tqref_sphere_moments(d, a, b, _p(m, C.c_double))
    return m


def half_to_double(h: int) -> float:
    return lib().tqref_half_to_double(int(h))


def double_to_half(x: float) -> int:
    return int(lib().tqref_double_to_half(float(x)))


# ------------------------------------------------------------------ quantizer

class Quantizer:
    """Host-side quantizer state: (d, bits, m), stored codebook, D, S."""

    def __init__(self, d: int, bits: int, m: int, diag: np.ndarray, S16: np.ndarray | None,
                 cb: Codebook | None = None):
        self.d, self.bits, self.m = d, bits, m
        self.cb = cb if cb is not None else codebook(d, bits)
        self.cent = np.ascontiguousarray(self.cb.centroids, np.float32)
        self.bnd = np.ascontiguousarray(np.concatenate([self.cb.boundaries, [0.0]]), np.float32)
        self.diag = np.ascontiguousarray(diag, np.uint32)
        if m > 0:
            assert S16 is not None and S16.shape == (m, d)
            self.S = np.ascontiguousarray(np.asarray(S16, np.float16).view(np.uint16))
        else:
            self.S = np.zeros(1, np.uint16)
        self._s = _Quantizer(d, bits, m, _p(self.cent, C.c_float), _p(self.bnd, C.c_float),
                             _p(self.diag, C.c_uint32), _p(self.S, C.c_uint16))

    @property
    def words(self) -> int:
        return (self.d + 31) // 32

    @property
    def sign_words(self) -> int:
        return (self.m + 31) // 32

    def S_f64(self) -> np.ndarray:
        return self.S.view(np.float16).astype(np.float64).reshape(self.m, self.d)


@dataclass
class Packed:
    codes: np.ndarray    # uint32 [n, bits * words] (group-major bit stream)
    signs: np.ndarray    # uint32 [n, sign_words] (empty when m = 0)
    norm: np.ndarray     # uint16 [n] fp16 bits
    rnorm: np.ndarray    # uint16 [n] fp16 bits (zeros when m = 0)

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    def take(self, idx) -> "Packed":
        return Packed(self.codes[idx], self.signs[idx] if self.signs.size else self.signs,
                      self.norm[idx], self.rnorm[idx])


def empty_packed(Q: Quantizer, n: int) -> Packed:
    return Packed(np.zeros((n, Q.bits * Q.words), np.uint32),
                  np.zeros((n, max(Q.sign_words, 0)), np.uint32),
                  np.zeros(n, np.uint16), np.zeros(n, np.uint16))


def quantize(Q: Quantizer, x: np.ndarray, want_y: bool = False, want_u: bool = False):
    """Quantize x [n, d] (exact values; fp16/fp32 inputs are widened exactly)."""
    x = np.ascontiguousarray(np.asarray(x, np.float64).reshape(-1, Q.d))
    n = x.shape[0]
    P = empty_packed(Q, n)
    y = np.zeros((n, Q.d), np.float64) if want_y else None
    u = np.zeros((n, max(Q.m, 1)), np.float64) if (want_u and Q.m) else None
    sg = P.signs if Q.m else np.zeros(1, np.uint32)
    lib().tqref_quantize(C.byref(Q._s), _p(x, C.c_double), n, _p(P.codes, C.c_uint32),
                         _p(sg, C.c_uint32), _p(P.norm, C.c_uint16), _p(P.rnorm, C.c_uint16),
                         _p(y, C.c_double) if y is not None else None,
                         _p(u, C.c_double) if u is not None else None)
    out = [P]
    if want_y:
        out.append(y)
    if want_u:
        out.append(u)
    return out[0] if len(out) == 1 else tuple(out)


def sketch(Q: Quantizer, y: np.ndarray, codes: np.ndarray, want_u: bool = False):
    """The QJL stage on given codes: (signs uint32 [n, m/32], rnorm fp16 bits [n]
    and, with want_u, u = S r [n, m]) for rotated unit vectors y [n, d] whose
    packed codes are ``codes`` -- what ``quantize`` writes when those are its
    own codes. Keys only (m > 0)."""
    assert Q.m > 0
    y = np.ascontiguousarray(np.asarray(y, np.float64).reshape(-1, Q.d))
    n = y.shape[0]
    codes = np.ascontiguousarray(np.asarray(codes, np.uint32).reshape(n, Q.bits * Q.words))
    signs = np.zeros((n, Q.sign_words), np.uint32)
    rnorm = np.zeros(n, np.uint16)
    u = np.zeros((n, Q.m), np.float64) if want_u else None
    lib().tqref_sketch(C.byref(Q._s), _p(y, C.c_double), _p(codes, C.c_uint32), n,
                       _p(signs, C.c_uint32), _p(rnorm, C.c_uint16),
                       _p(u, C.c_double) if u is not None else None)
    return (signs, rnorm, u) if want_u else (signs, rnorm)


def _packed_args(Q: Quantizer, P: Packed):
    codes = np.ascontiguousarray(P.codes, np.uint32)
    signs = np.ascontiguousarray(P.signs, np.uint32) if Q.m else np.zeros(1, np.uint32)
    norm = np.ascontiguousarray(P.norm, np.uint16)
    rnorm = np.ascontiguousarray(P.rnorm, np.uint16)
    return codes, signs, norm, rnorm


def scores(Q: Quantizer, P: Packed, q: np.ndarray) -> np.ndarray:
    """Estimated inner products [n_q, n_keys] in double."""
    q = np.ascontiguousarray(np.asarray(q, np.float64).reshape(-1, Q.d))
    codes, signs, norm, rnorm = _packed_args(Q, P)
    out = np.zeros((q.shape[0], P.n), np.float64)
    lib().tqref_scores(C.byref(Q._s), _p(codes, C.c_uint32), _p(signs, C.c_uint32),
                       _p(norm, C.c_uint16), _p(rnorm, C.c_uint16), P.n, _p(q, C.c_double),
                       q.shape[0], _p(out, C.c_double))
    return out


def dequantize(Q: Quantizer, P: Packed, include_qjl: bool = True) -> np.ndarray:
    codes, signs, norm, rnorm = _packed_args(Q, P)
    out = np.zeros((P.n, Q.d), np.float64)
    lib().tqref_dequantize(C.byref(Q._s), _p(codes, C.c_uint32), _p(signs, C.c_uint32),
                           _p(norm, C.c_uint16), _p(rnorm, C.c_uint16), P.n,
                           1 if include_qjl else 0, _p(out, C.c_double))
    return out


def decode_attn(QK: Quantizer, QV: Quantizer, PK: Packed, PV: Packed, n_streams: int, T: int,
                G: int, q: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Attention output [n_streams, G, d] over streams of T packed tokens."""
    assert PK.n == n_streams * T and PV.n == n_streams * T
    q = np.ascontiguousarray(np.asarray(q, np.float64).reshape(n_streams * G, QK.d))
    if scale is None:
        scale = 1.0 / np.sqrt(QK.d)
    kc, ks, kn, kr = _packed_args(QK, PK)
    vc, _, vn, _ = _packed_args(QV, PV)
    out = np.zeros((n_streams * G, QV.d), np.float64)
    lib().tqref_decode_attn(C.byref(QK._s), C.byref(QV._s), _p(kc, C.c_uint32),
                            _p(ks, C.c_uint32), _p(kn, C.c_uint16), _p(kr, C.c_uint16),
                            _p(vc, C.c_uint32), _p(vn, C.c_uint16), n_streams, T, G,
                            _p(q, C.c_double), float(scale), _p(out, C.c_double))
    return out.reshape(n_streams, G, QV.d)


def _group_bit(n: int, bits: int, i: np.ndarray, p: int) -> np.ndarray:
    """Stream bit of code bit p of coordinate i in the group-major layout."""
    G = n // 8 if n >= 8 else 1
    return 8 * bits * (i % G) + bits * (i // G) + p


def unpack_codes(Q: Quantizer, codes: np.ndarray) -> np.ndarray:
    """Code indices [n, d] from the group-major packed layout (test helper)."""
    codes = np.asarray(codes, np.uint32).reshape(-1, Q.bits * Q.words)
    i = np.arange(Q.d)
    out = np.zeros((codes.shape[0], Q.d), np.int64)
    for p in range(Q.bits):
        b = _group_bit(Q.d, Q.bits, i, p)
        bits = (codes[:, b // 32] >> (b % 32).astype(np.uint32)) & 1
        out |= bits.astype(np.int64) << p
    return out


def unpack_signs(Q: Quantizer, signs: np.ndarray) -> np.ndarray:
    """Sign bits [n, m] (1 = projection >= 0) from the group-major layout."""
    signs = np.asarray(signs, np.uint32).reshape(-1, Q.sign_words)
    j = np.arange(Q.m)
    b = _group_bit(Q.m, 1, j, 0)
    return ((signs[:, b // 32] >> (b % 32).astype(np.uint32)) & 1).astype(np.int64)
