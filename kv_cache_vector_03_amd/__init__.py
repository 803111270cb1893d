"""Python binding of libtq.so (C ABI in include/tq.h): argument marshalling only.

Every step of the hot path runs in the HIP kernels of libtq.so; this module
turns torch tensors into device pointers and structs, picks the current HIP
stream, and raises on non-zero status. There is no fallback: if libtq.so is
missing the import of the library fails loudly.

torch is imported first on purpose: its bundled HIP runtime carries the same
soname as the system one, so the library binds to the runtime torch already
loaded and torch's device pointers and streams are valid for it.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_SANITIZE=1 loads the host-sanitizer build (build.py --sanitize) instead
LIB_PATH = (os.path.join(os.path.dirname(_HERE), "_build", "san", "libtq_san.so")
            if os.environ.get("TQ_SANITIZE") == "1" else os.path.join(_HERE, "libtq.so"))

TQ_OK, TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_DEVICE, TQ_ERR_NOCONV = range(6)
TQ_F32, TQ_F16 = 0, 1
TQ_OP_SCORES, TQ_OP_DECODE_ATTN = 1, 2
TQ_LAW_GAUSSIAN = 0
TQ_LAW_SPHERE = 1


class TQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[tq status {code}] {msg}")
        self.code = code


class tq_quantizer(C.Structure):
    _fields_ = [("d", C.c_int), ("mse_bits", C.c_int), ("qjl_m", C.c_int),
                ("centroids", C.c_void_p), ("boundaries", C.c_void_p),
                ("diag_signs", C.c_void_p), ("S", C.c_void_p)]


class tq_packed(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("signs", C.c_void_p), ("norm", C.c_void_p),
                ("rnorm", C.c_void_p)]


EXPORTS = ("tq_codebook", "tq_quantize", "tq_scores", "tq_dequantize", "tq_decode_attn",
           "tq_decode_attn_noalloc", "tq_decode_step", "tq_workspace_size", "tq_last_error")
TQ_NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


def lib() -> C.CDLL:
    """Load libtq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m kv_cache_vector_03_amd.build`")
        L = C.CDLL(LIB_PATH)
        qp, pp, vp = C.POINTER(tq_quantizer), C.POINTER(tq_packed), C.c_void_p
        L.tq_codebook.argtypes = [C.c_int, C.c_int, C.c_int, vp, vp, C.POINTER(C.c_double)]
        L.tq_codebook.restype = C.c_int
        L.tq_quantize.argtypes = [qp, vp, C.c_int, C.c_int64, pp, vp]
        L.tq_quantize.restype = C.c_int
        L.tq_scores.argtypes = [qp, pp, C.c_int64, vp, C.c_int, C.c_int64, vp, vp, C.c_size_t, vp]
        L.tq_scores.restype = C.c_int
        L.tq_dequantize.argtypes = [qp, pp, C.c_int64, C.c_int, vp, C.c_int, vp]
        L.tq_dequantize.restype = C.c_int
        L.tq_decode_attn.argtypes = [qp, qp, pp, pp, C.c_int64, C.c_int64, C.c_int, vp, C.c_int,
                                     C.c_float, vp, vp, C.c_size_t, vp]
        L.tq_decode_attn.restype = C.c_int
        L.tq_decode_attn_noalloc.argtypes = [qp, qp, pp, pp, C.c_int64, C.c_int64, C.c_int, vp, C.c_int,
                                             C.c_float, vp, vp]
        L.tq_decode_attn_noalloc.restype = C.c_int
        L.tq_decode_step.argtypes = [qp, qp, pp, pp, C.c_int64, C.c_int64, C.c_int64, C.c_int, vp, vp,
                                     C.c_int, vp, C.c_int, C.c_float, vp, vp, C.c_size_t, vp]
        L.tq_decode_step.restype = C.c_int
        L.tq_workspace_size.argtypes = [C.c_int, qp, C.c_int64, C.c_int64, C.c_int]
        L.tq_workspace_size.restype = C.c_size_t
        L.tq_last_error.argtypes = []
        L.tq_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def tq_last_error() -> str:
    return lib().tq_last_error().decode()


def _check(rc: int) -> None:
    if rc != TQ_OK:
        raise TQError(rc, tq_last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    return int(t)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.float16:
        return TQ_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ------------------------------------------------------------------ state holders

class Quantizer:
    """Quantizer state on the device: codebook, random diagonal and JL matrix.

    ``diag`` is the uint32[d/32] bit mask (bit i set -> coordinate i negated);
    ``S`` the fp16 [qjl_m, d] matrix or None for codes-only (value) quantizers.
    """

    def __init__(self, d: int, mse_bits: int, qjl_m: int, diag, S=None, device="cuda", law: int = 0):
        self.d, self.mse_bits, self.qjl_m, self.law = d, mse_bits, qjl_m, law
        cent, bnd, dist = tq_codebook(d, mse_bits, law)
        self.distortion = dist
        self.centroids_host, self.boundaries_host = cent, bnd
        self.centroids = torch.from_numpy(cent).to(device)
        self.boundaries = torch.from_numpy(np.concatenate([bnd, np.zeros(1, np.float32)])).to(device)
        diag = np.ascontiguousarray(np.asarray(diag, dtype=np.uint32))
        self.diag = torch.from_numpy(diag.view(np.int32)).to(device)
        if qjl_m:
            S = torch.as_tensor(np.asarray(S, dtype=np.float16)) if not isinstance(S, torch.Tensor) else S
            self.S = S.to(device=device, dtype=torch.float16).contiguous()
            assert tuple(self.S.shape) == (qjl_m, d)
        else:
            self.S = None
        self.struct = tq_quantizer(d, mse_bits, qjl_m, _ptr(self.centroids), _ptr(self.boundaries),
                                   _ptr(self.diag), _ptr(self.S))

    @property
    def words(self) -> int:
        return self.d // 32


class Packed:
    """Packed vectors on the device (layout of include/tq.h)."""

    def __init__(self, codes, signs, norm, rnorm):
        self.codes, self.signs, self.norm, self.rnorm = codes, signs, norm, rnorm
        self.struct = tq_packed(_ptr(codes), _ptr(signs), _ptr(norm), _ptr(rnorm))

    @classmethod
    def empty(cls, q: Quantizer, n: int, device="cuda") -> "Packed":
        codes = torch.empty((n, q.mse_bits * q.words), dtype=torch.int32, device=device)
        signs = torch.empty((n, q.qjl_m // 32), dtype=torch.int32, device=device) if q.qjl_m else None
        norm = torch.empty(n, dtype=torch.int16, device=device)
        rnorm = torch.empty(n, dtype=torch.int16, device=device) if q.qjl_m else None
        return cls(codes, signs, norm, rnorm)

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    def slice(self, a: int, b: int) -> "Packed":
        """Vectors a..b-1 as views of the same device buffers."""
        def v(t):
            return t[a:b] if t is not None else None
        return Packed(v(self.codes), v(self.signs), v(self.norm), v(self.rnorm))

    def to_host(self):
        """numpy copies (codes/signs as uint32, norms as uint16 fp16 bits)."""
        c = self.codes.cpu().numpy().view(np.uint32)
        s = self.signs.cpu().numpy().view(np.uint32) if self.signs is not None else np.zeros((self.n, 0), np.uint32)
        nn = self.norm.cpu().numpy().view(np.uint16)
        r = self.rnorm.cpu().numpy().view(np.uint16) if self.rnorm is not None else np.zeros(self.n, np.uint16)
        return c, s, nn, r

    @classmethod
    def from_host(cls, codes, signs, norm, rnorm, device="cuda") -> "Packed":
        """Upload host arrays (uint32 codes/signs, uint16 fp16 norms)."""
        def t(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
        has_signs = signs is not None and np.asarray(signs).size > 0
        return cls(t(codes, np.int32), t(signs, np.int32) if has_signs else None,
                   t(norm, np.int16), t(rnorm, np.int16) if has_signs else None)


# ------------------------------------------------------------------ entry points

def tq_codebook(d: int, bits: int, law: int = TQ_LAW_GAUSSIAN):
    """Host Lloyd-Max solve: (centroids float32[2^bits], boundaries float32[2^bits-1], distortion)."""
    L = 1 << bits
    cent = np.zeros(L, np.float32)
    bnd = np.zeros(max(L - 1, 1), np.float32)
    dist = C.c_double()
    _check(lib().tq_codebook(d, bits, law, cent.ctypes.data, bnd.ctypes.data, C.byref(dist)))
    return cent, bnd[:L - 1], dist.value


def tq_workspace_size(op: int, qk: Quantizer, n_a: int, n_b: int, G: int = 0) -> int:
    return int(lib().tq_workspace_size(op, C.byref(qk.struct), n_a, n_b, G))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def tq_quantize(q: Quantizer, x: torch.Tensor, out: Packed, n: int | None = None, stream=None) -> None:
    n = x.shape[0] if n is None else n
    _check(lib().tq_quantize(C.byref(q.struct), _ptr(x), _dtype_code(x), n, C.byref(out.struct),
                             _stream(stream)))


def tq_scores(q: Quantizer, keys: Packed, n_keys: int, queries: torch.Tensor, scores: torch.Tensor,
              ws: torch.Tensor | None = None, stream=None) -> None:
    n_q = queries.shape[0]
    if ws is None:
        ws = workspace(tq_workspace_size(TQ_OP_SCORES, q, n_q, n_keys), queries.device)
    _check(lib().tq_scores(C.byref(q.struct), C.byref(keys.struct), n_keys, _ptr(queries),
                           _dtype_code(queries), n_q, _ptr(scores), _ptr(ws), ws.numel(),
                           _stream(stream)))


def tq_dequantize(q: Quantizer, packed: Packed, n: int, include_qjl: bool, out: torch.Tensor,
                  stream=None) -> None:
    _check(lib().tq_dequantize(C.byref(q.struct), C.byref(packed.struct), n, 1 if include_qjl else 0,
                               _ptr(out), _dtype_code(out), _stream(stream)))


def tq_decode_attn(qk: Quantizer, qv: Quantizer, k: Packed, v: Packed, n_streams: int, T: int, G: int,
                   q: torch.Tensor, out: torch.Tensor, scale: float = 0.0,
                   ws: torch.Tensor | None = None, stream=None) -> None:
    if ws is None:
        ws = workspace(tq_workspace_size(TQ_OP_DECODE_ATTN, qk, n_streams, T, G), q.device)
    _check(lib().tq_decode_attn(C.byref(qk.struct), C.byref(qv.struct), C.byref(k.struct),
                                C.byref(v.struct), n_streams, T, G, _ptr(q), _dtype_code(q),
                                float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def tq_decode_attn_noalloc(qk: Quantizer, qv: Quantizer, k: Packed, v: Packed, n_streams: int, T: int,
                           G: int, q: torch.Tensor, out: torch.Tensor, scale: float = 0.0, stream=None) -> None:
    """tq_decode_attn with the library's fixed per-device scratch as its
    workspace: the call allocates nothing (calls that overlap on one device race)."""
    _check(lib().tq_decode_attn_noalloc(C.byref(qk.struct), C.byref(qv.struct), C.byref(k.struct),
                                        C.byref(v.struct), n_streams, T, G, _ptr(q), _dtype_code(q),
                                        float(scale), _ptr(out), _stream(stream)))


def tq_decode_step(qk: Quantizer, qv: Quantizer, k: Packed, v: Packed, n_streams: int, T: int, cap: int,
                   G: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                   scale: float = 0.0, ws: torch.Tensor | None = None, stream=None) -> None:
    """Append each stream's new token (k_new, v_new: [n_streams][d]) at position T
    of caches laid out with `cap` vectors per stream, then attend over T + 1 tokens."""
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must have the same dtype")
    if ws is None:
        ws = workspace(tq_workspace_size(TQ_OP_DECODE_ATTN, qk, n_streams, T + 1, G), q.device)
    _check(lib().tq_decode_step(C.byref(qk.struct), C.byref(qv.struct), C.byref(k.struct),
                                C.byref(v.struct), n_streams, T, cap, G, _ptr(k_new), _ptr(v_new),
                                _dtype_code(k_new), _ptr(q), _dtype_code(q), float(scale), _ptr(out),
                                _ptr(ws), ws.numel(), _stream(stream)))
