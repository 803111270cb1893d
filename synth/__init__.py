"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no arithmetic of the compression method. It only draws
random numbers and shapes them into the workloads the benchmark pages
describe (KV tensors, queries, the random +-1 diagonal, the Gaussian JL
matrix). Every draw is counter based, so element ``i`` of any stream can be
produced alone, in any order, on the host (here, with numpy) or on the GPU
(``synth/gen.hip``), and both produce the same bits.

Generator definition (both sides implement exactly this):

* SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): with the golden gamma
  ``G = 0x9E3779B97F4A7C15`` and the finaliser
  ``mix(z) = z ^ (z >> 31)`` after ``z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9``
  and ``z = (z ^ (z >> 27)) * 0x94D049BB133111EB`` (all mod 2^64), draw ``i``
  of a stream with key ``k`` is ``mix(k + (i + 1) * G)``.
* The key of stream ``role`` under ``seed`` is ``mix(seed + (role + 1) * G)``.
* uniform ``i`` = ``(draw_i >> 11) * 2^-53`` in [0, 1).
* normal ``e`` (Box-Muller, both outputs used in order): with ``j = e // 2``,
  ``u1 = 1 - uniform(2j)``, ``u2 = uniform(2j + 1)``,
  ``r = sqrt(-2 ln u1)``, ``theta = 2 pi u2``; even ``e`` gives
  ``r cos theta``, odd ``e`` gives ``r sin theta``.
* ``ln``, ``sin`` and ``cos`` are evaluated with our own short series written
  with + - * / only (``_ln``, ``_sincos_2pi``) in a fixed order, so that the
  host and the GPU (built with fp-contraction off) give identical doubles.
  ``sqrt`` is the IEEE correctly rounded square root on both sides.
* Stored values are rounded once per step: double -> fp32 (RNE), and for fp16
  tensors fp32 -> fp16 (RNE).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream roles (one independent stream per role)
ROLE_DATA_K = 1
ROLE_DATA_V = 2
ROLE_QUERY = 3
ROLE_DIAG_K = 4
ROLE_PROJ_K = 5
ROLE_DIAG_V = 6
ROLE_SCALE_K = 7
ROLE_SCALE_V = 8
ROLE_OUTLIER = 9
ROLE_NEEDLE_POS = 10
ROLE_NEEDLE_NOISE = 11
ROLE_PAIR_Q = 12
ROLE_PROJ_V = 13

LN2 = 0.6931471805599453
SQRT2 = 1.4142135623730951
HALF_PI = 1.5707963267948966


def _mix(z):
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, role: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = np.uint64(seed % (1 << 64)) + np.uint64(role + 1) * GOLDEN
    return _mix(np.array([k], dtype=np.uint64))[0]


def draws(seed: int, role: int, idx) -> np.ndarray:
    """Raw 64-bit draws ``idx`` (array of non-negative ints) of a stream."""
    key = stream_key(seed, role)
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + (i + np.uint64(1)) * GOLDEN
    return _mix(z)


def uniforms(seed: int, role: int, idx) -> np.ndarray:
    d = draws(seed, role, idx)
    return (d >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


# inverse odd integers and inverse factorials, produced by correctly rounded
# divisions in a fixed order (the GPU side builds the same tables the same way)
_INV_ODD = [1.0 / (2 * j + 1) for j in range(12)]


def _inv_fact_table(n: int):
    t = [1.0]
    c = 1.0
    for k in range(1, n + 1):
        c = c / k
        t.append(c)
    return t


_INV_FACT = _inv_fact_table(24)


def _ln(x: np.ndarray) -> np.ndarray:
    """Natural log for x in (0, 1] by exponent split plus an atanh series."""
    f, e = np.frexp(x)          # x = f * 2^e, f in [0.5, 1)
    f = f * 2.0                 # [1, 2)
    e = e.astype(np.float64) - 1.0
    big = f > SQRT2
    f = np.where(big, f * 0.5, f)
    e = np.where(big, e + 1.0, e)
    s = (f - 1.0) / (f + 1.0)
    s2 = s * s
    p = np.full_like(s, _INV_ODD[11])
    for j in range(10, -1, -1):
        p = p * s2 + _INV_ODD[j]
    t = 2.0 * s
    t = t * p
    return e * LN2 + t


def _sincos_2pi(u: np.ndarray):
    """(sin, cos) of 2*pi*u for u in [0, 1) by quadrant split plus Taylor."""
    v = u * 4.0
    q = np.floor(v)
    f = v - q
    a = f * HALF_PI
    a2 = a * a
    # sin a = a * sum (-1)^k a^2k / (2k+1)!, k = 0..10
    ps = np.full_like(a, _INV_FACT[21])
    for k in range(9, -1, -1):
        c = _INV_FACT[2 * k + 1]
        ps = c - ps * a2
    s = a * ps
    # cos a = sum (-1)^k a^2k / (2k)!, k = 0..11
    pc = np.full_like(a, _INV_FACT[22])
    for k in range(10, -1, -1):
        c = _INV_FACT[2 * k]
        pc = c - pc * a2
    cs = pc
    qi = q.astype(np.int64)
    sin_t = np.select([qi == 0, qi == 1, qi == 2], [s, cs, -s], -cs)
    cos_t = np.select([qi == 0, qi == 1, qi == 2], [cs, -s, -cs], s)
    return sin_t, cos_t


def normals(seed: int, role: int, idx) -> np.ndarray:
    """Standard normal draws for element indices ``idx`` (float64)."""
    e = np.asarray(idx, dtype=np.int64)
    if e.size > _CHUNK:
        flat = e.reshape(-1)
        out = np.empty(flat.shape, dtype=np.float64)
        for a in range(0, flat.size, _CHUNK):
            out[a:a + _CHUNK] = _normals_flat(seed, role, flat[a:a + _CHUNK])
        return out.reshape(e.shape)
    return _normals_flat(seed, role, e)


_CHUNK = 1 << 15


def _normals_flat(seed: int, role: int, e: np.ndarray) -> np.ndarray:
    j = (e // 2).astype(np.uint64)
    u1 = 1.0 - uniforms(seed, role, j * np.uint64(2))
    u2 = uniforms(seed, role, j * np.uint64(2) + np.uint64(1))
    r = np.sqrt(-2.0 * _ln(u1))
    sn, cs = _sincos_2pi(u2)
    return np.where(e % 2 == 0, r * cs, r * sn)


def to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def to_f16(x: np.ndarray) -> np.ndarray:
    return to_f32(x).astype(np.float16)


# ---------------------------------------------------------------- quantizer state

def diag_signs(seed: int, role: int, d: int) -> np.ndarray:
    """Random +-1 diagonal as a bit mask: uint32[ceil(d/32)], bit i set -> -1."""
    bits = (draws(seed, role, np.arange(d)) >> np.uint64(63)).astype(np.uint32)
    words = np.zeros((d + 31) // 32, dtype=np.uint32)
    for i in range(d):
        words[i // 32] |= np.uint32(bits[i]) << np.uint32(i % 32)
    return words


def proj_matrix_f16(seed: int, role: int, m: int, d: int) -> np.ndarray:
    """Gaussian JL matrix S (m x d, row-major), entries N(0,1) rounded to fp16."""
    return to_f16(normals(seed, role, np.arange(m * d)).reshape(m, d))


# ---------------------------------------------------------------- workloads

def kv_elements(seed: int, role: int, shape, first_vector: int = 0, n_vectors=None,
                scales=None) -> np.ndarray:
    """Elements of a [..., d] tensor whose flat element index is the draw index.

    ``scales`` (optional) broadcasts over the leading vector index grid by
    (vector_index // tokens) and channel; see ``kv_f16``.
    """
    d = shape[-1]
    nvec_total = int(np.prod(shape[:-1]))
    if n_vectors is None:
        n_vectors = nvec_total - first_vector
    idx = (np.arange(first_vector, first_vector + n_vectors, dtype=np.int64)[:, None] * d
           + np.arange(d, dtype=np.int64)[None, :])
    return normals(seed, role, idx)


def lognormal_scales(seed: int, role: int, n_groups: int, d: int) -> np.ndarray:
    """Per-(group, channel) scales exp(z), z ~ N(0,1); float64 [n_groups, d]."""
    z = normals(seed, role, np.arange(n_groups * d)).reshape(n_groups, d)
    return np.exp(z)


def outlier_scales(seed: int, d: int, n_outliers: int = 4, factor: float = 20.0) -> np.ndarray:
    """Channel scales with ``n_outliers`` distinct seeded channels set to ``factor``."""
    chosen = []
    i = 0
    while len(chosen) < n_outliers:
        c = int(uniforms(seed, ROLE_OUTLIER, [i])[0] * d)
        i += 1
        if c not in chosen:
            chosen.append(c)
    s = np.ones(d, dtype=np.float64)
    s[chosen] = factor
    return s


def scaled_f16(z: np.ndarray, scale_rows: np.ndarray) -> np.ndarray:
    """fp16(fp32(z * scale)) with the product in double."""
    return to_f16(z * scale_rows)


@dataclass(frozen=True)
class KVShape:
    groups: int      # layers * kv_heads (one group = one stream)
    tokens: int
    d: int

    @property
    def n_vectors(self) -> int:
        return self.groups * self.tokens


def kv_stream_f16(seed: int, role: int, shp: KVShape, scales: np.ndarray,
                  vec_index: np.ndarray) -> np.ndarray:
    """fp16 values of selected vectors (flat index = group * tokens + token)."""
    vec_index = np.asarray(vec_index, dtype=np.int64)
    d = shp.d
    idx = vec_index[:, None] * d + np.arange(d, dtype=np.int64)[None, :]
    z = normals(seed, role, idx)
    grp = vec_index // shp.tokens
    return scaled_f16(z, scales[grp])


def unit_vectors_f32(seed: int, role: int, n: int, d: int, first: int = 0) -> np.ndarray:
    """Normalised N(0, I) vectors; the norm is summed in index order in double."""
    idx = (np.arange(first, first + n, dtype=np.int64)[:, None] * d
           + np.arange(d, dtype=np.int64)[None, :])
    z = normals(seed, role, idx)
    acc = np.zeros(n, dtype=np.float64)
    for i in range(d):
        acc = acc + z[:, i] * z[:, i]
    nrm = np.sqrt(acc)
    return to_f32(z / nrm[:, None])


def needle_case(seed: int, seq: int, d: int, noise: float = 0.1):
    """Needle test input: N(0,1) keys, N(0,1) query, one key = query + noise.

    Returns (keys float64 [seq, d], query float64 [d], position).
    """
    keys = normals(seed, ROLE_DATA_K, np.arange(seq * d)).reshape(seq, d)
    q = normals(seed, ROLE_QUERY, np.arange(d))
    pos = int(uniforms(seed, ROLE_NEEDLE_POS, [0])[0] * seq)
    keys[pos] = q + noise * normals(seed, ROLE_NEEDLE_NOISE, np.arange(d))
    return keys, q, pos
