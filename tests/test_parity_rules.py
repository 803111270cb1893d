"""The parity checker itself (CPU only): outputs built from the oracle with a
planted change stand in for a GPU result.

* A code moved one level inside the 1e-5 boundary window, with the sketch the
  oracle builds on that code, passes; so do its rebuilt signs and residual
  norm, which differ from the oracle's own.
* The same moved code with the oracle's original signs fails wherever a sign
  differs outside |u| < 1e-5 of the rebuilt projection.
* A sign flipped where |u| is large fails; a code moved outside the window fails.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle
import synth
from parity import WINDOW, check_quantize


def _setup(d=128, bits=2):
    diag = synth.diag_signs(5, synth.ROLE_DIAG_K, d)
    S = synth.proj_matrix_f16(5, synth.ROLE_PROJ_K, d, d)
    Q = oracle.Quantizer(d, bits, d, diag, S)
    i = np.arange(d)
    D = np.where((Q.diag[i // 32] >> (i % 32).astype(np.uint32)) & 1, -1.0, 1.0)
    R = hadamard(d) * D[None, :] / np.sqrt(d)          # y = R x / ||x||
    # unit vectors whose coordinate 9 sits 4e-6 above the central boundary
    y = synth.normals(8, synth.ROLE_DATA_K, np.arange(6 * d)).reshape(6, d)
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    t = float(Q.bnd[(1 << bits) // 2 - 1])
    y[:, 9] = 0.0
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    y *= np.sqrt(1 - (t + 4e-6) ** 2)
    y[:, 9] = t + 4e-6
    x = y @ R                                          # R orthogonal: x = R^T y
    return Q, x


def _move_code(Q, codes, v, i, k2):
    G = Q.d // 8
    codes = codes.copy()
    base = 8 * Q.bits * (i % G) + Q.bits * (i // G)
    for p in range(Q.bits):
        w, b = (base + p) // 32, (base + p) % 32
        codes[v, w] = (codes[v, w] & ~np.uint32(1 << b)) | np.uint32(((k2 >> p) & 1) << b)
    return codes


def test_in_window_code_with_rebuilt_sketch_passes():
    Q, x = _setup()
    P, y, u = oracle.quantize(Q, x, want_y=True, want_u=True)
    k = oracle.unpack_codes(Q, P.codes)[2, 9]
    codes = _move_code(Q, P.codes, 2, 9, k - 1)        # the adjacent level below
    s2, r2 = oracle.sketch(Q, y[2:3], codes[2:3])
    signs, rnorm = P.signs.copy(), P.rnorm.copy()
    signs[2], rnorm[2] = s2[0], r2[0]
    assert not np.array_equal(signs, P.signs)          # the rebuilt sketch really differs
    nbad, _, _ = check_quantize(Q, x, (codes, signs, P.norm, rnorm))
    assert nbad == 1


def test_in_window_code_with_stale_signs_fails():
    Q, x = _setup()
    P, y = oracle.quantize(Q, x, want_y=True)
    k = oracle.unpack_codes(Q, P.codes)[2, 9]
    codes = _move_code(Q, P.codes, 2, 9, k - 1)
    _, _, u2 = oracle.sketch(Q, y[2:3], codes[2:3], want_u=True)
    stale = oracle.unpack_signs(Q, P.signs[2:3])[0] != (u2[0] >= 0)
    assert np.any(stale & (np.abs(u2[0]) >= WINDOW))   # the stale signs are wrong somewhere
    _, r2 = oracle.sketch(Q, y[2:3], codes[2:3])
    rnorm = P.rnorm.copy()
    rnorm[2] = r2[0]
    with pytest.raises(AssertionError, match="sign mismatch"):
        check_quantize(Q, x, (codes, P.signs, P.norm, rnorm))


def test_sign_flip_outside_window_fails():
    Q, x = _setup()
    P, u = oracle.quantize(Q, x, want_u=True)
    j = int(np.argmax(np.abs(u[4])))                   # largest projection of vector 4
    G = Q.m // 8
    b = 8 * (j % G) + j // G
    signs = P.signs.copy()
    signs[4, b // 32] ^= np.uint32(1 << (b % 32))
    with pytest.raises(AssertionError, match="sign mismatch"):
        check_quantize(Q, x, (P.codes, signs, P.norm, P.rnorm))


def test_code_moved_outside_window_fails():
    Q, x = _setup()
    P = oracle.quantize(Q, x)
    idx = oracle.unpack_codes(Q, P.codes)
    k = idx[1, 40]
    codes = _move_code(Q, P.codes, 1, 40, k + 1 if k + 1 < 4 else k - 1)
    with pytest.raises(AssertionError, match="outside the boundary window"):
        check_quantize(Q, x, (codes, P.signs, P.norm, P.rnorm))
