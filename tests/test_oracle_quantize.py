"""Pins for the oracle's quantizer (rotation, codes, packing, QJL signs, scalars).

Independent references used here:
* ``scipy.linalg.hadamard`` (Sylvester construction, natural order) for H;
* one-hot inputs, whose rotated image is a known Hadamard column, so codes,
  packed words and residual signs are predictable by hand;
* brute force over all code vectors for tiny d;
* a projection matrix that is a cyclic shift, which fixes the orientation of S;
* numpy's float16 conversion for the stored scalars.
"""
import itertools

import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle
import synth


def make_q(d, bits, m, seed=3, S=None):
    diag = synth.diag_signs(seed, synth.ROLE_DIAG_K, d)
    if m and S is None:
        S = synth.proj_matrix_f16(seed, synth.ROLE_PROJ_K, m, d)
    return oracle.Quantizer(d, bits, m, diag, S)


def dvec(Q):
    i = np.arange(Q.d)
    return np.where((Q.diag[i // 32] >> (i % 32).astype(np.uint32)) & 1, -1.0, 1.0)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_one_hot_gives_hadamard_column(d):
    Q = make_q(d, 2, 0)
    H = hadamard(d).astype(np.float64)
    D = dvec(Q)
    for i in [0, 1, 5, d // 2 + 3, d - 1]:
        x = np.zeros((1, d))
        x[0, i] = 3.0
        _, y = oracle.quantize(Q, x, want_y=True)
        np.testing.assert_allclose(y[0], D[i] * H[:, i] / np.sqrt(d), atol=1e-15)


def test_rotation_is_orthogonal():
    d = 128
    Q = make_q(d, 3, 0)
    x = synth.normals(5, synth.ROLE_DATA_K, np.arange(64 * d)).reshape(64, d)
    _, y = oracle.quantize(Q, x, want_y=True)
    n = np.linalg.norm(x, axis=1)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), 1.0, atol=1e-13)
    G = (x / n[:, None]) @ (x / n[:, None]).T
    np.testing.assert_allclose(y @ y.T, G, atol=1e-13)
    # and equals R x / ||x|| with R = H D / sqrt(d) built from scipy's H
    R = hadamard(d) * dvec(Q)[None, :] / np.sqrt(d)
    np.testing.assert_allclose(y, (x / n[:, None]) @ R.T, atol=1e-13)


def test_one_hot_codes_and_packed_words():
    d = 128
    # 2-bit: |y| = 1/sqrt(d) lies above the outer boundary 0.981/sqrt(d) -> outer levels
    Q = make_q(d, 2, 0)
    D = dvec(Q)
    for i in (0, 1):
        x = np.zeros((1, d))
        x[0, i] = 1.0
        P = oracle.quantize(Q, x)
        idx = oracle.unpack_codes(Q, P.codes)[0]
        H = hadamard(d)[:, i] * D[i]
        assert np.array_equal(idx, np.where(H > 0, 3, 0))
        # group c holds coordinates c + 16 t, all of the parity of c; each group is a
        # 16-bit field of eight 2-bit codes, two groups per word (even group low)
        if i == 0:
            w = 0xFFFFFFFF if D[0] > 0 else 0
        else:
            w = 0x0000FFFF if D[1] > 0 else 0xFFFF0000
        assert np.all(P.codes[0] == w), [hex(v) for v in P.codes[0]]
    # 3-bit: |y| sqrt(d) = 1 lies between boundaries 0.5006 and 1.0500 -> levels 2 / 5
    Q3 = make_q(d, 3, 0)
    x = np.zeros((1, d))
    x[0, 7] = 1.0
    idx = oracle.unpack_codes(Q3, oracle.quantize(Q3, x).codes)[0]
    H = hadamard(d)[:, 7] * dvec(Q3)[7]
    assert np.array_equal(idx, np.where(H > 0, 5, 2))
    assert np.allclose(Q3.cent[[2, 5]] * np.sqrt(d), [-0.7560, 0.7560], atol=1e-3)


@pytest.mark.parametrize("d,bits", [(128, 3), (64, 2), (256, 4), (128, 1), (64, 5), (128, 6), (256, 7),
                                    (128, 8)])
def test_packing_bit_layout_against_manual_pack(d, bits):
    """Group-major stream: group c = coordinates c + (d/8) t; code t of group c
    at stream bits 8*bits*c + bits*t .. +bits-1; words little-endian."""
    Q = make_q(d, bits, 0)
    x = synth.normals(9, synth.ROLE_DATA_K, np.arange(16 * d)).reshape(16, d)
    P, y = oracle.quantize(Q, x, want_y=True)
    idx = (y[:, :, None] > Q.cb.boundaries.astype(np.float64)[None, None, :]).sum(-1)
    G = d // 8
    for v in range(16):
        stream = 0
        for c in range(G):
            for t in range(8):
                stream |= int(idx[v, c + G * t]) << (8 * bits * c + bits * t)
        words = [(stream >> (32 * w)) & 0xFFFFFFFF for w in range(bits * d // 32)]
        assert [int(a) for a in P.codes[v]] == words


def test_sign_layout_against_manual_pack():
    d = 128
    Q = make_q(d, 2, d)
    x = synth.normals(10, synth.ROLE_DATA_K, np.arange(8 * d)).reshape(8, d)
    P, u = oracle.quantize(Q, x, want_u=True)
    for v in range(8):
        stream = 0
        for j in range(d):
            if u[v, j] >= 0:
                stream |= 1 << (8 * (j % 16) + j // 16)
        assert [int(a) for a in P.signs[v]] == [(stream >> (32 * w)) & 0xFFFFFFFF for w in range(4)]


@pytest.mark.parametrize("d,bits", [(4, 2), (8, 2), (4, 3)])
def test_codes_are_the_brute_force_argmin(d, bits):
    Q = make_q(d, bits, 0)
    x = synth.normals(11, synth.ROLE_DATA_K, np.arange(40 * d)).reshape(40, d)
    P, y = oracle.quantize(Q, x, want_y=True)
    idx = oracle.unpack_codes(Q, P.codes)
    c = Q.cent.astype(np.float64)
    allc = np.array(list(itertools.product(range(1 << bits), repeat=d)))
    for v in range(40):
        err = ((y[v][None, :] - c[allc]) ** 2).sum(1)
        assert np.array_equal(allc[np.argmin(err)], idx[v])


@pytest.mark.parametrize("d,bits", [(64, 5), (128, 6), (128, 8), (256, 7)])
def test_wide_codes_are_the_nearest_centroid(d, bits):
    """Wide codebooks: the code of each coordinate is its nearest stored
    centroid (the distortion is separable over coordinates, so this is the
    argmin over whole code vectors); ties cannot occur on these inputs."""
    Q = make_q(d, bits, 0)
    x = synth.normals(12, synth.ROLE_DATA_K, np.arange(64 * d)).reshape(64, d)
    P, y = oracle.quantize(Q, x, want_y=True)
    idx = oracle.unpack_codes(Q, P.codes)
    c = Q.cent.astype(np.float64)
    dist = np.abs(y[..., None] - c[None, None, :])
    assert np.array_equal(np.argmin(dist, axis=-1), idx)


def test_projection_orientation_with_shift_matrix():
    """S with S[j, (j+1) % d] = 1 gives u_j = r_{j+1}; a transposed S would
    give r_{j-1}. One-hot input e_3 makes r periodic with period 4."""
    d = 128
    S = np.zeros((d, d), np.float16)
    S[np.arange(d), (np.arange(d) + 1) % d] = 1.0
    Q = make_q(d, 3, d, S=S)  # 2-bit MSE + 1-bit QJL ("b=3 total")
    Q = oracle.Quantizer(d, 2, d, Q.diag, S)
    x = np.zeros((1, d))
    x[0, 3] = 1.0
    P, y, u = oracle.quantize(Q, x, want_y=True, want_u=True)
    sgn = oracle.unpack_signs(Q, P.signs)[0]
    # y = D3 H[:,3]/sqrt(d): outer level, residual sign opposite to y (|y| < c_outer)
    h = hadamard(d)[:, 3] * dvec(Q)[3]
    r_sign = -h
    expect = (np.roll(r_sign, -1) >= 0).astype(int)   # r_{j+1}
    wrong = (np.roll(r_sign, 1) >= 0).astype(int)     # r_{j-1}
    assert np.array_equal(sgn, expect)
    assert not np.array_equal(sgn, wrong)


def test_stored_scalars_are_fp16_rne():
    d = 64
    Q = make_q(d, 2, d)
    x = synth.normals(13, synth.ROLE_DATA_K, np.arange(200 * d)).reshape(200, d) * 7.3
    P, y = oracle.quantize(Q, x, want_y=True)
    n = np.linalg.norm(x, axis=1)
    assert np.array_equal(P.norm, n.astype(np.float16).view(np.uint16))
    c = Q.cent.astype(np.float64)[oracle.unpack_codes(Q, P.codes)]
    g = np.linalg.norm(y - c, axis=1)
    assert np.array_equal(P.rnorm, g.astype(np.float16).view(np.uint16))


def test_zero_vector():
    d = 128
    for bits in (2, 3, 4):
        Q = make_q(d, bits, d)
        P, y = oracle.quantize(Q, np.zeros((1, d)), want_y=True)
        assert np.all(y == 0)
        L = 1 << bits
        assert np.all(oracle.unpack_codes(Q, P.codes) == L // 2 - 1)
        assert P.norm[0] == 0


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 1), (128, 2), (256, 3)])
def test_sketch_on_own_codes_reproduces_quantize(d, bits):
    """The QJL stage run on the oracle's own codes gives back exactly the
    signs, residual norms and projections ``quantize`` wrote."""
    Q = make_q(d, bits, d)
    x = synth.normals(13, synth.ROLE_DATA_K, np.arange(300 * d)).reshape(300, d)
    P, y, u = oracle.quantize(Q, x, want_y=True, want_u=True)
    s2, r2, u2 = oracle.sketch(Q, y, P.codes, want_u=True)
    assert np.array_equal(s2, P.signs) and np.array_equal(r2, P.rnorm)
    assert np.array_equal(u2, u)


def test_sketch_on_shifted_code_is_linear_in_the_change():
    """Moving coordinate i of a vector one level up changes the residual by
    -(c[k+1] - c[k]) e_i, so u = S r moves by -(c[k+1] - c[k]) S[:, i] and
    gamma^2 by -2 r_i dc + dc^2 (checked with numpy's S and the oracle's y);
    the packed code change is made by hand on the group-major layout."""
    d, bits = 128, 2
    Q = make_q(d, bits, d)
    x = synth.normals(29, synth.ROLE_DATA_K, np.arange(40 * d)).reshape(40, d)
    P, y, u = oracle.quantize(Q, x, want_y=True, want_u=True)
    idx = oracle.unpack_codes(Q, P.codes)
    S = Q.S_f64()
    cent = Q.cent.astype(np.float64)
    G = d // 8
    for v, i in [(0, 0), (3, 17), (11, 64), (39, 127)]:
        k = idx[v, i]
        k2 = k + 1 if k + 1 < (1 << bits) else k - 1
        codes = P.codes.copy()
        base = 8 * bits * (i % G) + bits * (i // G)
        for p in range(bits):
            w, b = (base + p) // 32, (base + p) % 32
            codes[v, w] = (codes[v, w] & ~np.uint32(1 << b)) | np.uint32(((k2 >> p) & 1) << b)
        s2, r2, u2 = oracle.sketch(Q, y[v:v + 1], codes[v:v + 1], want_u=True)
        dc = cent[k2] - cent[k]
        np.testing.assert_allclose(u2[0], u[v] - dc * S[:, i], rtol=0, atol=1e-13)
        r_i = y[v, i] - cent[k]
        g2 = np.sum((y[v] - cent[idx[v]]) ** 2) - 2 * r_i * dc + dc * dc
        assert abs(r2[0].view(np.float16).astype(np.float64) - np.sqrt(g2)) <= np.spacing(np.float16(np.sqrt(g2)))
        expect = (u2[0] >= 0).astype(np.int64)
        assert np.array_equal(oracle.unpack_signs(Q, s2)[0], expect)
