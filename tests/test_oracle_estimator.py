"""Pins for the oracle's score estimator, dequantizer and decode attention.

* QJL identity (textbook): for s ~ N(0, I), E[sign(<s,r>) <s,q>] = sqrt(2/pi) <q,r>/||r||,
  so gamma sqrt(pi/2)/m sum_j p_j sign(u_j) is unbiased for <q', r> with variance
  ((pi/2) ||q'||^2 gamma^2 - <q',r>^2) / m. Checked over many seeded S draws.
* Algebraic invariant: the estimated score equals <q, dequantize(k)>.
* Decode attention equals plain softmax attention (numpy, float64) over the
  dequantized cache.
* Special cases: zero vector scores 0; with many MSE bits the score tends to
  the exact inner product.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle
import synth


def make_q(d, bits, m, seed=3):
    diag = synth.diag_signs(seed, synth.ROLE_DIAG_K, d)
    S = synth.proj_matrix_f16(seed, synth.ROLE_PROJ_K, m, d) if m else None
    return oracle.Quantizer(d, bits, m, diag, S)


def test_qjl_unbiased_and_variance_over_S_draws():
    d = 32
    n_draws = 3000
    x = synth.normals(21, synth.ROLE_DATA_K, np.arange(d))[None, :]
    q = synth.normals(21, synth.ROLE_QUERY, np.arange(d))[None, :]
    diag = synth.diag_signs(21, synth.ROLE_DIAG_K, d)
    cb = oracle.codebook(d, 2)
    Qm = oracle.Quantizer(d, 2, 0, diag, None, cb=cb)
    Pm, y = oracle.quantize(Qm, x, want_y=True)
    s_mse = oracle.scores(Qm, Pm, q)[0, 0]
    # reference quantities from scipy's Hadamard, independent of the oracle
    i = np.arange(d)
    D = np.where((diag[i // 32] >> (i % 32).astype(np.uint32)) & 1, -1.0, 1.0)
    qr = (hadamard(d) * D[None, :] / np.sqrt(d)) @ q[0]
    r = y[0] - cb.centroids.astype(np.float64)[oracle.unpack_codes(Qm, Pm.codes)[0]]
    gamma = np.linalg.norm(r)
    est = np.empty(n_draws)
    g16 = None
    for k in range(n_draws):
        S = synth.proj_matrix_f16(1000 + k, synth.ROLE_PROJ_K, d, d)
        Qp = oracle.Quantizer(d, 2, d, diag, S, cb=cb)
        Pp = oracle.quantize(Qp, x)
        assert np.array_equal(Pp.codes, Pm.codes) and Pp.norm[0] == Pm.norm[0]
        g16 = oracle.half_to_double(Pp.rnorm[0])
        n16 = oracle.half_to_double(Pp.norm[0])
        est[k] = (oracle.scores(Qp, Pp, q)[0, 0] - s_mse) / n16
    target = qr @ r * g16 / gamma
    se = est.std(ddof=1) / np.sqrt(n_draws)
    assert abs(est.mean() - target) < 4 * se
    var_th = ((np.pi / 2) * (qr @ qr) * g16 ** 2 - target ** 2) / d
    assert abs(est.var(ddof=1) / var_th - 1) < 0.12


@pytest.mark.parametrize("bits,m", [(2, 128), (3, 0), (3, 128), (4, 0)])
def test_scores_equal_inner_product_with_dequantized(bits, m):
    d = 128
    Q = make_q(d, bits, m)
    x = synth.normals(23, synth.ROLE_DATA_K, np.arange(300 * d)).reshape(300, d) * 2.0
    q = synth.normals(23, synth.ROLE_QUERY, np.arange(7 * d)).reshape(7, d)
    P = oracle.quantize(Q, x)
    s = oracle.scores(Q, P, q)
    xh = oracle.dequantize(Q, P, include_qjl=True)
    np.testing.assert_allclose(s, q @ xh.T, atol=1e-10)
    if m:
        # without the QJL term the dequantized vector is the MSE reconstruction
        xm = oracle.dequantize(Q, P, include_qjl=False)
        assert np.abs(xm - xh).max() > 1e-3


def test_decode_attention_is_softmax_over_dequantized_cache():
    d, T, G, ns = 64, 300, 4, 3
    QK = make_q(d, 2, d, seed=5)
    QV = oracle.Quantizer(d, 3, 0, synth.diag_signs(5, synth.ROLE_DIAG_V, d), None)
    K = synth.normals(31, synth.ROLE_DATA_K, np.arange(ns * T * d)).reshape(ns * T, d) * 1.5
    V = synth.normals(31, synth.ROLE_DATA_V, np.arange(ns * T * d)).reshape(ns * T, d)
    q = synth.normals(31, synth.ROLE_QUERY, np.arange(ns * G * d)).reshape(ns, G, d)
    PK = oracle.quantize(QK, K)
    PV = oracle.quantize(QV, V)
    out = oracle.decode_attn(QK, QV, PK, PV, ns, T, G, q)
    Kh = oracle.dequantize(QK, PK).reshape(ns, T, d)
    Vh = oracle.dequantize(QV, PV).reshape(ns, T, d)
    for s in range(ns):
        z = q[s] @ Kh[s].T / np.sqrt(d)
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(out[s], p @ Vh[s], atol=1e-12)
    # explicit scale is honoured
    out2 = oracle.decode_attn(QK, QV, PK, PV, ns, T, G, q, scale=0.05)
    z = q[0] @ Kh[0].T * 0.05
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(out2[0], p @ Vh[0], atol=1e-12)


def test_zero_vector_scores_zero():
    d = 128
    Q = make_q(d, 2, d)
    x = np.zeros((2, d))
    x[1, 5] = 1.0
    P = oracle.quantize(Q, x)
    q = synth.normals(3, synth.ROLE_QUERY, np.arange(d))[None, :]
    s = oracle.scores(Q, P, q)
    assert s[0, 0] == 0.0
    assert np.all(oracle.dequantize(Q, P)[0] == 0.0)


def test_many_bits_approach_exact_inner_product():
    d = 64
    x = synth.normals(41, synth.ROLE_DATA_K, np.arange(50 * d)).reshape(50, d)
    q = synth.normals(41, synth.ROLE_QUERY, np.arange(3 * d)).reshape(3, d)
    exact = q @ x.T
    errs = []
    for bits in (2, 4, 6, 8):
        Q = make_q(d, bits, 0)
        s = oracle.scores(Q, oracle.quantize(Q, x), q)
        errs.append(np.abs(s - exact).max())
    assert all(a > b for a, b in zip(errs, errs[1:]))
    # 8 bits: error dominated by the fp16 norm and the fp16 centroid rounding
    assert errs[-1] < 0.02 * np.abs(exact).max()
