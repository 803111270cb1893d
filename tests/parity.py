"""Parity rules between the HIP path and the oracle (shared by the GPU tests).

* codes: bit-exact, except coordinates whose oracle value lies within 1e-5 of
  a boundary; those may differ by one adjacent level, on at most 1e-5 of the
  coordinates (rounded up to at least one);
* signs: bit-exact, except rows whose oracle projection |u| < 1e-5. On a
  vector whose codes differ from the oracle's (inside the boundary window),
  the oracle's residual, projection, signs and residual norm are rebuilt from
  the GPU's codes first (one changed code moves u by ~0.1 and flips many
  signs), and the GPU's signs and residual norm are checked against those;
* norm and residual norm: within one fp16 ulp;
* scores and attention outputs: within 1e-4 absolute, on identical packed inputs.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

WINDOW = 1e-5
TOL = 1e-4


def fp16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in units of fp16 spacing, for fp16 bit patterns of equal sign."""
    ia = np.asarray(a, np.uint16).astype(np.int64)
    ib = np.asarray(b, np.uint16).astype(np.int64)
    sa, sb = ia >> 15, ib >> 15
    va = np.where(sa == 1, -(ia & 0x7FFF), ia & 0x7FFF)
    vb = np.where(sb == 1, -(ib & 0x7FFF), ib & 0x7FFF)
    return np.abs(va - vb)


def check_codes(Q: oracle.Quantizer, gpu_codes: np.ndarray, ref_codes: np.ndarray, y: np.ndarray):
    """Returns (n_mismatch_coordinates, vectors_with_mismatch)."""
    gi = oracle.unpack_codes(Q, gpu_codes)
    ri = oracle.unpack_codes(Q, ref_codes)
    bad = gi != ri
    nbad = int(bad.sum())
    if nbad:
        b = Q.cb.boundaries.astype(np.float64)
        dist = np.min(np.abs(y[..., None] - b), axis=-1)
        assert np.all(dist[bad] < WINDOW), "code mismatch outside the boundary window"
        assert np.all(np.abs(gi[bad] - ri[bad]) == 1), "code mismatch by more than one level"
        allowed = max(1, math.ceil(WINDOW * gi.size))
        assert nbad <= allowed, f"{nbad} code mismatches > {allowed}"
    return nbad, np.nonzero(bad.any(axis=1))[0]


def check_signs(Q: oracle.Quantizer, gpu_signs, ref_signs, u):
    gs = oracle.unpack_signs(Q, gpu_signs)
    rs = oracle.unpack_signs(Q, ref_signs)
    bad = gs != rs
    if bad.any():
        assert np.all(np.abs(u[bad]) < WINDOW), "sign mismatch outside |u| < 1e-5"
    return int(bad.sum())


def check_scalars(gpu, ref, what="norm"):
    d = fp16_ulp_diff(gpu, ref)
    assert int(d.max(initial=0)) <= 1, f"{what}: {int(d.max())} fp16 ulp"
    return int((d > 0).sum())


def check_close(gpu: np.ndarray, ref: np.ndarray, tol: float = TOL, what: str = ""):
    err = float(np.max(np.abs(np.asarray(gpu, np.float64) - ref), initial=0.0))
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"
    return err


def check_quantize(Q: oracle.Quantizer, x: np.ndarray, gpu_packed):
    """Full quantizer parity for vectors x (host values) and the GPU's packed output."""
    c, s, n, r = gpu_packed
    res = oracle.quantize(Q, np.asarray(x, np.float64), want_y=True, want_u=bool(Q.m))
    if Q.m:
        ref, y, u = res
    else:
        ref, y = res
        u = None
    nbad, badvec = check_codes(Q, c, ref.codes, y)
    check_scalars(n, ref.norm, "norm")
    sbad = 0
    if Q.m:
        ref_signs, ref_rnorm, ref_u = ref.signs, ref.rnorm, u
        if len(badvec):
            # the oracle's QJL stage on the GPU's codes for those vectors
            ref_signs, ref_rnorm, ref_u = ref_signs.copy(), ref_rnorm.copy(), ref_u.copy()
            s2, r2, u2 = oracle.sketch(Q, y[badvec], np.asarray(c)[badvec], want_u=True)
            ref_signs[badvec], ref_rnorm[badvec], ref_u[badvec] = s2, r2, u2
        sbad = check_signs(Q, s, ref_signs, ref_u)
        check_scalars(r, ref_rnorm, "rnorm")
    return nbad, sbad, ref
