"""Whole-set parity of a quantized tensor against the method's definitions.

For sets too large for the oracle to recompute vector by vector, every vector
is checked in fp64 on the device with plain torch operations that restate the
definitions (the rotation, the code rule, the sketch); nothing is shared with
the kernels, and the limits are the parity rules of parity.py.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import parity


def _hadamard(d, dev):
    """Natural-order (Sylvester) H_d in fp64: H_ij = (-1)^popcount(i & j)."""
    h = torch.ones((1, 1), dtype=torch.float64, device=dev)
    while h.shape[0] < d:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    return h


def _unpack_fields(words, n_groups, width):
    """[n, n_groups * 8] values from group-major fields: group c (bytes
    width c .. width c + width - 1) holds member t at bit width t; member t of
    group c is element c + n_groups t."""
    b = words.contiguous().view(torch.uint8).reshape(-1, n_groups, width).to(torch.int64)
    f = torch.zeros(b.shape[:2], dtype=torch.int64, device=b.device)
    for k in range(width):
        f |= b[:, :, k] << (8 * k)
    sh = torch.arange(8, device=b.device, dtype=torch.int64) * width
    v = (f[:, :, None] >> sh) & ((1 << width) - 1)          # [n, group, member]
    return v.permute(0, 2, 1).reshape(-1, n_groups * 8)


def check_full_set(qo, x, p, chunk=1 << 18):
    """Every vector of a quantized set against the method's definitions, in
    fp64 on the device (plain torch operations, nothing shared with the
    kernels): y = H (D x / ||x||) / sqrt(d); code = #{boundaries < y}, equal
    except where y lies within 1e-5 of a boundary (one level, at most 1e-5 of
    the coordinates); with the sketch, r = y - c[GPU code], u = S r and the
    sign bit [u >= 0], equal except where |u| < 1e-5; norms and residual
    norms within one fp16 ulp of the fp16 rounding of ||x|| and ||r||."""
    d, B, m = qo.d, qo.bits, qo.m
    dev = x.device
    H = _hadamard(d, dev) / math.sqrt(d)
    lane = torch.arange(d, device=dev)
    dw = torch.from_numpy(qo.diag.astype(np.int64)).to(dev)
    dsign = 1.0 - 2.0 * ((dw[lane >> 5] >> (lane & 31)) & 1).to(torch.float64)
    bnd = torch.from_numpy(qo.cb.boundaries.astype(np.float64)).to(dev)
    cent = torch.from_numpy(qo.cent.astype(np.float64)).to(dev)
    S = torch.from_numpy(qo.S.view(np.float16).astype(np.float64).reshape(m, d)).to(dev) if m else None
    n = x.shape[0]
    bad_total = 0
    for a in range(0, n, chunk):
        xs = x[a:a + chunk].to(torch.float64)
        nrm = torch.linalg.vector_norm(xs, dim=1)
        y = ((xs * dsign) / nrm[:, None]) @ H.T
        ref = torch.bucketize(y, bnd)                       # boundaries strictly below y
        got = _unpack_fields(p.codes[a:a + chunk], d // 8, B)
        bad = got != ref
        if bool(bad.any()):
            near = (y[..., None] - bnd).abs().min(dim=-1).values < parity.WINDOW
            assert bool(near[bad].all()), "code mismatch outside the boundary window"
            assert bool(((got - ref).abs()[bad] == 1).all()), "code mismatch by more than one level"
            bad_total += int(bad.sum())
        gn = p.norm[a:a + chunk].view(torch.float16).to(torch.float64)
        ulp = (gn.abs().clamp_min(2.0 ** -14).log2().floor() - 10).exp2()
        # one ulp from the exact value's fp16 rounding: at most 1.5 ulp from the exact value
        assert bool(((gn - nrm).abs() <= 1.5 * ulp).all()), "norm beyond 1 fp16 ulp"
        if m:
            r = y - cent[got]
            u = r @ S.T
            gs = _unpack_fields(p.signs[a:a + chunk], m // 8, 1)
            sbad = gs != (u >= 0).to(torch.int64)
            assert bool((u.abs()[sbad.bool()] < parity.WINDOW).all()), "sign mismatch outside |u| < 1e-5"
            gr = p.rnorm[a:a + chunk].view(torch.float16).to(torch.float64)
            rn = torch.linalg.vector_norm(r, dim=1)
            ulp = (gr.abs().clamp_min(2.0 ** -14).log2().floor() - 10).exp2()
            assert bool(((gr - rn).abs() <= 1.5 * ulp).all()), "residual norm beyond 1 fp16 ulp"
    allowed = max(1, math.ceil(parity.WINDOW * n * d))
    assert bad_total <= allowed, f"{bad_total} code mismatches > {allowed}"
    return bad_total


def scores_reference(qo, p, q, rows=None):
    """The estimator s = n (<q', c[code]> + gamma sqrt(pi/2)/m <S q', 2 sign - 1>)
    with q' = H (D q) / sqrt(d), in fp64 on the device, for packed keys p and
    queries q [n_q, d] (all rows, or the slice `rows`)."""
    d, B, m = qo.d, qo.bits, qo.m
    dev = q.device
    H = _hadamard(d, dev) / math.sqrt(d)
    lane = torch.arange(d, device=dev)
    dw = torch.from_numpy(qo.diag.astype(np.int64)).to(dev)
    dsign = 1.0 - 2.0 * ((dw[lane >> 5] >> (lane & 31)) & 1).to(torch.float64)
    cent = torch.from_numpy(qo.cent.astype(np.float64)).to(dev)
    n = p.norm.view(torch.float16).to(torch.float64)
    kv = n[:, None] * cent[_unpack_fields(p.codes, d // 8, B)]      # n c, rotated domain
    qs = q if rows is None else q[rows]
    qr = (qs.to(torch.float64) * dsign) @ H.T
    out = qr @ kv.T
    if m:
        S = torch.from_numpy(qo.S.view(np.float16).astype(np.float64).reshape(m, d)).to(dev)
        sg = 2.0 * _unpack_fields(p.signs, m // 8, 1).to(torch.float64) - 1.0
        g = n * p.rnorm.view(torch.float16).to(torch.float64) * (math.sqrt(math.pi / 2.0) / m)
        out += (qr @ S.T) @ (sg * g[:, None]).T
    return out


def check_scores_full(qo, p, q, sc, tol=parity.TOL, chunk=256):
    """Every score of sc [n_q, n_keys] against scores_reference, within tol."""
    worst = 0.0
    for a in range(0, q.shape[0], chunk):
        rows = torch.arange(a, min(a + chunk, q.shape[0]), device=q.device)
        err = float((sc[rows].to(torch.float64) - scores_reference(qo, p, q, rows)).abs().max())
        assert err <= tol, f"scores rows {a}..: max abs error {err:.3e} > {tol:.1e}"
        worst = max(worst, err)
    return worst
