"""GPU parity of the wide-code path (MSE code widths 5..8, any d) against the
oracle, through the C ABI: quantize, scores, dequantize, decode attention and
the decode step, including mixed key/value widths (one side narrow, the other
wide) and the 8-bit key / 4-bit value split."""
import numpy as np
import pytest
import torch

import oracle
import synth

from parity import TOL, check_close, check_quantize

pytestmark = pytest.mark.gpu
DEV = "cuda"


def tqmod():
    import kv_cache_vector_03_amd as tq
    return tq


def pair(d, bits, m, role_diag=synth.ROLE_DIAG_K, seed=7):
    tq = tqmod()
    diag = synth.diag_signs(seed, role_diag, d)
    S = synth.proj_matrix_f16(seed, synth.ROLE_PROJ_K, d, d) if m else None
    return tq.Quantizer(d, bits, m, diag, S, DEV), oracle.Quantizer(d, bits, m, diag, S)


def opacked(qo, host):
    c, s, n, r = host
    if qo.m == 0:
        s, r = np.zeros((c.shape[0], 0), np.uint32), np.zeros(c.shape[0], np.uint16)
    return oracle.Packed(c, s, n, r)


def gpu_quantize(qg, x_host):
    tq = tqmod()
    p = tq.Packed.empty(qg, x_host.shape[0], DEV)
    tq.tq_quantize(qg, torch.from_numpy(np.ascontiguousarray(x_host)).to(DEV), p)
    torch.cuda.synchronize()
    return p


QCASES = [(64, 5, 64), (64, 8, 0), (128, 5, 128), (128, 6, 0), (128, 7, 128), (128, 8, 0), (256, 6, 256),
          (256, 8, 256)]


@pytest.mark.parametrize("d,bits,m", QCASES)
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_wide_quantize_parity(d, bits, m, dtype):
    qg, qo = pair(d, bits, m)
    n = 257 + 3   # several blocks of four vectors and a ragged tail
    x = (synth.normals(51, synth.ROLE_DATA_K, np.arange(n * d)).reshape(n, d) * 2.0).astype(np.float32)
    x = x.astype(dtype)
    check_quantize(qo, x.astype(np.float64), gpu_quantize(qg, x).to_host())


@pytest.mark.parametrize("d,bits,m", [(64, 6, 64), (128, 7, 128), (128, 8, 0), (256, 5, 256)])
@pytest.mark.parametrize("n_q,n_keys", [(1, 1), (19, 600)])
def test_wide_scores_parity(d, bits, m, n_q, n_keys):
    tq = tqmod()
    qg, qo = pair(d, bits, m)
    x = synth.to_f16(synth.normals(53, synth.ROLE_DATA_K, np.arange(n_keys * d)).reshape(n_keys, d) * 2.0)
    q = synth.to_f16(synth.normals(53, synth.ROLE_QUERY, np.arange(n_q * d)).reshape(n_q, d))
    qd = torch.from_numpy(q).to(DEV)
    p = gpu_quantize(qg, x)
    sc = torch.empty((n_q, n_keys), dtype=torch.float32, device=DEV)
    tq.tq_scores(qg, p, n_keys, qd, sc)
    torch.cuda.synchronize()
    check_close(sc.cpu().numpy(), oracle.scores(qo, opacked(qo, p.to_host()), q.astype(np.float64)),
                what="wide scores on GPU-packed keys")
    # oracle-packed keys into the GPU score kernel
    ref = oracle.quantize(qo, x.astype(np.float64))
    po = tq.Packed.from_host(ref.codes, ref.signs if m else None, ref.norm, ref.rnorm if m else None, DEV)
    tq.tq_scores(qg, po, n_keys, qd, sc)
    torch.cuda.synchronize()
    check_close(sc.cpu().numpy(), oracle.scores(qo, ref, q.astype(np.float64)), what="wide scores, oracle-packed")


@pytest.mark.parametrize("d,bits,m", [(64, 5, 64), (128, 8, 128), (256, 7, 0)])
@pytest.mark.parametrize("include_qjl", [True, False])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16])
def test_wide_dequantize_parity(d, bits, m, include_qjl, out_dtype):
    tq = tqmod()
    qg, qo = pair(d, bits, m)
    n = 131
    x = synth.normals(55, synth.ROLE_DATA_K, np.arange(n * d)).reshape(n, d).astype(np.float32) * 2
    p = gpu_quantize(qg, x)
    out = torch.empty((n, d), dtype=out_dtype, device=DEV)
    tq.tq_dequantize(qg, p, n, include_qjl, out)
    torch.cuda.synchronize()
    ref = oracle.dequantize(qo, opacked(qo, p.to_host()), include_qjl=include_qjl)
    tol = TOL if out_dtype == torch.float32 else 2.0 ** -11 * np.abs(ref).max() + TOL
    check_close(out.float().cpu().numpy(), ref, tol=tol, what="wide dequantize")


DCASES = [
    # d, key mse bits, key QJL, value bits, streams, tokens, G
    # MFMA kernel (d = 128, G <= 8, values of 3, 4 or 8 bits with any keys)
    (128, 7, True, 4, 2, 700, 8),     # 8-bit keys (7 + QJL), 4-bit values
    (128, 7, True, 3, 3, 1300, 8),    # 8-bit keys (7 + QJL), 3-bit values
    (128, 5, False, 3, 2, 333, 4),
    (128, 2, True, 8, 2, 300, 8),     # narrow keys, 8-bit values
    (128, 8, True, 8, 2, 2100, 8),    # 8-bit codes + QJL keys, 8-bit values, several steps per wave
    (128, 5, False, 4, 3, 257, 3),
    (128, 6, True, 8, 1, 4100, 8),
    # scalar wide kernel (other widths, G > 8, other d)
    (128, 6, True, 6, 2, 300, 8),
    (128, 8, False, 8, 1, 513, 16),   # 8-bit codes-only keys and values, G = 16
    (64, 5, True, 6, 3, 257, 4),
    (256, 6, True, 3, 2, 256, 5),
]


def _decode_case(d, kb, k_qjl, vb, ns, T, G):
    tq = tqmod()
    qkg, qko = pair(d, kb, d if k_qjl else 0)
    qvg, qvo = pair(d, vb, 0, role_diag=synth.ROLE_DIAG_V)
    K = synth.to_f16(synth.normals(57, synth.ROLE_DATA_K, np.arange(ns * T * d)).reshape(ns * T, d) * 2)
    V = synth.to_f16(synth.normals(57, synth.ROLE_DATA_V, np.arange(ns * T * d)).reshape(ns * T, d))
    Q = synth.to_f16(synth.normals(57, synth.ROLE_QUERY, np.arange(ns * G * d)).reshape(ns, G, d))
    return tq, qkg, qko, qvg, qvo, K, V, Q


@pytest.mark.parametrize("d,kb,k_qjl,vb,ns,T,G", DCASES)
def test_wide_decode_parity(d, kb, k_qjl, vb, ns, T, G):
    tq, qkg, qko, qvg, qvo, K, V, Q = _decode_case(d, kb, k_qjl, vb, ns, T, G)
    pk, pv = gpu_quantize(qkg, K), gpu_quantize(qvg, V)
    out = torch.empty((ns, G, d), dtype=torch.float32, device=DEV)
    tq.tq_decode_attn(qkg, qvg, pk, pv, ns, T, G, torch.from_numpy(Q).to(DEV), out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn(qko, qvo, opacked(qko, pk.to_host()), opacked(qvo, pv.to_host()), ns, T, G,
                             Q.astype(np.float64))
    check_close(out.cpu().numpy(), ref, what="wide decode")


@pytest.mark.parametrize("d,kb,k_qjl,vb,ns,T,G", [(128, 7, True, 4, 2, 300, 8), (64, 3, True, 8, 2, 130, 8)])
def test_wide_decode_step(d, kb, k_qjl, vb, ns, T, G):
    tq, qkg, qko, qvg, qvo, K, V, Q = _decode_case(d, kb, k_qjl, vb, ns, T + 1, G)
    cap = T + 6  # even: every stream's slice of a 24-byte code row stays 16-byte aligned
    pk, pv = tq.Packed.empty(qkg, ns * cap, DEV), tq.Packed.empty(qvg, ns * cap, DEV)
    K3, V3 = K.reshape(ns, T + 1, d), V.reshape(ns, T + 1, d)
    for st in range(ns):
        sl = slice(st * cap, st * cap + T)
        for qg, pkd, X in ((qkg, pk, K3), (qvg, pv, V3)):
            sub = tq.Packed(pkd.codes[sl], pkd.signs[sl] if pkd.signs is not None else None, pkd.norm[sl],
                            pkd.rnorm[sl] if pkd.rnorm is not None else None)
            tq.tq_quantize(qg, torch.from_numpy(np.ascontiguousarray(X[st, :T])).to(DEV), sub)
    out = torch.empty((ns, G, d), dtype=torch.float32, device=DEV)
    kn = np.ascontiguousarray(K3[:, T])
    vn = np.ascontiguousarray(V3[:, T])
    tq.tq_decode_step(qkg, qvg, pk, pv, ns, T, cap, G, torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV),
                      torch.from_numpy(Q).to(DEV), out)
    torch.cuda.synchronize()
    hk, hv = pk.to_host(), pv.to_host()
    slots = np.arange(ns) * cap + T
    check_quantize(qko, kn.astype(np.float64), tuple(a[slots] for a in hk))
    check_quantize(qvo, vn.astype(np.float64), tuple(a[slots] for a in hv))
    rows = (np.arange(ns)[:, None] * cap + np.arange(T + 1)[None, :]).reshape(-1)
    ref = oracle.decode_attn(qko, qvo, opacked(qko, tuple(a[rows] for a in hk)),
                             opacked(qvo, tuple(a[rows] for a in hv)), ns, T + 1, G, Q.astype(np.float64))
    check_close(out.cpu().numpy(), ref, what="wide decode step")
