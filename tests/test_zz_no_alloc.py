"""tq_decode_attn_noalloc through the C ABI against tq_decode_attn (caller
workspace) on the same packed caches: two calls in a row on the library's fixed
scratch, the second with a smaller input, for the MFMA kernel (d = 128) and
the scalar kernels (d = 64). Outputs must equal the workspace entry point's
(same kernels and work split) and the oracle's within 1e-4."""
import numpy as np
import pytest
import torch

import oracle
import synth

from parity import check_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(d, kb, vb, ns, T, G, seed):
    import kv_cache_vector_03_amd as tq
    diag_k = synth.diag_signs(seed, synth.ROLE_DIAG_K, d)
    diag_v = synth.diag_signs(seed, synth.ROLE_DIAG_V, d)
    S = synth.proj_matrix_f16(seed, synth.ROLE_PROJ_K, d, d)
    qkg, qvg = tq.Quantizer(d, kb, d, diag_k, S, DEV), tq.Quantizer(d, vb, 0, diag_v, None, DEV)
    qko, qvo = oracle.Quantizer(d, kb, d, diag_k, S), oracle.Quantizer(d, vb, 0, diag_v, None)
    K = synth.to_f16(synth.normals(seed, synth.ROLE_DATA_K, np.arange(ns * T * d)).reshape(ns * T, d) * 2)
    V = synth.to_f16(synth.normals(seed, synth.ROLE_DATA_V, np.arange(ns * T * d)).reshape(ns * T, d))
    Q = synth.to_f16(synth.normals(seed, synth.ROLE_QUERY, np.arange(ns * G * d)).reshape(ns, G, d))
    pk, pv = tq.Packed.empty(qkg, ns * T, DEV), tq.Packed.empty(qvg, ns * T, DEV)
    tq.tq_quantize(qkg, torch.from_numpy(K).to(DEV), pk)
    tq.tq_quantize(qvg, torch.from_numpy(V).to(DEV), pv)
    q = torch.from_numpy(Q).to(DEV)
    out_ws = torch.empty((ns, G, d), dtype=torch.float32, device=DEV)
    tq.tq_decode_attn(qkg, qvg, pk, pv, ns, T, G, q, out_ws)
    out_na = torch.full((ns, G, d), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_decode_attn_noalloc(qkg, qvg, pk, pv, ns, T, G, q, out_na)
    torch.cuda.synchronize()
    hk, hv = pk.to_host(), pv.to_host()
    ref = oracle.decode_attn(qko, qvo, oracle.Packed(*hk),
                             oracle.Packed(hv[0], np.zeros((ns * T, 0), np.uint32), hv[2], np.zeros(ns * T, np.uint16)),
                             ns, T, G, Q.astype(np.float64))
    a, b = out_na.cpu().numpy(), out_ws.cpu().numpy()
    assert np.array_equal(a, b), float(np.nanmax(np.abs(a - b)))
    err = check_close(a, ref, what=f"noalloc d={d} ns={ns} T={T}")
    print(f"noalloc d={d} kb={kb} vb={vb} ns={ns} T={T} G={G}: equal to the workspace call; max |err| {err:.2e}")


@pytest.mark.parametrize("d,kb,vb,G", [(128, 2, 4, 8), (64, 2, 3, 8)])
def test_noalloc_decode_two_calls(d, kb, vb, G):
    _case(d, kb, vb, ns=12, T=3001, G=G, seed=71)
    _case(d, kb, vb, ns=3, T=257, G=G, seed=72)   # smaller: the scratch keeps the last call's contents
