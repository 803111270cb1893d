"""GPU parity of the fused decode attention against the oracle (through the C ABI).

Small cases cover ragged token counts around the chunk size, every supported
head-group size range, all d and bit widths. The 8K-model and 128K-layer
workloads run at full size in the same launch configuration the
benchmark times; the oracle recomputes sampled streams one by one, both on
the GPU's packed cache and on an oracle-packed copy of the stream.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W

from full_set import check_full_set
from parity import check_close, check_quantize

pytestmark = pytest.mark.gpu
DEV = "cuda"


def tqmod():
    import kv_cache_vector_03_amd as tq
    return tq


def make(d, kb, vb, seed=7, k_qjl=True):
    tq = tqmod()
    diag_k = synth.diag_signs(seed, synth.ROLE_DIAG_K, d)
    diag_v = synth.diag_signs(seed, synth.ROLE_DIAG_V, d)
    S = synth.proj_matrix_f16(seed, synth.ROLE_PROJ_K, d, d)
    m = d if k_qjl else 0
    return (tq.Quantizer(d, kb, m, diag_k, S if m else None, DEV), tq.Quantizer(d, vb, 0, diag_v, None, DEV),
            oracle.Quantizer(d, kb, m, diag_k, S if m else None), oracle.Quantizer(d, vb, 0, diag_v, None))


def opacked(qo, host):
    c, s, n, r = host
    if qo.m == 0:
        s, r = np.zeros((c.shape[0], 0), np.uint32), np.zeros(c.shape[0], np.uint16)
    return oracle.Packed(c, s, n, r)


def run_decode(qkg, qvg, pk, pv, ns, T, G, q, scale=0.0):
    tq = tqmod()
    out = torch.empty((ns, G, qkg.d), dtype=torch.float32, device=DEV)
    tq.tq_decode_attn(qkg, qvg, pk, pv, ns, T, G, q, out, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SMALL = [
    # d, kb, vb, ns, T, G, k_qjl
    (128, 2, 3, 2, 1, 8, True),
    (128, 2, 3, 3, 255, 8, True),
    (128, 2, 3, 2, 256, 8, True),
    (128, 2, 3, 2, 257, 8, True),
    (128, 2, 4, 1, 1000, 16, True),
    (128, 3, 3, 2, 700, 1, True),
    (128, 2, 2, 2, 513, 4, False),
    (64, 2, 3, 3, 600, 8, True),
    (256, 2, 4, 2, 300, 5, True),
    (256, 1, 1, 1, 260, 2, True),
    # the scalar kernel's largest LDS footprint: d = 256, sketch keys, G = 16
    (256, 2, 4, 2, 300, 16, True),
    # more streams than the 512 block slots: several chunks per stream chosen to fill
    # whole rounds of blocks
    (128, 2, 4, 600, 130, 8, True),
    (128, 2, 4, 640, 600, 8, True),
    # one long stream split into many chunks
    (128, 2, 3, 1, 70000, 8, True),
]


@pytest.mark.parametrize("d,kb,vb,ns,T,G,k_qjl", SMALL)
def test_decode_small(d, kb, vb, ns, T, G, k_qjl):
    tq = tqmod()
    qkg, qvg, qko, qvo = make(d, kb, vb, k_qjl=k_qjl)
    K = synth.to_f16(synth.normals(31, synth.ROLE_DATA_K, np.arange(ns * T * d)).reshape(ns * T, d) * 2)
    V = synth.to_f16(synth.normals(31, synth.ROLE_DATA_V, np.arange(ns * T * d)).reshape(ns * T, d))
    Q = synth.to_f16(synth.normals(31, synth.ROLE_QUERY, np.arange(ns * G * d)).reshape(ns, G, d))
    pk, pv = tq.Packed.empty(qkg, ns * T, DEV), tq.Packed.empty(qvg, ns * T, DEV)
    tq.tq_quantize(qkg, torch.from_numpy(K).to(DEV), pk)
    tq.tq_quantize(qvg, torch.from_numpy(V).to(DEV), pv)
    qd = torch.from_numpy(Q).to(DEV)
    out = run_decode(qkg, qvg, pk, pv, ns, T, G, qd)
    ref = oracle.decode_attn(qko, qvo, opacked(qko, pk.to_host()), opacked(qvo, pv.to_host()), ns, T, G,
                             Q.astype(np.float64))
    check_close(out, ref, what="decode on GPU-packed cache")
    # oracle-packed cache into the GPU kernel
    rk = oracle.quantize(qko, K.astype(np.float64))
    rv = oracle.quantize(qvo, V.astype(np.float64))
    pk2 = tq.Packed.from_host(rk.codes, rk.signs if k_qjl else None, rk.norm, rk.rnorm, DEV)
    pv2 = tq.Packed.from_host(rv.codes, None, rv.norm, None, DEV)
    out2 = run_decode(qkg, qvg, pk2, pv2, ns, T, G, qd)
    check_close(out2, oracle.decode_attn(qko, qvo, rk, rv, ns, T, G, Q.astype(np.float64)),
                what="decode on oracle-packed cache")
    # explicit scale, and run-to-run determinism
    out3 = run_decode(qkg, qvg, pk, pv, ns, T, G, qd, scale=0.03)
    check_close(out3, oracle.decode_attn(qko, qvo, opacked(qko, pk.to_host()), opacked(qvo, pv.to_host()),
                                         ns, T, G, Q.astype(np.float64), scale=0.03))
    assert np.array_equal(out, run_decode(qkg, qvg, pk, pv, ns, T, G, qd))


def test_decode_zero_and_large_norm_tokens():
    """Zero vectors (n = 0) and tokens with norms near 10^4 in the same
    stream: the weight scaling must keep every product in fp16 range."""
    tq = tqmod()
    d, ns, T, G = 128, 2, 700, 8
    qkg, qvg, qko, qvo = make(d, 2, 4)
    K = synth.normals(41, synth.ROLE_DATA_K, np.arange(ns * T * d)).reshape(ns * T, d)
    V = synth.normals(41, synth.ROLE_DATA_V, np.arange(ns * T * d)).reshape(ns * T, d)
    K[::7] = 0.0
    V[::11] = 0.0
    V[5::13] *= 900.0   # ||v|| ~ 1e4
    K[3::17] *= 3.0
    K, V = synth.to_f16(K), synth.to_f16(V)
    Q = synth.to_f16(synth.normals(41, synth.ROLE_QUERY, np.arange(ns * G * d)).reshape(ns, G, d) * 0.5)
    pk, pv = tq.Packed.empty(qkg, ns * T, DEV), tq.Packed.empty(qvg, ns * T, DEV)
    tq.tq_quantize(qkg, torch.from_numpy(K).to(DEV), pk)
    tq.tq_quantize(qvg, torch.from_numpy(V).to(DEV), pv)
    out = run_decode(qkg, qvg, pk, pv, ns, T, G, torch.from_numpy(Q).to(DEV))
    ref = oracle.decode_attn(qko, qvo, opacked(qko, pk.to_host()), opacked(qvo, pv.to_host()), ns, T, G,
                             Q.astype(np.float64))
    # the contract's 1e-4 absolute bound, also with these norms
    err = check_close(out, ref, what="zero / large-norm tokens")
    print(f"zero / large-norm tokens: max |out - oracle| {err:.3e} at output scale {float(np.abs(ref).max()):.3e}")


STEP = [
    # d, kb, vb, ns, T, cap, G, k_qjl, new-token dtype
    (128, 2, 4, 3, 300, 320, 8, True, np.float16),   # MFMA path: the append inside the decode kernel
    (128, 2, 3, 2, 0, 4, 8, True, np.float32),       # empty caches: attend over the new token only
    (128, 3, 3, 2, 1000, 1001, 4, False, np.float16),  # last slot; codes-only keys
    (128, 2, 4, 2, 2047, 4096, 8, True, np.float16),  # T + 1 = 2048: full steps only
    (128, 6, 8, 2, 500, 640, 8, True, np.float32),   # 6-bit keys, 8-bit values: codes by binary search
    (128, 2, 4, 8, 20000, 20480, 8, True, np.float16),  # 8 streams, many blocks per stream
    (128, 1, 2, 5, 129, 200, 3, True, np.float16),   # 1-bit keys, 2-bit values, G = 3
    (64, 2, 3, 2, 200, 260, 8, True, np.float32),    # d = 64: separate append kernel
    (128, 2, 4, 2, 130, 200, 16, True, np.float16),  # G = 16: separate append kernel
]


@pytest.mark.parametrize("d,kb,vb,ns,T,cap,G,k_qjl,dt", STEP)
def test_decode_step_append(d, kb, vb, ns, T, cap, G, k_qjl, dt):
    """tq_decode_step: the new token of each stream is quantized into slot T of
    a cache with `cap` slots per stream, nothing else in the caches changes,
    and the output is the attention over tokens 0..T."""
    tq = tqmod()
    qkg, qvg, qko, qvo = make(d, kb, vb, k_qjl=k_qjl)
    K = synth.to_f16(synth.normals(37, synth.ROLE_DATA_K, np.arange(ns * cap * d)).reshape(ns, cap, d) * 2)
    V = synth.to_f16(synth.normals(37, synth.ROLE_DATA_V, np.arange(ns * cap * d)).reshape(ns, cap, d))
    Q = synth.to_f16(synth.normals(37, synth.ROLE_QUERY, np.arange(ns * G * d)).reshape(ns, G, d))
    kn = (synth.normals(41, synth.ROLE_DATA_K, np.arange(ns * d)).reshape(ns, d) * 2).astype(dt)
    vn = synth.normals(41, synth.ROLE_DATA_V, np.arange(ns * d)).reshape(ns, d).astype(dt)
    pk, pv = tq.Packed.empty(qkg, ns * cap, DEV), tq.Packed.empty(qvg, ns * cap, DEV)
    for t in [a for a in (pk.codes, pk.signs, pk.norm, pk.rnorm, pv.codes, pv.norm) if a is not None]:
        t.fill_(-1)
    # the caches: tokens 0..T-1 of stream s at slots s*cap + t
    for st in range(ns):
        if T == 0:
            break
        sl = slice(st * cap, st * cap + T)
        for qg, pkd, X in ((qkg, pk, K), (qvg, pv, V)):
            sub = tq.Packed(pkd.codes[sl], pkd.signs[sl] if pkd.signs is not None else None, pkd.norm[sl],
                            pkd.rnorm[sl] if pkd.rnorm is not None else None)
            tq.tq_quantize(qg, torch.from_numpy(np.ascontiguousarray(X[st, :T])).to(DEV), sub)
    torch.cuda.synchronize()
    before_k, before_v = pk.to_host(), pv.to_host()
    out = torch.empty((ns, G, d), dtype=torch.float32, device=DEV)
    tq.tq_decode_step(qkg, qvg, pk, pv, ns, T, cap, G, torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV),
                      torch.from_numpy(Q).to(DEV), out)
    torch.cuda.synchronize()
    after_k, after_v = pk.to_host(), pv.to_host()
    slots = np.arange(ns) * cap + T
    keep = np.ones(ns * cap, bool)
    keep[slots] = False
    for b, a in zip(before_k + before_v, after_k + after_v):
        if a is not None and a.size:
            assert np.array_equal(b[keep], a[keep]), "cache changed outside the appended slots"
    # the appended tokens against the oracle's quantizer
    check_quantize(qko, kn.astype(np.float64), tuple(a[slots] for a in after_k))
    check_quantize(qvo, vn.astype(np.float64), tuple(a[slots] for a in after_v))
    # attention over tokens 0..T of each stream, on the cache as the GPU left it
    rows = (np.arange(ns)[:, None] * cap + np.arange(T + 1)[None, :]).reshape(-1)
    gk = opacked(qko, tuple(a[rows] for a in after_k))
    gv = opacked(qvo, tuple(a[rows] for a in after_v))
    ref = oracle.decode_attn(qko, qvo, gk, gv, ns, T + 1, G, Q.astype(np.float64))
    check_close(out.cpu().numpy(), ref, what="decode step after append")


def test_decode_step_argument_errors():
    tq = tqmod()
    qkg, qvg, _, _ = make(128, 2, 4)
    pk, pv = tq.Packed.empty(qkg, 8, DEV), tq.Packed.empty(qvg, 8, DEV)
    z = torch.zeros((2, 128), dtype=torch.float16, device=DEV)
    q = torch.zeros((2, 8, 128), dtype=torch.float16, device=DEV)
    out = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
    for T, cap in ((4, 4), (-1, 4)):
        with pytest.raises(tq.TQError):
            tq.tq_decode_step(qkg, qvg, pk, pv, 2, T, cap, 8, z, z, q, out)


def test_decode_with_exact_law_codebooks():
    """Quantize and decode with codebooks solved for the exact coordinate law
    (keys 2 + 1, values 3-bit); the oracle uses the same codebooks."""
    tq = tqmod()
    d, ns, T, G = 128, 3, 777, 8
    diag_k = synth.diag_signs(7, synth.ROLE_DIAG_K, d)
    diag_v = synth.diag_signs(7, synth.ROLE_DIAG_V, d)
    S = synth.proj_matrix_f16(7, synth.ROLE_PROJ_K, d, d)
    qkg = tq.Quantizer(d, 2, d, diag_k, S, DEV, law=tq.TQ_LAW_SPHERE)
    qvg = tq.Quantizer(d, 3, 0, diag_v, None, DEV, law=tq.TQ_LAW_SPHERE)
    qko = oracle.Quantizer(d, 2, d, diag_k, S, cb=oracle.codebook(d, 2, oracle.LAW_SPHERE))
    qvo = oracle.Quantizer(d, 3, 0, diag_v, None, cb=oracle.codebook(d, 3, oracle.LAW_SPHERE))
    K = synth.to_f16(synth.normals(43, synth.ROLE_DATA_K, np.arange(ns * T * d)).reshape(ns * T, d) * 2)
    V = synth.to_f16(synth.normals(43, synth.ROLE_DATA_V, np.arange(ns * T * d)).reshape(ns * T, d))
    Q = synth.to_f16(synth.normals(43, synth.ROLE_QUERY, np.arange(ns * G * d)).reshape(ns, G, d))
    pk, pv = tq.Packed.empty(qkg, ns * T, DEV), tq.Packed.empty(qvg, ns * T, DEV)
    tq.tq_quantize(qkg, torch.from_numpy(K).to(DEV), pk)
    tq.tq_quantize(qvg, torch.from_numpy(V).to(DEV), pv)
    hk, hv = pk.to_host(), pv.to_host()
    check_quantize(qko, K.astype(np.float64), hk)
    check_quantize(qvo, V.astype(np.float64), hv)
    out = run_decode(qkg, qvg, pk, pv, ns, T, G, torch.from_numpy(Q).to(DEV))
    check_close(out, oracle.decode_attn(qko, qvo, opacked(qko, hk), opacked(qvo, hv), ns, T, G,
                                        Q.astype(np.float64)), what="exact-law codebooks")


def _runs(heads):
    """Consecutive runs [h0, h1) of a sorted list of heads."""
    out, h0 = [], heads[0]
    for a, b in zip(heads, heads[1:] + [None]):
        if b != a + 1:
            out.append((h0, a + 1))
            h0 = b
    return out


def _kv_case(cfg, layers, sample):
    """Generate, quantize and decode ``layers`` of cfg on the GPU; every quantized
    vector is checked against the definitions (check_full_set), and sampled
    streams against the oracle.

    sample: list of (layer, head) streams recomputed by the oracle."""
    tq = tqmod()
    d = cfg.d
    diag_k, S, diag_v = W.quantizer_inputs(d)
    qkg = tq.Quantizer(d, cfg.k_mse_bits, d, diag_k, S, DEV)
    qvg = tq.Quantizer(d, cfg.v_bits, 0, diag_v, None, DEV)
    qko = oracle.Quantizer(d, cfg.k_mse_bits, d, diag_k, S)
    qvo = oracle.Quantizer(d, cfg.v_bits, 0, diag_v, None)
    nl = len(layers)
    per_layer = cfg.kv_heads * cfg.tokens
    pk, pv = tq.Packed.empty(qkg, nl * per_layer, DEV), tq.Packed.empty(qvg, nl * per_layer, DEV)
    kbuf = torch.empty((per_layer, d), dtype=torch.float16, device=DEV)
    from synth import gpu
    q_all = []
    for li, layer in enumerate(layers):
        for role, qg, pkd in ((synth.ROLE_DATA_K, qkg, pk), (synth.ROLE_DATA_V, qvg, pv)):
            sc = gpu.scales_to_device(W.kv_seed_scales(cfg, layer, role), DEV)
            W.kv_layer_device(cfg, layer, role, kbuf, sc)
            sub = tq.Packed(pkd.codes[li * per_layer:(li + 1) * per_layer],
                            pkd.signs[li * per_layer:(li + 1) * per_layer] if pkd.signs is not None else None,
                            pkd.norm[li * per_layer:(li + 1) * per_layer],
                            pkd.rnorm[li * per_layer:(li + 1) * per_layer] if pkd.rnorm is not None else None)
            tq.tq_quantize(qg, kbuf, sub)
            # every vector of the layer's K (or V) against the definitions
            check_full_set(qko if role == synth.ROLE_DATA_K else qvo, kbuf, sub)
        q_all.append(W.kv_queries_host(cfg, layer))
    Q = np.stack(q_all).reshape(nl * cfg.kv_heads, cfg.G, d)
    ns = nl * cfg.kv_heads
    out = run_decode(qkg, qvg, pk, pv, ns, cfg.tokens, cfg.G, torch.from_numpy(Q).to(DEV))
    host_k, host_v = pk.to_host(), pv.to_host()
    T = cfg.tokens
    worst = 0.0
    # the sampled streams of each layer are decoded by the oracle in one call
    # (consecutive heads are consecutive streams of the packed caches)
    for layer in sorted({l for l, _ in sample}):
        heads = sorted(h for l, h in sample if l == layer)
        li = layers.index(layer)
        for h0, h1 in _runs(heads):
            s0, s1 = li * cfg.kv_heads + h0, li * cfg.kv_heads + h1
            sl = slice(s0 * T, s1 * T)
            gk = oracle.Packed(*(a[sl] for a in host_k))
            gv = oracle.Packed(host_v[0][sl], np.zeros((s1 * T - s0 * T, 0), np.uint32), host_v[2][sl],
                               np.zeros(s1 * T - s0 * T, np.uint16))
            ref = oracle.decode_attn(qko, qvo, gk, gv, s1 - s0, T, cfg.G, Q[s0:s1].astype(np.float64))
            worst = max(worst, check_close(out[s0:s1], ref, what=f"{cfg.name} layer {layer} heads {h0}..{h1 - 1}"))
        for head in heads:
            s = li * cfg.kv_heads + head
            sl = slice(s * T, (s + 1) * T)
            # quantizer parity on tokens spread over the whole stream (host-drawn inputs)
            toks = np.unique(np.linspace(0, T - 1, 1024).astype(np.int64))
            kx = W.kv_vectors_host(cfg, layer, synth.ROLE_DATA_K, head, toks).astype(np.float64)
            vx = W.kv_vectors_host(cfg, layer, synth.ROLE_DATA_V, head, toks).astype(np.float64)
            check_quantize(qko, kx, tuple(a[sl][toks] for a in host_k))
            check_quantize(qvo, vx, tuple(a[sl][toks] for a in host_v))
    print(f"{cfg.name}: {len(sample)} streams checked, max |out - oracle| {worst:.2e}")
    return qkg, qvg, qko, qvo, Q


def test_kv_8k_full_one_call():
    """All 36 layers in one call; every one of the 72 streams checked."""
    cfg = W.KV_8K
    _kv_case(cfg, list(range(cfg.layers)), [(l, h) for l in range(cfg.layers) for h in range(cfg.kv_heads)])


def test_kv_8k_stream_oracle_packed():
    """One whole 8K stream quantized by the oracle, decoded by the GPU kernel."""
    tq = tqmod()
    cfg = W.KV_8K
    d, T = cfg.d, cfg.tokens
    diag_k, S, diag_v = W.quantizer_inputs(d)
    qkg = tq.Quantizer(d, cfg.k_mse_bits, d, diag_k, S, DEV)
    qvg = tq.Quantizer(d, cfg.v_bits, 0, diag_v, None, DEV)
    qko = oracle.Quantizer(d, cfg.k_mse_bits, d, diag_k, S)
    qvo = oracle.Quantizer(d, cfg.v_bits, 0, diag_v, None)
    layer, head = 9, 1
    toks = np.arange(T)
    rk = oracle.quantize(qko, W.kv_vectors_host(cfg, layer, synth.ROLE_DATA_K, head, toks).astype(np.float64))
    rv = oracle.quantize(qvo, W.kv_vectors_host(cfg, layer, synth.ROLE_DATA_V, head, toks).astype(np.float64))
    Q = W.kv_queries_host(cfg, layer)[head:head + 1]
    out = run_decode(qkg, qvg, tq.Packed.from_host(rk.codes, rk.signs, rk.norm, rk.rnorm, DEV),
                     tq.Packed.from_host(rv.codes, None, rv.norm, None, DEV), 1, T, cfg.G,
                     torch.from_numpy(np.ascontiguousarray(Q)).to(DEV))
    check_close(out, oracle.decode_attn(qko, qvo, rk, rv, 1, T, cfg.G, Q.astype(np.float64)),
                what="8K stream, oracle-packed")


def test_kv_128k_layers_first_and_last():
    """Layers 0 and 79 in one call; all 16 streams checked."""
    cfg = W.KV_128K
    _kv_case(cfg, [0, 79], [(l, h) for l in (0, 79) for h in range(cfg.kv_heads)])


@pytest.mark.parametrize("which", ["128k_layer", "8k_model"])
def test_decode_step_full_size(which):
    """The decode step at full size, in the launch configurations the benchmark
    times: the 128K layer (8 streams, tokens 0..131070 cached and token 131071
    appended; 4-bit values) and the 8K model in one call (all 36 layers, 72
    streams of 8191 cached tokens plus the appended one; 3-bit values). The
    append runs inside the decode kernel, in the first block of each stream.
    The appended slots match the oracle's quantizer, the rest of the caches is
    unchanged, and the attention of the first and last stream over all tokens
    matches the oracle on the cache as the GPU left it."""
    tq = tqmod()
    cfg = W.KV_128K if which == "128k_layer" else W.KV_8K
    layers = [0] if which == "128k_layer" else list(range(cfg.layers))
    d, T, G = cfg.d, cfg.tokens, cfg.G
    H = cfg.kv_heads * len(layers)  # streams of the call
    diag_k, S, diag_v = W.quantizer_inputs(d)
    qkg = tq.Quantizer(d, cfg.k_mse_bits, d, diag_k, S, DEV)
    qvg = tq.Quantizer(d, cfg.v_bits, 0, diag_v, None, DEV)
    qko = oracle.Quantizer(d, cfg.k_mse_bits, d, diag_k, S)
    qvo = oracle.Quantizer(d, cfg.v_bits, 0, diag_v, None)
    from synth import gpu
    per = H * T
    pl = cfg.kv_heads * T  # vectors per layer
    pk, pv = tq.Packed.empty(qkg, per, DEV), tq.Packed.empty(qvg, per, DEV)
    news = []
    for role, qg, pkd in ((synth.ROLE_DATA_K, qkg, pk), (synth.ROLE_DATA_V, qvg, pv)):
        X = torch.empty((per, d), dtype=torch.float16, device=DEV)
        for li, layer in enumerate(layers):
            W.kv_layer_device(cfg, layer, role, X[li * pl:(li + 1) * pl],
                              gpu.scales_to_device(W.kv_seed_scales(cfg, layer, role), DEV))
        tq.tq_quantize(qg, X, pkd)
        news.append(X.view(H, T, d)[:, T - 1].contiguous())
        del X
    # the appended slots start out as garbage, so the step must write them
    slots = np.arange(H) * T + T - 1
    sl_t = torch.from_numpy(slots).to(DEV)
    for a in (pk.codes, pk.signs, pk.norm, pk.rnorm, pv.codes, pv.norm):
        a[sl_t] = -1
    torch.cuda.synchronize()
    before_k, before_v = pk.to_host(), pv.to_host()
    Q = np.stack([W.kv_queries_host(cfg, layer) for layer in layers]).reshape(H, G, d)
    out = torch.empty((H, G, d), dtype=torch.float32, device=DEV)
    tq.tq_decode_step(qkg, qvg, pk, pv, H, T - 1, T, G, news[0], news[1], torch.from_numpy(Q).to(DEV), out)
    torch.cuda.synchronize()
    after_k, after_v = pk.to_host(), pv.to_host()
    keep = np.ones(per, bool)
    keep[slots] = False
    for b, a in zip(before_k + before_v, after_k + after_v):
        if a is not None and a.size:
            assert np.array_equal(b[keep], a[keep]), "cache changed outside the appended slots"
    last = np.array([T - 1])
    sh = [(layer, h) for layer in layers for h in range(cfg.kv_heads)]  # stream -> (layer, head)
    kx = np.concatenate([W.kv_vectors_host(cfg, l, synth.ROLE_DATA_K, h, last) for l, h in sh]).astype(np.float64)
    vx = np.concatenate([W.kv_vectors_host(cfg, l, synth.ROLE_DATA_V, h, last) for l, h in sh]).astype(np.float64)
    check_quantize(qko, kx, tuple(a[slots] for a in after_k))
    check_quantize(qvo, vx, tuple(a[slots] for a in after_v))
    o = out.cpu().numpy()
    worst = 0.0
    for st in (0, H - 1):
        sl = slice(st * T, (st + 1) * T)
        gk = oracle.Packed(*(a[sl] for a in after_k))
        gv = oracle.Packed(after_v[0][sl], np.zeros((T, 0), np.uint32), after_v[2][sl], np.zeros(T, np.uint16))
        ref = oracle.decode_attn(qko, qvo, gk, gv, 1, T, G, Q[st:st + 1].astype(np.float64))
        worst = max(worst, check_close(o[st:st + 1], ref, what=f"decode step, {which} stream {st}"))
    print(f"{which} decode step: appended slots checked, max |out - oracle| {worst:.2e}")
