"""The pages' own checks run through the HIP path (tq_quantize, tq_scores).

* Synthetic needle ("[Benchmark] TurboQuant 實測 ...", section
  "Needle-in-Haystack（Synthetic）": EXACT retrieval at seq 512 / 2048 / 8192 for
  2 / 3 / 4 bits): N(0, I) keys and query, the needle q + 0.1 N(0, I) at a seeded
  position, 16 positions per (seq, bits), with both MSE-only codes of b bits and
  (b - 1)-bit codes plus the QJL sketch. The GPU quantizes and scores; the
  argmax must hit the needle, the packed keys must match the oracle's
  quantizer, and the scores the oracle's estimate on the GPU's packed keys.
* "MSE-Only vs QJL：bias 差異確認": over 4096 (key, fresh query) pairs of random
  unit vectors, scores from GPU-packed keys are shrunk for MSE-only codes (the
  multiplicative bias equals the quadrature shrinkage under the exact
  coordinate law, and is clearly positive at 2 and 3 bits) and unbiased with
  QJL; the signed means are noise-level, as the printed values are. d = 64,
  128, 256 (the sweep's dimensions), total widths 2..4.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import stats

from parity import check_close, check_quantize
from test_oracle_pages import beta_shrinkage

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))
NEEDLE_POSITIONS = 16


def tqmod():
    import kv_cache_vector_03_amd as tq
    return tq


def quantizers(d, bits, m, seed=3):
    tq = tqmod()
    diag = synth.diag_signs(seed, synth.ROLE_DIAG_K, d)
    S = synth.proj_matrix_f16(seed, synth.ROLE_PROJ_K, m, d) if m else None
    return tq.Quantizer(d, bits, m, diag, S, DEV), oracle.Quantizer(d, bits, m, diag, S)


def gpu_packed_to_oracle(qo, host):
    c, s, n, r = host
    if qo.m == 0:
        s, r = np.zeros((c.shape[0], 0), np.uint32), np.zeros(c.shape[0], np.uint16)
    return oracle.Packed(c, s, n, r)


def needle_case(s, seq, d=128):
    """fp32 keys [seq, d] with the needle planted, the query, and its position."""
    seed = 100 + s
    keys = synth.normals(seed, synth.ROLE_DATA_K, np.arange(seq * d)).reshape(seq, d)
    qv = synth.normals(seed, synth.ROLE_QUERY, np.arange(d))
    pos = int(synth.uniforms(seed, synth.ROLE_NEEDLE_POS, [seq])[0] * seq)
    keys[pos] = qv + 0.1 * synth.normals(seed, synth.ROLE_NEEDLE_NOISE, np.arange(d))
    return synth.to_f32(keys), synth.to_f32(qv), pos


@pytest.mark.parametrize("bits", GOLDEN["needle"]["bits"])
@pytest.mark.parametrize("mode", ["mse", "qjl"])
def test_needle_on_gpu(bits, mode):
    tq = tqmod()
    d = 128
    m = 0 if mode == "mse" else d
    qg, qo = quantizers(d, bits if mode == "mse" else bits - 1, m)
    worst = 0.0
    for seq in GOLDEN["needle"]["seq"]:
        for s in range(NEEDLE_POSITIONS):
            keys, qv, pos = needle_case(s, seq, d)
            assert stats.needle_hit(keys.astype(np.float64) @ qv.astype(np.float64), pos)  # exact scores hit
            x = torch.from_numpy(keys).to(DEV)
            p = tq.Packed.empty(qg, seq, DEV)
            tq.tq_quantize(qg, x, p)
            sc = torch.empty((1, seq), dtype=torch.float32, device=DEV)
            tq.tq_scores(qg, p, seq, torch.from_numpy(qv[None, :]).to(DEV), sc)
            torch.cuda.synchronize()
            est = sc.cpu().numpy()[0]
            assert stats.needle_hit(est, pos), (bits, mode, seq, s, int(np.argmax(est)), pos)
            host = p.to_host()
            check_quantize(qo, keys.astype(np.float64), host)
            ref = oracle.scores(qo, gpu_packed_to_oracle(qo, host), qv[None, :].astype(np.float64))[0]
            worst = max(worst, check_close(est, ref, what=f"needle scores seq={seq} s={s}"))
    print(f"needle bits={bits} {mode}: 48 retrievals hit; max |score - oracle| {worst:.2e}")


@pytest.fixture(scope="module")
def pair_sets():
    n = 4096
    out = {}
    for d in (64, 128, 256):
        x = synth.unit_vectors_f32(6, synth.ROLE_DATA_K, n, d)
        q = synth.unit_vectors_f32(6, synth.ROLE_PAIR_Q, n, d)
        exact = np.sum(x.astype(np.float64) * q.astype(np.float64), axis=1)
        out[d] = (x, q, exact)
    return out


def gpu_pair_scores(qg, x, q):
    """Diagonal of the GPU's score matrix: the estimate for pair (q_i, x_i)."""
    tq = tqmod()
    n = x.shape[0]
    p = tq.Packed.empty(qg, n, DEV)
    tq.tq_quantize(qg, torch.from_numpy(x).to(DEV), p)
    sc = torch.empty((n, n), dtype=torch.float32, device=DEV)
    tq.tq_scores(qg, p, n, torch.from_numpy(q).to(DEV), sc)
    torch.cuda.synchronize()
    return torch.diagonal(sc).cpu().numpy().astype(np.float64), p.to_host()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("mode", ["mse", "qjl"])
def test_bias_on_gpu_packed_keys(pair_sets, d, bits, mode):
    x, q, exact = pair_sets[d]
    m = 0 if mode == "mse" else d
    qg, qo = quantizers(d, bits if mode == "mse" else bits - 1, m)
    est, host = gpu_pair_scores(qg, x, q)
    check_quantize(qo, x.astype(np.float64), host)
    # the estimates equal the oracle's on the GPU's packed keys (first 512 pairs)
    P = gpu_packed_to_oracle(qo, host)
    ref = np.diag(oracle.scores(qo, P.take(slice(0, 512)), q[:512].astype(np.float64)))
    check_close(est[:512], ref, what="pair scores")
    bm, se = stats.bias_mult(est, exact), stats.bias_mult_se(est, exact)
    sd = np.std(est - exact, ddof=1) / np.sqrt(len(est))
    bs = stats.bias_signed(est, exact)
    print(f"d={d} b={bits} {mode}: bias_signed {bs:+.6f} (sd {sd:.1e}), bias_mult {bm:+.5f} (se {se:.1e})")
    assert abs(bs) < 4 * sd
    if mode == "mse":
        assert abs(bm - beta_shrinkage(d, qo.cb)) < 4 * se
        if bits <= 3:
            assert bm / se > 5
    else:
        assert abs(bm) < 4 * se
