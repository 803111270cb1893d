"""The benchmark workloads as seeded synthetic inputs (shapes, value laws, seeds).

These stand in for the pages' workloads; no real model weights or datasets are
used anywhere. Every tensor can be drawn on the host for any subset of vectors
(``*_host``) or in full on the GPU (``*_device``), bit-identically.

tiny       d=128, 1024 fp32 N(0,1) keys, 8 fp32 queries; keys 2-bit codes + 1-bit QJL.
outlier    d=128, 8192 fp16 N(0,1) keys with 4 seeded channels x20, 64 fp16 queries;
             keys 2-bit codes + QJL (the GB10 synthetic shape of the benchmark page).
8K model   36 layers x 2 KV heads x 8192 tokens x 128, fp16 K and V = N(0,1) times a
             per-(layer, head, channel) lognormal(0,1) scale; K 2-bit + QJL, V 3-bit;
             16 query heads per layer (G = 8), fp16 N(0,1).
sweep      d in {64,128,256}, 2^20 normalised N(0,I) fp32 vectors.
128K layer one layer's share: 8 KV heads x 131072 tokens x 128, fp16 K/V with
             per-channel lognormal scales, 80 layer instances (layer l draws from
             seed + l); K 2-bit + QJL, V 4-bit; 64 query heads per layer (G = 8).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (ROLE_DATA_K, ROLE_DATA_V, ROLE_DIAG_K, ROLE_DIAG_V, ROLE_PROJ_K, ROLE_QUERY,
               ROLE_SCALE_K, ROLE_SCALE_V, diag_signs, lognormal_scales, normals, outlier_scales,
               proj_matrix_f16, to_f16, to_f32)

QUANT_SEED = 7  # one K and one V quantizer shared by every layer of a model


@dataclass(frozen=True)
class KVConfig:
    name: str
    d: int
    layers: int
    kv_heads: int
    tokens: int
    G: int
    k_mse_bits: int       # key codes; keys always carry the 1-bit QJL sketch (m = d)
    v_bits: int           # value codes (codes only)
    seed: int
    per_layer_seed: bool  # layer l draws its K/V/scales/queries from seed + l

    @property
    def streams_per_layer(self) -> int:
        return self.kv_heads

    @property
    def n_streams(self) -> int:
        return self.layers * self.kv_heads

    def layer_seed(self, layer: int) -> int:
        return self.seed + layer if self.per_layer_seed else self.seed


KV_8K = KVConfig("qwen2.5-3b-shaped 8K", 128, 36, 2, 8192, 8, 2, 3, 3003, False)
KV_128K = KVConfig("llama-3.3-70b-shaped 128K, one layer's share", 128, 80, 8, 131072, 8, 2, 4,
                   5005, True)


def quantizer_inputs(d: int, seed: int = QUANT_SEED):
    """(diag_k, S_k fp16 [d, d], diag_v) shared by all layers."""
    return (diag_signs(seed, ROLE_DIAG_K, d), proj_matrix_f16(seed, ROLE_PROJ_K, d, d),
            diag_signs(seed, ROLE_DIAG_V, d))


# ------------------------------------------------------------------ the two small key sets

def tiny_keys_host():
    d = 128
    keys = to_f32(normals(1001, ROLE_DATA_K, np.arange(1024 * d)).reshape(1024, d))
    q = to_f32(normals(1001, ROLE_QUERY, np.arange(8 * d)).reshape(8, d))
    return keys, q


def outlier_keys_host():
    d = 128
    sc = outlier_scales(2002, d)
    keys = to_f16(normals(2002, ROLE_DATA_K, np.arange(8192 * d)).reshape(8192, d) * sc[None, :])
    q = to_f16(normals(2002, ROLE_QUERY, np.arange(64 * d)).reshape(64, d))
    return keys, q


# ------------------------------------------------------------------ the KV-cache workloads

def kv_scales(cfg: KVConfig, layer: int, role: int) -> np.ndarray:
    """lognormal scales [kv_heads, d] of one layer (float64)."""
    seed = cfg.layer_seed(layer)
    if cfg.per_layer_seed:
        return lognormal_scales(seed, role, cfg.kv_heads, cfg.d)
    full = lognormal_scales(seed, role, cfg.layers * cfg.kv_heads, cfg.d)
    return full[layer * cfg.kv_heads:(layer + 1) * cfg.kv_heads]


def kv_all_scales(cfg: KVConfig, role: int) -> np.ndarray:
    """scales [layers * kv_heads, d] (float64)."""
    return np.concatenate([kv_scales(cfg, l, role) for l in range(cfg.layers)])


def _first_vector(cfg: KVConfig, layer: int) -> int:
    # flat vector index of (layer, head 0, token 0) within its seed's stream
    return 0 if cfg.per_layer_seed else layer * cfg.kv_heads * cfg.tokens


def kv_vectors_host(cfg: KVConfig, layer: int, role: int, head: int, tokens) -> np.ndarray:
    """fp16 values [len(tokens), d] of K (role ROLE_DATA_K) or V of one (layer, head)."""
    seed = cfg.layer_seed(layer)
    scale_role = ROLE_SCALE_K if role == ROLE_DATA_K else ROLE_SCALE_V
    sc = kv_scales(cfg, layer, scale_role)[head]
    t = np.asarray(tokens, dtype=np.int64)
    vec = _first_vector(cfg, layer) + head * cfg.tokens + t
    idx = vec[:, None] * cfg.d + np.arange(cfg.d, dtype=np.int64)[None, :]
    return to_f16(normals(seed, role, idx) * sc[None, :])


def kv_queries_host(cfg: KVConfig, layer: int) -> np.ndarray:
    """fp16 queries [kv_heads, G, d] of one layer (query head j -> KV head j // G)."""
    seed = cfg.layer_seed(layer)
    nq = cfg.kv_heads * cfg.G
    first = 0 if cfg.per_layer_seed else layer * nq
    idx = (first + np.arange(nq))[:, None] * cfg.d + np.arange(cfg.d)[None, :]
    return to_f16(normals(seed, ROLE_QUERY, idx)).reshape(cfg.kv_heads, cfg.G, cfg.d)


def kv_seed_scales(cfg: KVConfig, layer: int, role: int) -> np.ndarray:
    """Scale rows of the stream that holds ``layer``, indexed by flat vector // tokens:
    the layer's own [kv_heads, d] for per-layer seeds, else the whole model's."""
    scale_role = ROLE_SCALE_K if role == ROLE_DATA_K else ROLE_SCALE_V
    if cfg.per_layer_seed:
        return kv_scales(cfg, layer, scale_role)
    return lognormal_scales(cfg.seed, scale_role, cfg.layers * cfg.kv_heads, cfg.d)


def kv_layer_device(cfg: KVConfig, layer: int, role: int, out, scales_dev):
    """Fill ``out`` (torch fp16 [kv_heads * tokens, d], cuda) with one layer's K or V;
    ``scales_dev`` is ``kv_seed_scales`` on the device as float64."""
    from . import gpu
    return gpu.fill_f16(out, cfg.layer_seed(layer), role, first=_first_vector(cfg, layer) * cfg.d,
                        d=cfg.d, tokens=cfg.tokens, scales=scales_dev)
