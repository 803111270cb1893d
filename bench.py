"""Benchmark of the TurboQuant KV hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
quantize every layer's K (2-bit codes + 1-bit QJL sketch + fp16 norms) and V
(codes + fp16 norm), then one decode-attention step over every layer's
compressed cache (query preparation, the fused score/softmax/value scan and
the combine). Inputs are resident in HBM before timing starts; caches are
decoded only after all layers were quantized, so the decode reads them from
HBM rather than from the last-level cache.

Default workload: Llama-3.3-70B-shaped 128K decode, one layer's share
(8 KV heads x 131072 tokens x head_dim 128, 64 query heads, G = 8) repeated
over 80 layer instances with their own seeds. ``--workload 8k`` runs the
Qwen2.5-3B-shaped 8K cache (36 layers x 2 KV heads x 8192 tokens) as one call
per op over the whole model, with replicas to exceed the last-level cache.

Prints ONE JSON line. ``value`` is whole-step packed-KV throughput:
algorithmic bytes of all ops of a step / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "packed-KV GB/s & % HBM peak (quantize, score, decode-attn); keys/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=["128k", "8k"], default="128k")
    ap.add_argument("--replicas", type=int, default=5, help="8k workload: cache replicas")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (debug)")
    ap.add_argument("--cpu-batches", type=int, default=0,
                    help="batches the oracle baseline runs on (default 5 for 128k, 8 for 8k)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the small-keyset and prefill-scale score measurements")
    ap.add_argument("--scores-only", action="store_true",
                    help="only the small-keyset and prefill-scale score measurements (one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (profiler byte-counter calibration)")
    return ap.parse_args()


def packed_bytes_per_vector(d, mse_bits, qjl):
    b = mse_bits * d // 8 + 2
    if qjl:
        b += d // 8 + 2
    return b


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "quantize_k": ["kv_cache_vector_03_amd/csrc/tq_quantize_m128.hip", "kv_cache_vector_03_amd/csrc/tq_device.h"],
    "quantize_v": ["kv_cache_vector_03_amd/csrc/tq_quantize_m128.hip", "kv_cache_vector_03_amd/csrc/tq_device.h"],
    "decode_attn": ["kv_cache_vector_03_amd/csrc/tq_decode.hip", "kv_cache_vector_03_amd/csrc/tq_attn.hip",
                    "kv_cache_vector_03_amd/csrc/tq_append.h", "kv_cache_vector_03_amd/csrc/tq_device.h",
                    "kv_cache_vector_03_amd/csrc/tq_host.cpp"],
}


def traffic_for(op, launch_alg_bytes, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{op}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(KERNEL_SOURCES[op]):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.scores_only:
        scores_only()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures the data-parallel path on one GPU; "
                                   "runs on several GPUs are not part of it", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_vector_03_amd as tq
    import synth
    from synth import gpu as sgpu
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.KV_128K if args.workload == "128k" else W.KV_8K
    d, T, G, H = cfg.d, cfg.tokens, cfg.G, cfg.kv_heads
    layers = args.layers or cfg.layers
    diag_k, S, diag_v = W.quantizer_inputs(d)
    qk = tq.Quantizer(d, cfg.k_mse_bits, d, diag_k, S, dev)
    qv = tq.Quantizer(d, cfg.v_bits, 0, diag_v, None, dev)

    # ---- batches: one per layer (128k) or one per replica of the whole model (8k)
    units = []
    if args.workload == "128k":
        for l in range(layers):
            units.append(dict(layers=[l], ns=H))
    else:
        for r in range(args.replicas):
            units.append(dict(layers=list(range(layers)), ns=layers * H))
    t_gen = time.time()
    # one packed buffer pair for the whole step (batches are slices of it), so that
    # every layer's cache can also be attended in a single call
    n_all = sum(u["ns"] for u in units) * T
    PK_all, PV_all = tq.Packed.empty(qk, n_all, dev), tq.Packed.empty(qv, n_all, dev)
    off = 0
    for u in units:
        nvec = u["ns"] * T
        u["K"] = torch.empty((nvec, d), dtype=torch.float16, device=dev)
        u["V"] = torch.empty((nvec, d), dtype=torch.float16, device=dev)
        per = H * T
        for li, l in enumerate(u["layers"]):
            for role, buf in ((synth.ROLE_DATA_K, u["K"]), (synth.ROLE_DATA_V, u["V"])):
                sc = sgpu.scales_to_device(W.kv_seed_scales(cfg, l, role), dev)
                W.kv_layer_device(cfg, l, role, buf[li * per:(li + 1) * per], sc)
        q = np.stack([W.kv_queries_host(cfg, l) for l in u["layers"]]).reshape(u["ns"], G, d)
        u["Q"] = torch.from_numpy(np.ascontiguousarray(q)).to(dev)
        u["PK"], u["PV"] = PK_all.slice(off, off + nvec), PV_all.slice(off, off + nvec)
        off += nvec
        u["out"] = torch.empty((u["ns"], G, d), dtype=torch.float32, device=dev)
    max_ns = max(u["ns"] for u in units)
    ws = tq.workspace(tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, qk, max_ns, T, G), dev)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    stream = torch.cuda.current_stream()
    ops = ("quantize_k", "quantize_v", "decode_attn")
    events = {o: [] for o in ops}

    def step(record):
        # each op's launches of the step back to back between two events (one pair
        # per op and step, so the events add nothing between launches): every
        # layer's K, then every layer's V, then one decode call per batch
        def group(op, fn):
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for u in units:
                    fn(u)
                b.record(stream)
                events[op].append((a, b))
            else:
                for u in units:
                    fn(u)
        group("quantize_k", lambda u: tq.tq_quantize(qk, u["K"], u["PK"]))
        group("quantize_v", lambda u: tq.tq_quantize(qv, u["V"], u["PV"]))
        group("decode_attn", lambda u: tq.tq_decode_attn(qk, qv, u["PK"], u["PV"], u["ns"], T, G, u["Q"],
                                                        u["out"], ws=ws))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # ---- algorithmic bytes per launch
    kb = packed_bytes_per_vector(d, cfg.k_mse_bits, True)
    vb = packed_bytes_per_vector(d, cfg.v_bits, False)
    per_launch = {}
    for u in units[:1]:
        nvec = u["ns"] * T
        per_launch["quantize_k"] = nvec * (2 * d + kb)
        per_launch["quantize_v"] = nvec * (2 * d + vb)
        per_launch["decode_attn"] = nvec * (kb + vb) + u["ns"] * G * d * (2 + 4)
    units_per_launch = {"quantize_k": units[0]["ns"] * T, "quantize_v": units[0]["ns"] * T,
                        "decode_attn": units[0]["ns"] * T}
    launches = {o: len(events[o]) * len(units) for o in ops}
    kern = {}
    for o in ops:
        ms = [a.elapsed_time(b) / len(units) for a, b in events[o]]
        avg_s = float(np.mean(ms)) * 1e-3
        gbs = per_launch[o] / avg_s / 1e9
        kern[o] = {"us_per_launch": round(avg_s * 1e6, 2), "alg_bytes_per_launch": per_launch[o],
                   "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                   "keys_per_s": round(units_per_launch[o] / avg_s, 1),
                   "launches_per_step": launches[o] // args.steps,
                   "time_share": None}
    tot = sum(kern[o]["us_per_launch"] * kern[o]["launches_per_step"] for o in ops)
    for o in ops:
        kern[o]["time_share"] = round(kern[o]["us_per_launch"] * kern[o]["launches_per_step"] / tot, 3)
    step_bytes = sum(per_launch[o] * launches[o] // args.steps for o in ops)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom = max(ops, key=lambda o: kern[o]["time_share"])
    for o in ops:
        kern[o]["traffic"] = traffic_for(o, per_launch[o], args.workload)
    roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GB_per_s"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kern[dom]["frac_hbm_peak"], "traffic": kern[dom]["traffic"]}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name if args.workload == "8k" else
                   "llama-3.3-70b-shaped 128K decode, one layer's share, x80 layer instances",
                   "layers": layers, "kv_heads": H, "tokens": T, "head_dim": d, "G": G,
                   "k_bits": f"{cfg.k_mse_bits}+1qjl", "v_bits": cfg.v_bits, "input": "fp16",
                   "batches_per_step": len(units)},
        "keys_per_s": round(units_per_launch["decode_attn"] * launches["decode_attn"] / args.steps
                            / (ms_per_step * 1e-3), 1),
        "roofline": roof,
        "kernels": kern,
        "setup_s": round(t_gen, 2),
    }

    if not args.no_extras:
        result["decode_step"] = decode_step(tq, qk, qv, units, T, G, d, kern["decode_attn"]["us_per_launch"],
                                            kb + vb, dev)
        result["unfused_baseline"] = unfused_baseline(tq, qk, qv, units, T, G, d,
                                                      kern["decode_attn"]["us_per_launch"], dev)
        result["small_keyset"] = small_keyset(tq, qk, dev)
        result["wide_widths"] = wide_widths(tq, qv, units[0], T, G, d, diag_k, S, diag_v, dev)
        if args.workload == "128k":
            result["sweep_quantize"] = sweep_quantize(tq, dev)
        if args.workload == "128k":
            result["prefill_scores"] = prefill_scores(tq, qk, units[0]["PK"], T, dev)
            result["decode_all_layers_one_call"] = decode_one_call(
                tq, qk, qv, PK_all, PV_all, units, T, G, d, kern["decode_attn"]["us_per_launch"], kb + vb, dev)
            result["workload_8k"] = workload_8k(tq, dev, steps=max(3, args.steps // 2), warmup=2)

    if not args.no_cpu_baseline:
        nb = args.cpu_batches or (5 if args.workload == "128k" else 8)
        result["cpu_baseline"] = cpu_baseline(cfg, diag_k, S, diag_v, kb, vb, units, nb)
    print(json.dumps(result))


def cpu_baseline(cfg, diag_k, S, diag_v, kb, vb, units, n_batches):
    """The oracle on a bounded sample of the same workload: the first
    ``n_batches`` batches of a step (taken cyclically when the step has
    fewer), each quantized (K and V) and decoded with its G query heads, on
    the same fp16 inputs the GPU quantizes. Host copies are made outside the
    timed region."""
    import oracle
    d, G, T = cfg.d, cfg.G, cfg.tokens
    qko = oracle.Quantizer(d, cfg.k_mse_bits, d, diag_k, S)
    qvo = oracle.Quantizer(d, cfg.v_bits, 0, diag_v, None)
    dt, alg, toks = 0.0, 0, 0
    for i in range(n_batches):
        u = units[i % len(units)]
        ns = u["ns"]
        n = ns * T
        K = u["K"].cpu().numpy().astype("float64")
        V = u["V"].cpu().numpy().astype("float64")
        Q = u["Q"].cpu().numpy().astype("float64")
        if i == 0:
            oracle.quantize(qko, K[:256])
        t0 = time.perf_counter()
        pk = oracle.quantize(qko, K)
        pv = oracle.quantize(qvo, V)
        oracle.decode_attn(qko, qvo, pk, pv, ns, T, G, Q)
        dt += time.perf_counter() - t0
        alg += n * (2 * d + kb) + n * (2 * d + vb) + n * (kb + vb) + ns * G * d * 6
        toks += n
        del K, V, pk, pv
    cores = oracle.max_threads()
    # the same on one core: the first stream of the first batch
    u = units[0]
    K = u["K"][:T].cpu().numpy().astype("float64")
    V = u["V"][:T].cpu().numpy().astype("float64")
    Q = u["Q"][:1].cpu().numpy().astype("float64")
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        pk = oracle.quantize(qko, K)
        pv = oracle.quantize(qvo, V)
        oracle.decode_attn(qko, qvo, pk, pv, 1, T, G, Q)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(cores)
    alg1 = T * (2 * d + kb) + T * (2 * d + vb) + T * (kb + vb) + G * d * 6
    return {"value": round(alg / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n_batches} batches of the step ({toks} tokens in all): quantize K and V, decode "
                      f"with {G} query heads per stream; {dt:.1f} s of oracle time",
            "value_1core": round(alg1 / dt1 / 1e9, 5),
            "sample_1core": f"one stream ({T} tokens) of the first batch, the same three steps, on one "
                            f"thread; {dt1:.1f} s"}


def timed_us(fn, passes, stream):
    """Mean microseconds per call of fn over `passes` calls (after one untimed call)."""
    import torch
    fn()
    ev = []
    for _ in range(passes):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e3


def decode_one_call(tq, qk, qv, PK_all, PV_all, units, T, G, d, layer_us, tok_bytes, dev, passes=3):
    """Every layer's cache attended in one call (all layers x KV heads streams
    over the step's single packed buffer pair), beside the per-layer calls."""
    import torch
    ns = sum(u["ns"] for u in units)
    Q = torch.cat([u["Q"] for u in units])
    out = torch.empty((ns, G, d), dtype=torch.float32, device=dev)
    ws = tq.workspace(tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, qk, ns, T, G), dev)
    us = timed_us(lambda: tq.tq_decode_attn(qk, qv, PK_all, PV_all, ns, T, G, Q, out, ws=ws), passes,
                  torch.cuda.current_stream())
    alg = ns * T * tok_bytes + ns * G * d * 6
    return {"streams": ns, "us_per_launch": round(us, 1), "GB_per_s": round(alg / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "per_layer_calls_us": round(layer_us * len(units), 1)}


def workload_8k(tq, dev, steps=10, warmup=2, replicas=5):
    """The Qwen2.5-3B-shaped 8K workload (36 layers x 2 KV heads x 8192 tokens,
    K 2+1 QJL, V 3-bit): quantize K and V of the whole model per call, decode
    all 72 streams in one call (the model's KV for one decode step), and decode
    one layer per call (2 streams, 36 calls); `replicas` copies of the cache
    rotate so consecutive calls do not hit in cache. us per launch, GB/s of
    algorithmic bytes, fraction of 8 TB/s, and counter traffic when profiles/
    holds it for the current sources."""
    import numpy as np
    import torch
    import synth
    from synth import gpu as sgpu
    from synth import workloads as W
    cfg = W.KV_8K
    d, T, G, H, L = cfg.d, cfg.tokens, cfg.G, cfg.kv_heads, cfg.layers
    diag_k, S, diag_v = W.quantizer_inputs(d)
    qk = tq.Quantizer(d, cfg.k_mse_bits, d, diag_k, S, dev)
    qv = tq.Quantizer(d, cfg.v_bits, 0, diag_v, None, dev)
    ns, per = L * H, H * T
    n = ns * T
    reps = []
    for r in range(replicas):
        u = {"K": torch.empty((n, d), dtype=torch.float16, device=dev),
             "V": torch.empty((n, d), dtype=torch.float16, device=dev)}
        for l in range(L):
            for role, buf in ((synth.ROLE_DATA_K, u["K"]), (synth.ROLE_DATA_V, u["V"])):
                sc = sgpu.scales_to_device(W.kv_seed_scales(cfg, l, role), dev)
                W.kv_layer_device(cfg, l, role, buf[l * per:(l + 1) * per], sc)
        q = np.stack([W.kv_queries_host(cfg, l) for l in range(L)]).reshape(ns, G, d)
        u["Q"] = torch.from_numpy(np.ascontiguousarray(q)).to(dev)
        u["PK"], u["PV"] = tq.Packed.empty(qk, n, dev), tq.Packed.empty(qv, n, dev)
        u["out"] = torch.empty((ns, G, d), dtype=torch.float32, device=dev)
        reps.append(u)
    ws = tq.workspace(tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, qk, ns, T, G), dev)
    stream = torch.cuda.current_stream()
    kb = packed_bytes_per_vector(d, cfg.k_mse_bits, True)
    vb = packed_bytes_per_vector(d, cfg.v_bits, False)
    ops = {
        "quantize_k": (lambda u: tq.tq_quantize(qk, u["K"], u["PK"]), n * (2 * d + kb)),
        "quantize_v": (lambda u: tq.tq_quantize(qv, u["V"], u["PV"]), n * (2 * d + vb)),
        "decode_attn": (lambda u: tq.tq_decode_attn(qk, qv, u["PK"], u["PV"], ns, T, G, u["Q"], u["out"], ws=ws),
                        n * (kb + vb) + ns * G * d * 6),
    }
    for u in reps:
        for o in ops:
            ops[o][0](u)
    torch.cuda.synchronize()
    res = {"workload": cfg.name, "layers": L, "kv_heads": H, "tokens": T, "G": G,
           "k_bits": f"{cfg.k_mse_bits}+1qjl", "v_bits": cfg.v_bits, "replicas": replicas}
    for o, (fn, alg) in ops.items():
        for i in range(warmup):
            fn(reps[i % replicas])
        # one event pair per pass over the replicas
        ev = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for u in reps:
                fn(u)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in ev) / (len(ev) * replicas) * 1e3
        gbs = alg / (us * 1e-6) / 1e9
        res[o] = {"us_per_launch": round(us, 2), "alg_bytes_per_launch": alg, "GB_per_s": round(gbs, 1),
                  "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_for(o, alg, "8k")}
    # one layer per call: streams 2 l, 2 l + 1 of a replica's buffers
    outs = torch.empty((H, G, d), dtype=torch.float32, device=dev)

    def layer_calls(u):
        for l in range(L):
            tq.tq_decode_attn(qk, qv, u["PK"].slice(l * per, (l + 1) * per), u["PV"].slice(l * per, (l + 1) * per),
                              H, T, G, u["Q"][l * H:(l + 1) * H], outs, ws=ws)
    us = timed_us(lambda: layer_calls(reps[0]), max(3, steps), stream) / L
    alg = per * (kb + vb) + H * G * d * 6
    res["decode_attn_per_layer"] = {"calls_per_step": L, "us_per_launch": round(us, 2),
                                    "GB_per_s": round(alg / (us * 1e-6) / 1e9, 1),
                                    "frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del reps
    torch.cuda.empty_cache()
    return res


def small_keyset(tq, qk, dev, reps=50):
    """The score path on the pages' small benchmark shape (GB10 section of the
    GX10 page): quantize 8192 fp16 keys (prod 2+1, d = 128, four outlier
    channels), then score 64 queries against all of them. Both are single
    launches of a few MB, so they are latency-bound; reported in microseconds
    beside the page's PyTorch timings (31.04 ms and 11.16 ms on a GB10)."""
    import torch
    from synth import workloads as W
    keys, qs = W.outlier_keys_host()
    x = torch.from_numpy(keys).to(dev)
    q = torch.from_numpy(qs).to(dev)
    pk = tq.Packed.empty(qk, x.shape[0], dev)
    scores = torch.empty((q.shape[0], x.shape[0]), dtype=torch.float32, device=dev)
    ws = tq.workspace(tq.tq_workspace_size(tq.TQ_OP_SCORES, qk, q.shape[0], x.shape[0]), dev)
    stream = torch.cuda.current_stream()
    out = {}
    for name, fn in (("quantize_8192_keys", lambda: tq.tq_quantize(qk, x, pk)),
                     ("scores_64x8192", lambda: tq.tq_scores(qk, pk, x.shape[0], q, scores, ws=ws))):
        for _ in range(5):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        out[name + "_us"] = round(a.elapsed_time(b) / reps * 1e3, 2)
    out["page_gb10_ms"] = {"quantize_8192_keys": 31.04, "scores_64x8192": 11.16}
    return out


def decode_step(tq, qk, qv, units, T, G, d, attn_us, tok_bytes, dev, passes=3):
    """The fused append + attend step (tq_decode_step) on the same caches: each
    stream's last token is re-quantized from its fp16 K and V into slot T - 1
    (the append), then the attention runs over all T tokens. Timed as
    decode_attn is (one call per batch, every batch's calls back to back between
    two events), in passes alternating with passes of decode_attn alone, so the
    difference is the append's cost."""
    import torch
    apps = []
    for u in units:
        ns = u["ns"]
        apps.append((u["K"].view(ns, T, d)[:, T - 1].contiguous(), u["V"].view(ns, T, d)[:, T - 1].contiguous()))
    max_ns = max(u["ns"] for u in units)
    ws = tq.workspace(tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, qk, max_ns, T, G), dev)
    stream = torch.cuda.current_stream()

    def step_pass():
        for u, (kn, vn) in zip(units, apps):
            tq.tq_decode_step(qk, qv, u["PK"], u["PV"], u["ns"], T - 1, T, G, kn, vn, u["Q"], u["out"], ws=ws)

    def attn_pass():
        for u in units:
            tq.tq_decode_attn(qk, qv, u["PK"], u["PV"], u["ns"], T, G, u["Q"], u["out"], ws=ws)

    def timed(fn, ev):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        ev.append((a, b))

    step_pass()
    attn_pass()
    ev_s, ev_a = [], []
    for _ in range(passes):
        timed(step_pass, ev_s)
        timed(attn_pass, ev_a)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in ev_s) / (len(ev_s) * len(units)) * 1e3
    us_a = sum(a.elapsed_time(b) for a, b in ev_a) / (len(ev_a) * len(units)) * 1e3
    ns = units[0]["ns"]
    alg = ns * T * tok_bytes + ns * G * d * 6 + ns * 2 * d * 2
    return {"us_per_launch": round(us, 2), "decode_attn_us_per_launch": round(us_a, 2),
            "append_overhead_us": round(us - us_a, 2), "GB_per_s": round(alg / (us * 1e-6) / 1e9, 1),
            "note": "append of one new token per stream inside the decode launch (the new token's partial "
                    "joins the stream's combine); decode_attn timed alongside in alternating passes"}


def wide_widths(tq, qv, u, T, G, d, diag_k, S, diag_v, dev, passes=3):
    """Code widths above 4 bits on the first batch: 8-bit keys (7-bit codes + the
    1-bit sketch) beside the workload's values, and 8-bit values; quantize and
    decode times per launch with their algorithmic GB/s."""
    import torch
    ns = u["ns"]
    nvec = ns * T
    qk8 = tq.Quantizer(d, 7, d, diag_k, S, dev)
    qv8 = tq.Quantizer(d, 8, 0, diag_v, None, dev)
    pk8, pv8 = tq.Packed.empty(qk8, nvec, dev), tq.Packed.empty(qv8, nvec, dev)
    ws = tq.workspace(tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, qk8, ns, T, G), dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        ev = []
        for _ in range(passes):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e3

    kb8 = packed_bytes_per_vector(d, 7, True)
    vbw = packed_bytes_per_vector(d, qv.mse_bits, False)
    vb8 = packed_bytes_per_vector(d, 8, False)
    res = {}
    for name, fn, alg in (
            ("quantize_k8", lambda: tq.tq_quantize(qk8, u["K"], pk8), nvec * (2 * d + kb8)),
            ("quantize_v8", lambda: tq.tq_quantize(qv8, u["V"], pv8), nvec * (2 * d + vb8)),
            (f"decode_k8v{qv.mse_bits}",
             lambda: tq.tq_decode_attn(qk8, qv, pk8, u["PV"], ns, T, G, u["Q"], u["out"], ws=ws),
             nvec * (kb8 + vbw) + ns * G * d * 6),
            ("decode_k8v8", lambda: tq.tq_decode_attn(qk8, qv8, pk8, pv8, ns, T, G, u["Q"], u["out"], ws=ws),
             nvec * (kb8 + vb8) + ns * G * d * 6)):
        us = timed(fn)
        res[name] = {"us_per_launch": round(us, 2), "GB_per_s": round(alg / (us * 1e-6) / 1e9, 1),
                     "frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    res["note"] = ("MFMA quantizer with binary-search codes; MFMA decode with single-code tables "
                   "(values of 4 or 8 bits)")
    return res


def sweep_quantize(tq, dev, n=1 << 20, passes=3, n_pairs=4096):
    """Quantize throughput of the sweep workload: 2^20 unit-norm fp32 vectors
    (normalised N(0, I)) for d in {64, 128, 256} and total widths 2..4, with
    the QJL sketch (width - 1 code bits) and without; us per launch and
    algorithmic GB/s (fp32 input read, packed output written). From the same
    GPU-packed vectors: the distortion per coordinate of the code stage
    (mean (x - x_hat)^2 over all coordinates, x_hat dequantized without the
    sketch term), and the score bias over n_pairs (key, query) pairs of unit
    vectors, est = tq_scores: signed mean(est - exact) and the shrinkage
    1 - sum(est exact) / sum(exact^2) with its delta-method standard error
    ("MSE-Only vs QJL" section of the benchmark page; its printed distortion
    is 0.000270 at d = 128, b = 3 and 0.000135 at d = 256)."""
    import torch
    import synth
    from synth import gpu as sgpu
    from synth import workloads as W
    stream = torch.cuda.current_stream()
    res = {}
    for d in (64, 128, 256):
        diag_k, S, diag_v = W.quantizer_inputs(d)
        g = torch.empty((n, d), dtype=torch.float32, device=dev)
        sgpu.fill_f32(g, 61, synth.ROLE_DATA_K)
        x = g / torch.linalg.vector_norm(g, dim=1, keepdim=True)
        sgpu.fill_f32(g[:n_pairs], 62, synth.ROLE_PAIR_Q)
        qp = (g[:n_pairs] / torch.linalg.vector_norm(g[:n_pairs], dim=1, keepdim=True)).contiguous()
        del g
        exact = (x[:n_pairs].double() * qp.double()).sum(dim=1)
        xhat = torch.empty((n, d), dtype=torch.float32, device=dev)
        sc = torch.empty((n_pairs, n_pairs), dtype=torch.float32, device=dev)
        for bits in (2, 3, 4):
            for qjl in (False, True):
                mse = bits - 1 if qjl else bits
                q = tq.Quantizer(d, mse, d if qjl else 0, diag_k if qjl else diag_v, S if qjl else None, dev)
                p = tq.Packed.empty(q, n, dev)
                tq.tq_quantize(q, x, p)
                ev = []
                for _ in range(passes):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    tq.tq_quantize(q, x, p)
                    b.record(stream)
                    ev.append((a, b))
                torch.cuda.synchronize()
                us = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e3
                alg = n * (4 * d + packed_bytes_per_vector(d, mse, qjl))
                tq.tq_dequantize(q, p, n, False, xhat)
                dist = float(((x - xhat).double() ** 2).mean())
                tq.tq_scores(q, p, n_pairs, qp, sc)
                est = torch.diagonal(sc).double()
                s2 = float((exact * exact).sum())
                b = float((est * exact).sum()) / s2
                resid = exact * (est - b * exact)
                res[f"d{d}_b{bits}_{'qjl' if qjl else 'mse'}"] = {
                    "us_per_launch": round(us, 2), "GB_per_s": round(alg / (us * 1e-6) / 1e9, 1),
                    "frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "code_bits": mse, "distortion_per_coord": float(f"{dist:.4g}"),
                    "bias_signed": float(f"{float((est - exact).mean()):.3g}"),
                    "bias_mult": round(1.0 - b, 5),
                    "bias_mult_se": float(f"{float(torch.sqrt((resid * resid).sum())) / s2:.2g}")}
        del x, xhat, sc
    return res


def unfused_baseline(tq, qk, qv, units, T, G, d, fused_us, dev, passes=3, n_units=8):
    """The engines' unfused design on the same caches, for comparison: each
    batch's packed K and V are dequantized to fp16 (tq_dequantize, keys with
    the QJL term so scores match the estimator), then dense attention runs
    with torch (fp16 batched products, fp32 softmax). Timed per batch over up
    to n_units distinct batches; reported beside the fused decode_attn."""
    import torch
    ns = units[0]["ns"]
    n = ns * T
    Kd = torch.empty((n, d), dtype=torch.float16, device=dev)
    Vd = torch.empty((n, d), dtype=torch.float16, device=dev)
    scale = 1.0 / (d ** 0.5)
    stream = torch.cuda.current_stream()

    def dequant(u):
        tq.tq_dequantize(qk, u["PK"], n, True, Kd)
        tq.tq_dequantize(qv, u["PV"], n, False, Vd)

    def attend(u):
        K3, V3 = Kd.view(ns, T, d), Vd.view(ns, T, d)
        qt = u["Q"].to(torch.float16).transpose(1, 2).contiguous()      # [ns, d, G]
        z = torch.bmm(K3, qt).float() * scale                              # [ns, T, G]
        w = torch.softmax(z, dim=1).transpose(1, 2).contiguous().to(torch.float16)
        return torch.bmm(w, V3).float()                                    # [ns, G, d]

    us = [u for u in units if u["ns"] == ns][:n_units]
    dequant(us[0]); attend(us[0])
    ev_d, ev_a = [], []
    for _ in range(passes):
        for u in us:
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record(stream)
            dequant(u)
            b.record(stream)
            attend(u)
            c.record(stream)
            ev_d.append((a, b))
            ev_a.append((b, c))
    torch.cuda.synchronize()
    dq = sum(a.elapsed_time(b) for a, b in ev_d) / len(ev_d) * 1e3
    at = sum(a.elapsed_time(b) for a, b in ev_a) / len(ev_a) * 1e3
    # agreement with the fused step on the last batch (fp16 rounding of the dequantized cache)
    u = us[-1]
    dequant(u)
    ref = attend(u)
    fused = torch.empty((ns, G, d), dtype=torch.float32, device=dev)
    tq.tq_decode_attn(qk, qv, u["PK"], u["PV"], ns, T, G, u["Q"], fused)
    torch.cuda.synchronize()
    diff = float((ref - fused).abs().max())
    # the unfused design's floor at the rate a plain device copy reaches here:
    # packed K and V read, fp16 K and V written, then read by the attention
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_us = timed_us(lambda: dst.copy_(src), 5, stream)
    del src, dst
    copy_gbs = 2 * nbytes / (copy_us * 1e-6) / 1e9
    kb = packed_bytes_per_vector(d, qk.mse_bits, qk.qjl_m > 0)
    vb = packed_bytes_per_vector(d, qv.mse_bits, False)
    unfused_bytes = n * (kb + vb) + 2 * (2 * n * d * 2)
    floor_us = unfused_bytes / (copy_gbs * 1e9) * 1e6
    return {"us_per_launch": round(dq + at, 2), "dequantize_us": round(dq, 2), "dense_attention_us": round(at, 2),
            "fused_decode_attn_us": fused_us, "fused_speedup": round((dq + at) / fused_us, 2),
            "unfused_floor_us": round(floor_us, 1), "copy_GB_per_s": round(copy_gbs, 1),
            "fused_speedup_vs_floor": round(floor_us / fused_us, 2),
            "max_abs_diff_vs_fused": round(diff, 5),
            "note": ("dequantize to fp16 + torch fp16 attention on the same packed caches; the floor is "
                     "that design's bytes (packed read, fp16 K and V written and read back) at the "
                     "measured device-copy rate")}


def prefill_scores(tq, qk, pk, T, dev, n_q=2048, reps=5):
    """Multi-query scoring at prefill scale: a 256-token chunk of queries for
    one KV head (256 x 8 query heads = 2048 queries, seeded N(0, 1) fp16)
    against that head's whole compressed 128K prefix (the first stream of a
    quantized layer), scores[2048][131072] in fp32 (1 GiB). Reported as
    scores/s, output GB/s and the MFMA rate it implies (1024 executed flop
    per score: eight 16x16x32 fp16 MFMAs per 8-query x 16-key tile)."""
    import numpy as np
    import torch
    import synth
    keys = tq.Packed(pk.codes[:T], pk.signs[:T], pk.norm[:T], pk.rnorm[:T])
    qh = synth.to_f16(synth.normals(97, synth.ROLE_QUERY, np.arange(n_q * qk.d)).reshape(n_q, qk.d))
    q = torch.from_numpy(qh).to(dev)
    scores = torch.empty((n_q, T), dtype=torch.float32, device=dev)
    ws = tq.workspace(tq.tq_workspace_size(tq.TQ_OP_SCORES, qk, n_q, T), dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        tq.tq_scores(qk, keys, T, q, scores, ws=ws)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        tq.tq_scores(qk, keys, T, q, scores, ws=ws)
    b.record(stream)
    torch.cuda.synchronize()
    s = a.elapsed_time(b) / reps * 1e-3
    n = n_q * T
    out_bytes = n * 4
    in_bytes = T * packed_bytes_per_vector(qk.d, qk.mse_bits, True) + n_q * qk.d * 2
    return {"queries": n_q, "keys": T, "us": round(s * 1e6, 1), "scores_per_s": round(n / s, 1),
            "GB_per_s": round((out_bytes + in_bytes) / s / 1e9, 1),
            "frac_hbm_peak": round((out_bytes + in_bytes) / s / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_TFLOP_per_s": round(n * 1024 / s / 1e12, 1)}


def scores_only():
    """The two score workloads on their own: the small keyset, and the
    prefill-scale scores over one stream of a quantized 128K layer (layer 0,
    KV head 0, quantized here)."""
    import torch
    import kv_cache_vector_03_amd as tq
    import synth
    from synth import gpu as sgpu
    from synth import workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.KV_128K
    d, T = cfg.d, cfg.tokens
    diag_k, S, _ = W.quantizer_inputs(d)
    qk = tq.Quantizer(d, cfg.k_mse_bits, d, diag_k, S, dev)
    per = cfg.kv_heads * T
    K = torch.empty((per, d), dtype=torch.float16, device=dev)
    W.kv_layer_device(cfg, 0, synth.ROLE_DATA_K, K, sgpu.scales_to_device(W.kv_seed_scales(cfg, 0, synth.ROLE_DATA_K), dev))
    pk = tq.Packed.empty(qk, T, dev)
    tq.tq_quantize(qk, K[:T], pk)
    print(json.dumps({"small_keyset": small_keyset(tq, qk, dev), "prefill_scores": prefill_scores(tq, qk, pk, T, dev)}))


def calibrate_copy():
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) of a profiler run."""
    import torch
    nbytes = 1 << 30
    src = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": 3}))


if __name__ == "__main__":
    main()
