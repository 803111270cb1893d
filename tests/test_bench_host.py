"""Host-side checks of bench.py (no GPU): the single-GPU contract and the
algorithmic byte counts that every bandwidth figure divides by.

Packed sizes per vector follow the layout of the quantizer's output (codes of
b bits per coordinate, the 1-bit sketch of m = d projections for keys, fp16
norm and, for keys, fp16 residual norm), as in "[Benchmark] TurboQuant 實測：
KV Cache 3-bit 壓縮，真的零損失？", sections "TurboQuant 是什麼：30 秒懶人包"
(the two stages) and "壓縮率與精度" (bytes per cached vector).
"""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == n and "one GPU" in line["error"]


@pytest.mark.parametrize("d,bits,qjl,expect", [
    (128, 2, True, 32 + 16 + 4),   # keys 2+1 at d = 128: 52 bytes
    (128, 3, False, 48 + 2),       # 3-bit values: 50 bytes
    (128, 4, False, 64 + 2),       # 4-bit values: 66 bytes
    (64, 2, True, 16 + 8 + 4),
    (256, 3, True, 96 + 32 + 4),
    (256, 1, False, 32 + 2),
])
def test_packed_bytes_per_vector(d, bits, qjl, expect):
    assert _bench().packed_bytes_per_vector(d, bits, qjl) == expect


def test_step_bytes_of_the_128k_layer():
    # 8 KV heads x 131072 tokens per layer: K 52 MiB and V (4-bit) 66 MiB packed,
    # 256 MiB of fp16 input each
    b = _bench()
    n = 8 * 131072
    assert n * b.packed_bytes_per_vector(128, 2, True) == 52 * 2**20
    assert n * b.packed_bytes_per_vector(128, 4, False) == 66 * 2**20
    assert n * 2 * 128 == 256 * 2**20


def test_traffic_record_ignored_when_sources_differ(tmp_path, monkeypatch):
    # a counter record whose source hash does not match the kernel sources
    # must not be reported as the current kernels' traffic
    b = _bench()
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setitem(b.KERNEL_SOURCES, "quantize_k", ["k.hip"])
    rec = {"op": "quantize_k", "workload": "128k", "hbm_bytes_per_launch": 123, "source_sha": b.source_sha(["k.hip"])}
    (prof / "traffic_quantize_k_128k.json").write_text(json.dumps(rec))
    assert b.traffic_for("quantize_k", 1, "128k") == 123
    src.write_text("kernel source, changed\n")
    assert b.traffic_for("quantize_k", 1, "128k") is None
    assert b.traffic_for("quantize_k", 1, "8k") is None  # no record at all
