"""Build the native libraries in-tree for gfx950.

* ``kv_cache_vector_03_amd/libtq.so`` -- the product: C ABI in include/tq.h
  (host validation and codebook in C++, kernels in HIP).
* ``synth/libtqsynth.so`` -- the GPU twin of the seeded input generators
  (built with floating-point contraction off so it matches numpy bit for bit).

Run ``python -m kv_cache_vector_03_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

LIB = os.path.join(PKG, "libtq.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libtqsynth.so")

HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", f"-I{INCLUDE}",
              f"-I{CSRC}"]

# per-source extra hipcc flags: keep MFMA results in ordinary VGPRs (no AGPR
# copies) where the results feed VALU code right away
EXTRA_FLAGS = {"tq_quantize_m128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

SOURCES = ["tq_host.cpp", "tq_api.cpp", "tq_quantize.hip", "tq_quantize_m128.hip", "tq_attn.hip",
           "tq_decode.hip", "tq_launch.hip", "tq_wide.hip"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {os.path.basename(cmd[-1])}")
    return r


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = ["g++", *HOST_FLAGS, "-c", path, "-o", obj]
    _run(cmd)
    return obj


def build_product(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


# Host-only sanitizer build: the C++ host code (argument validation, plans,
# codebook solver) with AddressSanitizer and UBSan, linked with the ordinary
# kernel objects of build_product; the kernels themselves are not instrumented.
SAN_LIB = os.path.join(BUILD, "san", "libtq_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]
HOST_SOURCES = [s for s in SOURCES if s.endswith(".cpp")]


def build_sanitized() -> str:
    """_build/san/libtq_san.so: host objects with SAN_FLAGS (g++), kernel
    objects as built by build_product (run that first). Loaded instead of
    libtq.so when TQ_SANITIZE=1; see tests/sanitize_cpu_suite.sh."""
    sdir = os.path.join(BUILD, "san")
    os.makedirs(sdir, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(sdir, src + ".o")
        _run(["g++", *HOST_FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in SOURCES:
        if src.endswith(".hip"):
            obj = os.path.join(BUILD, src + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing: run build_product first")
            objs.append(obj)
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-shared", *SAN_FLAGS, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", tmp])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def build_synth() -> str:
    src = os.path.join(ROOT, "synth", "gen.hip")
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-O2", "-fPIC", "-shared", "-std=c++17",
          "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-x", "hip", src, "-o", tmp])
    os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def build_all() -> None:
    with ThreadPoolExecutor(max_workers=2) as ex:
        a = ex.submit(build_product)
        b = ex.submit(build_synth)
        a.result()
        b.result()


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        if not os.path.exists(LIB):
            build_product()
        print(build_sanitized())
    else:
        build_all()
        print(LIB)
        print(SYNTH_LIB)
