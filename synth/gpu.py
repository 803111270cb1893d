"""Device-side twin of the seeded generators (``synth/gen.hip``), for inputs too
large to draw on the host. Produces the same bits as ``synth.normals`` and
friends; a GPU test checks that on samples. No method arithmetic here.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch  # first: binds the library to torch's HIP runtime

from . import stream_key  # noqa: F401  (same stream definition as the host side)

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtqsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} missing: run `python -m kv_cache_vector_03_amd.build`")
        L = C.CDLL(_LIB_PATH)
        vp = C.c_void_p
        L.synth_fill_f16.argtypes = [C.c_uint64, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_int64,
                                     vp, vp, vp]
        L.synth_fill_f32.argtypes = [C.c_uint64, C.c_int, C.c_int64, C.c_int64, vp, vp]
        L.synth_unit_f32.argtypes = [C.c_uint64, C.c_int, C.c_int64, C.c_int64, C.c_int, vp, vp]
        for f in (L.synth_fill_f16, L.synth_fill_f32, L.synth_unit_f32):
            f.restype = C.c_int
        _lib = L
    return _lib


def _s():
    return torch.cuda.current_stream().cuda_stream


def fill_f16(out: torch.Tensor, seed: int, role: int, first: int = 0, d: int = 1, tokens: int = 1,
             scales: torch.Tensor | None = None) -> torch.Tensor:
    """out.flat[i] = fp16(fp32(normal(first + i) * scales[group, channel]))."""
    assert out.dtype == torch.float16 and out.is_contiguous()
    if scales is not None:
        assert scales.dtype == torch.float64 and scales.is_cuda
    rc = lib().synth_fill_f16(seed % (1 << 64), role, first, out.numel(), d, tokens,
                              scales.data_ptr() if scales is not None else None, out.data_ptr(), _s())
    if rc:
        raise RuntimeError("synth_fill_f16 launch failed")
    return out


def fill_f32(out: torch.Tensor, seed: int, role: int, first: int = 0) -> torch.Tensor:
    assert out.dtype == torch.float32 and out.is_contiguous()
    if lib().synth_fill_f32(seed % (1 << 64), role, first, out.numel(), out.data_ptr(), _s()):
        raise RuntimeError("synth_fill_f32 launch failed")
    return out


def unit_f32(out: torch.Tensor, seed: int, role: int, first_vec: int = 0) -> torch.Tensor:
    assert out.dtype == torch.float32 and out.is_contiguous() and out.dim() == 2
    if lib().synth_unit_f32(seed % (1 << 64), role, first_vec, out.shape[0], out.shape[1],
                            out.data_ptr(), _s()):
        raise RuntimeError("synth_unit_f32 launch failed")
    return out


def scales_to_device(scales: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(scales, np.float64)).to(device)
