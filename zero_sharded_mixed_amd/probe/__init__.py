"""ctypes binding of libzero_probe.so (include/zero_probe.h): memory-bandwidth probes in the
pipeline kernels' access patterns, used by the benchmark to report achievable ceilings.
Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(_HERE, "libzero_probe.so")
EXPORTS = ("zero_probe_read", "zero_probe_write", "zero_probe_copy", "zero_probe_adam_streams")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build with zero_sharded_mixed_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        for name, args in (("zero_probe_read", [vp, i64, vp, vp]), ("zero_probe_write", [vp, i64, vp]),
                           ("zero_probe_copy", [vp, vp, i64, vp]),
                           ("zero_probe_adam_streams", [vp, vp, vp, vp, vp, i64, vp])):
            f = getattr(L, name)
            f.restype = ctypes.c_int32
            f.argtypes = args
        _lib = L
    return _lib


def _p(t: torch.Tensor) -> int:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("contiguous device tensor expected")
    return t.data_ptr()


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _s(stream) -> int:
    return (stream or torch.cuda.current_stream()).cuda_stream


def _ok(st: int, what: str) -> None:
    if st != 0:
        raise RuntimeError(f"{what}: status {st}")


def read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    if _nbytes(sink) < 16:
        raise ValueError("sink needs 16 bytes")
    _ok(lib().zero_probe_read(_p(src), _nbytes(src), _p(sink), _s(stream)), "zero_probe_read")


def write(dst: torch.Tensor, stream=None) -> None:
    _ok(lib().zero_probe_write(_p(dst), _nbytes(dst), _s(stream)), "zero_probe_write")


def copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    if _nbytes(dst) < _nbytes(src):
        raise ValueError("destination smaller than source")
    _ok(lib().zero_probe_copy(_p(src), _p(dst), _nbytes(src), _s(stream)), "zero_probe_copy")


def adam_streams(g, p, m, v, lp, stream=None) -> None:
    n = g.numel()
    for t, es in ((g, 4), (p, 4), (m, 4), (v, 4), (lp, 2)):
        if t.numel() < n or t.element_size() != es:
            raise ValueError("adam_streams: four fp32 arrays and one 16-bit array of n elements expected")
    if n % 2048:
        raise ValueError("adam_streams: n must be a multiple of 2048 (whole 2048-column spans)")
    _ok(lib().zero_probe_adam_streams(_p(g), _p(p), _p(m), _p(v), _p(lp), n, _s(stream)), "zero_probe_adam_streams")
