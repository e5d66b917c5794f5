"""The C-ABI library loads, exports every function include/zero_shard.h declares, and rejects
bad arguments before touching the device (no kernel runs here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import zero_sharded_mixed_amd as Z
from zero_sharded_mixed_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_shard.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):  # CPU-only container: build it (never on the GPU machine)
        from zero_sharded_mixed_amd import build
        build.build()
    return Z.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(zero_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def _create(L, numels, nd=8, rank=0, bucket_bytes=0, dtype=1, out=True):
    arr = (ctypes.c_int64 * max(len(numels), 1))(*numels)
    h = ctypes.c_void_p(123)
    st = L.zero_plan_create(arr, len(numels), nd, rank, bucket_bytes, dtype, ctypes.byref(h) if out else None)
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(numels=[]), B.ZERO_EINVAL),
    (dict(numels=[5], nd=0), B.ZERO_EINVAL),
    (dict(numels=[5], nd=65536), B.ZERO_EINVAL),
    (dict(numels=[5], rank=8), B.ZERO_EINVAL),
    (dict(numels=[5], rank=-1), B.ZERO_EINVAL),
    (dict(numels=[5, -1]), B.ZERO_EINVAL),
    (dict(numels=[5], bucket_bytes=-2), B.ZERO_EINVAL),
    (dict(numels=[5], dtype=3), B.ZERO_EINVAL),
    (dict(numels=[1 << 48]), B.ZERO_ERANGE),
    (dict(numels=[(1 << 47)] * 40000), B.ZERO_ERANGE),
])
def test_plan_create_rejects(L, kw, status):
    st, h = _create(L, **kw)
    assert st == status, Z.zero_last_error()
    assert h.value is None  # *out cleared on failure
    assert Z.zero_last_error().startswith("zero_plan_create")


def test_plan_create_null_out(L):
    st, _ = _create(L, [5], out=False)
    assert st == B.ZERO_EINVAL


def test_hot_calls_reject_null_plan(L):
    vp = ctypes.c_void_p
    assert L.zero_pack_bucket(None, 0, vp(16), vp(16), None) == B.ZERO_EINVAL
    assert L.zero_reduce_shard(None, 0, vp(16), 8, vp(16), vp(16), None, None) == B.ZERO_EINVAL
    assert L.zero_overflow_check(None, vp(16), vp(16), vp(16), None) == B.ZERO_EINVAL
    hp = B.zero_adam_hparams(1e-3, 0.9, 0.999, 1e-8, 1.0)
    assert L.zero_adam_step(None, vp(16), vp(16), vp(16), vp(16), vp(16), vp(16), ctypes.byref(hp), None, vp(16),
                            None) == B.ZERO_EINVAL
    assert L.zero_unpack(None, 0, vp(16), vp(16), None) == B.ZERO_EINVAL
    assert L.zero_shard_init(None, vp(16), 0, vp(16), None) == B.ZERO_EINVAL
    assert L.zero_pack_bucket_check(None, 0, vp(16), vp(16), vp(16), None) == B.ZERO_EINVAL
    assert L.zero_adam_prepare(None, vp(16), vp(16), ctypes.byref(hp), None, None) == B.ZERO_EINVAL
    assert L.zero_reduce_adam_bucket(None, 0, vp(16), 8, vp(16), vp(16), vp(16), vp(16), None, vp(16),
                                     None) == B.ZERO_EINVAL
    s = B.zero_plan_summary()
    assert L.zero_plan_get_summary(None, ctypes.byref(s)) == B.ZERO_EINVAL
    L.zero_plan_destroy(None)  # no-op


@pytest.mark.parametrize("psi,nd", [(7.5e9, 64), (1.5e9, 1), (1e12, 1024), (123456789.0, 3)])
def test_accounting_matches_oracle(L, psi, nd):
    for stage in range(4):
        assert Z.zero_model_state_bytes(psi, nd, stage) == oracle.model_state_bytes(psi, nd, stage)
    out = ctypes.c_double()
    assert L.zero_model_state_bytes(psi, nd, 4, ctypes.byref(out)) == B.ZERO_EINVAL
    assert L.zero_model_state_bytes(psi, 0.5, 1, ctypes.byref(out)) == B.ZERO_EINVAL
    assert L.zero_model_state_bytes(-1.0, nd, 1, ctypes.byref(out)) == B.ZERO_EINVAL
