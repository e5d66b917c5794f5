"""The C-ABI library loads, exports every function include/zero_shard.h declares, and rejects
bad arguments before touching the device (no kernel runs here)."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle
import zero_sharded_mixed_amd as Z
from zero_sharded_mixed_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_shard.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):  # not built yet: build it (hipcc cross-compiles without a GPU)
        from zero_sharded_mixed_amd import build
        build.build()
    return Z.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTS)


def test_probe_library_exports_its_header():
    """libzero_probe.so (the bandwidth probes beside the pipeline) exports every function
    include/zero_probe.h declares, and its binding names the same set."""
    from zero_sharded_mixed_amd import probe
    if not os.path.exists(probe.LIB_PATH):
        from zero_sharded_mixed_amd import build
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "zero_probe.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(zero_probe_[a-z_0-9]+)\s*\(", text)))
    assert declared == sorted(probe.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(zero_probe_\w+)$", out, flags=re.M))
    assert set(declared) <= exported
    L = probe.lib()
    for name in declared:
        assert hasattr(L, name)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(zero_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_small_grid_build_exports_the_same_symbols(L):
    """The small-grid build the GPU tests run (the same sources, grids capped at a few blocks)
    loads through the binding and exports every declared function; the binding's calls return
    to the main library when its block ends."""
    if not os.path.exists(B.SMALL_GRID_LIB_PATH):
        from zero_sharded_mixed_amd import build
        build.build()
    out = subprocess.run(["nm", "-D", "--defined-only", B.SMALL_GRID_LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(zero_\w+)$", out, flags=re.M))
    with B.library(B.SMALL_GRID_LIB_PATH) as S:
        assert B.lib() is S and S is not L
        for name in declared_functions():
            assert name in exported, name
            assert hasattr(S, name)
    assert B.lib() is L


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


@pytest.mark.parametrize("kw,status", [
    (dict(numels=[]), B.ZERO_EINVAL),
    (dict(numels=[5], nd=0), B.ZERO_EINVAL),
    (dict(numels=[5, -1]), B.ZERO_EINVAL),
    (dict(numels=[1 << 48]), B.ZERO_ERANGE),
])
def test_grouped_plan_create_rejects(L, kw, status):
    """The grouped entry point validates exactly as zero_plan_create (before any device work)."""
    numels = kw.pop("numels")
    arr = (ctypes.c_int64 * max(len(numels), 1))(*numels)
    groups = (ctypes.c_int32 * max(len(numels), 1))(*range(len(numels)))
    h = ctypes.c_void_p(123)
    args = dict(nd=8, rank=0, bucket_bytes=0, dtype=1)
    args.update(kw)
    st = L.zero_plan_create_grouped(arr, groups, len(numels), args["nd"], args["rank"], args["bucket_bytes"],
                                    args["dtype"], ctypes.byref(h))
    assert st == status and h.value is None


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
    cfg = B.zero_loss_scaler(2.0 ** 16, 0, 100, 2.0, 0.5, 1.0, 2.0 ** 24, 0)
    assert L.zero_loss_scaler_init(None, vp(16), None) == B.ZERO_EINVAL
    assert L.zero_loss_scaler_init(ctypes.byref(cfg), None, None) == B.ZERO_EINVAL
    assert L.zero_loss_scaler_init(ctypes.byref(cfg), vp(18), None) == B.ZERO_EINVAL  # misaligned
    assert L.zero_loss_scaler_update(None, vp(16), None) == B.ZERO_EINVAL
    assert L.zero_loss_scaler_update(vp(16), None, None) == B.ZERO_EINVAL
    s = B.zero_plan_summary()
    assert L.zero_plan_get_summary(None, ctypes.byref(s)) == B.ZERO_EINVAL
    L.zero_plan_destroy(None)  # no-op


@pytest.mark.parametrize("bad", [dict(scale=0.0), dict(scale=float("inf")), dict(scale=float("nan")),
                                 dict(min_scale=0.0, scale=1.0), dict(scale=0.5),  # below min_scale
                                 dict(scale=2.0 ** 25),  # above max_scale
                                 dict(growth_interval=0), dict(growth_factor=0.5), dict(backoff_factor=0.0),
                                 dict(backoff_factor=1.5), dict(good_steps=100), dict(good_steps=-1),
                                 dict(overflows=-1), dict(max_scale=float("inf"))])
def test_loss_scaler_init_rejects(L, bad):
    """Configuration checks happen on the host, before anything is launched."""
    f = dict(scale=2.0 ** 16, good_steps=0, growth_interval=100, growth_factor=2.0, backoff_factor=0.5,
             min_scale=1.0, max_scale=2.0 ** 24, overflows=0)
    f.update(bad)
    cfg = B.zero_loss_scaler(**f)
    assert L.zero_loss_scaler_init(ctypes.byref(cfg), ctypes.c_void_p(16), None) == B.ZERO_EINVAL
    assert Z.zero_last_error().startswith("zero_loss_scaler_init")


def test_struct_layouts_match_the_header(tmp_path):
    """The binding's ctypes structures have the C layout of include/zero_shard.h (gcc, host)."""
    structs = {"zero_loss_scaler": B.zero_loss_scaler, "zero_adam_hparams": B.zero_adam_hparams,
               "zero_param_info": B.zero_param_info, "zero_bucket_info": B.zero_bucket_info,
               "zero_plan_summary": B.zero_plan_summary}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "zero_shard.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'printf("{name} %zu\\n", sizeof({name}));')
        for fname, _ in cls._fields_:
            lines.append(f'printf("{name}.{fname} %zu\\n", offsetof({name}, {fname}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for name, cls in structs.items():
        assert int(got[name]) == ctypes.sizeof(cls), name
        for fname, _ in cls._fields_:
            assert int(got[f"{name}.{fname}"]) == getattr(cls, fname).offset, (name, fname)


@pytest.mark.parametrize("psi,nd", [(7.5e9, 64), (1.5e9, 1), (1e12, 1024), (123456789.0, 3)])
def test_accounting_matches_oracle(L, psi, nd):
    for stage in range(4):
        assert Z.zero_model_state_bytes(psi, nd, stage) == oracle.model_state_bytes(psi, nd, stage)
    out = ctypes.c_double()
    assert L.zero_model_state_bytes(psi, nd, 4, ctypes.byref(out)) == B.ZERO_EINVAL
    assert L.zero_model_state_bytes(psi, 0.5, 1, ctypes.byref(out)) == B.ZERO_EINVAL
    assert L.zero_model_state_bytes(-1.0, nd, 1, ctypes.byref(out)) == B.ZERO_EINVAL


def test_ptr_table_keeps_its_targets_alive(monkeypatch):
    """A pointer table must keep the tensors it points at allocated: a table that outlives
    them would send kernels (or a replayed graph) into freed memory.  Checked on CPU tensors,
    with the device check of the pointer helper stubbed out."""
    import gc
    import weakref

    import torch

    from zero_sharded_mixed_amd import _binding as B

    monkeypatch.setattr(B, "_ptr", lambda t: None if t is None else t.data_ptr())
    a, b = torch.zeros(16, dtype=torch.int16), torch.ones(8, dtype=torch.int16)
    wa, wb = weakref.ref(a), weakref.ref(b)
    table = B.ptr_table([a, None, b], device="cpu")
    assert table.tolist() == [a.data_ptr(), 0, b.data_ptr()]
    del a, b
    gc.collect()
    assert wa() is not None and wb() is not None
    del table
    gc.collect()
    assert wa() is None and wb() is None
