"""The binding's argument checks, on the CPU: every buffer a kernel reads or writes through a
raw pointer is checked against the plan's sizes before anything is launched (a mis-sized
buffer would otherwise become an out-of-bounds device access).  Stand-in plan and tensor
objects carry exactly the attributes the checks read, so no device is needed; the GPU tests
drive the same checks through the real entry points."""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

from zero_sharded_mixed_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class FakePlan:
    """Sizes of a plan: 3 parameters (1000, 37, 5000 elements) at Nd = 8, one bucket."""
    n, nd, device = 3, 8, 0
    n_buckets = 1
    numels = np.array([1000, 37, 5000], dtype=np.int64)
    row_stride = [760]
    block_offset = [0]
    shard_numel = 760
    arena_numel = 8 * 760
    block_elems = B.Plan.block_elems
    rows_elems = B.Plan.rows_elems


class FakeTensor:
    """The attributes of a device tensor that the checks read."""

    def __init__(self, numel, dtype=torch.int16, device=0, contiguous=True):
        self._n, self.dtype, self._contig = numel, dtype, contiguous
        self.is_cuda = device is not None
        self.device = torch.device("cuda", device) if device is not None else torch.device("cpu")

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return 0x10000


def fake_table(tensors):
    t = FakeTensor(len(tensors), torch.int64)
    t.zero_targets = list(tensors)
    t.zero_numels = np.array([0 if x is None else x.numel() for x in tensors], dtype=np.int64)
    t.zero_elem_sizes = np.array([0 if x is None else x.element_size() for x in tensors], dtype=np.int64)
    t.zero_devices = {x.device.index for x in tensors if x is not None}
    return t


P = FakePlan()


def test_buffer_sizes_checked():
    assert B._buf(P, FakeTensor(P.block_elems(0)), "packed", P.block_elems(0), elem_size=2) == 0x10000
    with pytest.raises(ValueError, match="at least"):
        B._buf(P, FakeTensor(P.block_elems(0) - 1), "packed", P.block_elems(0), elem_size=2)
    with pytest.raises(ValueError, match="2-byte"):
        B._buf(P, FakeTensor(P.block_elems(0), torch.float32), "packed", P.block_elems(0), elem_size=2)
    with pytest.raises(ValueError, match="dtype"):
        B._buf(P, FakeTensor(P.shard_numel, torch.float16), "g32", P.shard_numel, B.F32)
    with pytest.raises(ValueError, match="cuda:0"):
        B._buf(P, FakeTensor(P.shard_numel, torch.float32, device=1), "g32", P.shard_numel, B.F32)
    with pytest.raises(ValueError, match="cuda:0"):
        B._buf(P, FakeTensor(P.shard_numel, torch.float32, device=None), "g32", P.shard_numel, B.F32)
    with pytest.raises(ValueError, match="contiguous"):
        B._buf(P, FakeTensor(P.shard_numel, torch.float32, contiguous=False), "g32", P.shard_numel, B.F32)
    assert B._buf(P, None, "flag", 1, B.I32) is None


def test_rows_extent_of_a_reduce():
    # rows of a reduce: row k at k * row_stride, the last one L_b long
    assert P.rows_elems(0, 760) == 7 * 760 + 760
    assert P.rows_elems(0, 1000) == 7 * 1000 + 760
    assert P.rows_elems(5, 760) == 0  # bad index: left to the library, which rejects it
    with pytest.raises(ValueError):
        B._buf(P, FakeTensor(7 * 1000 + 759), "rows", P.rows_elems(0, 1000), elem_size=2)


def test_pointer_tables_checked_entry_by_entry():
    ok = [FakeTensor(1000), FakeTensor(37), FakeTensor(5000)]
    assert B._table(P, fake_table(ok), "grads", 2) == 0x10000
    assert B._table(P, fake_table([ok[0], None, ok[2]]), "grads", 2) == 0x10000  # no gradient: NULL entry
    with pytest.raises(ValueError, match="entry 1 holds 36"):
        B._table(P, fake_table([ok[0], FakeTensor(36), ok[2]]), "unpack targets", 2)
    with pytest.raises(ValueError, match="4-byte"):
        B._table(P, fake_table(ok), "fp32 masters", 4)  # 16-bit sources passed as fp32 masters
    with pytest.raises(ValueError, match="entries"):
        B._table(P, fake_table(ok[:2]), "grads", 2)
    with pytest.raises(ValueError, match="cuda:0"):
        B._table(P, fake_table([ok[0], ok[1], FakeTensor(5000, device=1)]), "grads", 2)
    bare = FakeTensor(3, torch.int64)  # a copy or slice of a table carries no sizes
    with pytest.raises(ValueError, match="ptr_table"):
        B._table(P, bare, "grads", 2)


def test_empty_parameters_need_no_buffer():
    class Empty(FakePlan):
        numels = np.array([0, 0, 0], dtype=np.int64)
    # a zero-element parameter's entry is never dereferenced: any element size passes
    assert B._table(Empty(), fake_table([FakeTensor(0)] * 3), "fp32 masters", 4) == 0x10000


def test_grid_cap_keeps_dispatches_under_2_to_the_32():
    """grid_for at the extremes: never more than 2^23 blocks (2^31 work-items of 256 threads),
    never fewer than one."""
    src = os.path.join(ROOT, "zero_sharded_mixed_amd", "csrc")
    prog = r'''
#include <cstdio>
#include "zs_grid.h"
int main() {
    const long long cases[] = {-5, 0, 1, 255, 1LL << 23, (1LL << 23) + 1, 1LL << 31, 1LL << 40, 65535LL * 8388608};
    for (long long w : cases) std::printf("%lld %d\n", w, zs::grid_for(w));
    std::printf("cap4 %d\n", zs::grid_for(100, 4));
}
'''
    exe = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"zs_grid_test_{os.getpid()}")
    subprocess.run(["g++", "-std=c++17", "-I", src, "-x", "c++", "-", "-o", exe], input=prog, text=True, check=True)
    try:
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    finally:
        os.remove(exe)
    got = dict(line.split() for line in out if line)
    assert got["-5"] == "1" and got["0"] == "1" and got["1"] == "1" and got["255"] == "255"
    assert int(got[str(1 << 23)]) == 1 << 23
    for w in (str((1 << 23) + 1), str(1 << 31), str(1 << 40), str(65535 * 8388608)):
        assert int(got[w]) == 1 << 23  # 2^23 blocks x 256 threads = 2^31 work-items < 2^32
    assert got["cap4"] == "4"


def test_z3_step_pieces_checked():
    """Every bucket of every piece is checked against its own block size; piece lengths above
    the maximum and a row-stride list of the wrong length are refused."""
    ok = fake_table([FakeTensor(x) for x in P.numels])
    with pytest.raises(ValueError, match="at least"):
        B.zero_z3_step(P, gather_b0=0, gathered=[FakeTensor(P.block_elems(0) - 1)], param_ptrs=ok)
    with pytest.raises(ValueError, match="entry 2"):
        B.zero_z3_step(P, gather_b0=0, gathered=[FakeTensor(P.block_elems(0))],
                       param_ptrs=fake_table([FakeTensor(1000), None, FakeTensor(4999)]))
    with pytest.raises(ValueError, match="at least"):
        B.zero_z3_step(P, pack_b0=0, grad_ptrs=ok, packed=[FakeTensor(P.block_elems(0) - 8)])
    with pytest.raises(ValueError, match="at least"):  # rows of a reduce at a stride above L_b
        B.zero_z3_step(P, reduce_b0=0, rows=[FakeTensor(P.rows_elems(0, 800) - 1)], row_strides=[800],
                       live=FakeTensor(3, torch.uint8), g32=FakeTensor(P.shard_numel, torch.float32))
    with pytest.raises(ValueError, match="row strides"):
        B.zero_z3_step(P, reduce_b0=0, rows=[FakeTensor(P.rows_elems(0, 800))], row_strides=[])
    with pytest.raises(ValueError, match="at most"):
        B.zero_z3_step(P, gather_b0=0, gathered=[FakeTensor(1)] * (B.Z3_MAX_BUCKETS + 1), param_ptrs=ok)


def test_z3_pieces_layout_matches_the_header():
    """The ctypes mirror of zero_z3_pieces has the C struct's size and field offsets (the host
    compiler lays out the header's struct; x86-64 and the device share the layout rules)."""
    inc = os.path.join(ROOT, "include")
    fields = [f for f, _ in B.zero_z3_pieces._fields_]
    prog = "#include <cstdio>\n#include <cstddef>\n#include \"zero_shard.h\"\nint main() {\n"
    prog += '    std::printf("size %zu\\n", sizeof(zero_z3_pieces));\n'
    prog += "".join(f'    std::printf("{f} %zu\\n", offsetof(zero_z3_pieces, {f}));\n' for f in fields)
    prog += '    std::printf("max %d\\n", ZERO_Z3_MAX_BUCKETS);\n}\n'
    exe = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"zs_z3_layout_{os.getpid()}")
    subprocess.run(["g++", "-std=c++17", "-I", inc, "-x", "c++", "-", "-o", exe], input=prog, text=True, check=True)
    try:
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    finally:
        os.remove(exe)
    got = {k: int(v) for k, v in (line.split() for line in out if line)}
    assert got["max"] == B.Z3_MAX_BUCKETS
    assert got["size"] == ctypes.sizeof(B.zero_z3_pieces)
    for f in fields:
        assert got[f] == getattr(B.zero_z3_pieces, f).offset, f
