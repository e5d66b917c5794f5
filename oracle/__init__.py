"""CPU oracle of the ZeRO-1/2 per-rank shard pipeline — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The arithmetic lives in ``zero_oracle.c`` (plain C, one
IEEE-754 operation per source operation, fp64 for Adam); this module only marshals numpy
arrays into it.  It shares no code with the GPU library.

Pages the C functions follow (title, section): ColossalAI issue "[zero] improving
compatibility of low level zero" (Design: INIT, BWD, Optim); briefia.fr "L'IA sur
plusieurs GPU : ZeRO et FSDP" (Implémentation simplifiée); llm-engineer card "ZeRO-3"
(the ZeRO-1/2 all-gather); upskillscore summary of "ZeRO: Memory Optimizations Toward
Training Trillion Parameter Models" (model states, ZeRO-DP stages).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zero_oracle.c")
_LIB = os.path.join(_HERE, "libzero_oracle.so")

BF16 = 1
FP16 = 2

# Parameter record fields (the order of the C enum).
P_NUMEL, P_PAD, P_PADDED, P_SHARD, P_START, P_END, P_OFFSET, P_BUCKET, P_COL = range(9)
# Bucket record fields.
B_FIRST, B_COUNT, B_ROW, B_STRIDE, B_BASE = range(5)

GCC_FLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
             "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror"]
# ORACLE_SANITIZE=1: build with AddressSanitizer and UBSan (host code; run the tests with
# LD_PRELOAD of gcc's libasan.so and libubsan.so and ASAN_OPTIONS=detect_leaks=0)
SANITIZE_FLAGS = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_library(force: bool = True) -> str:
    """Compile zero_oracle.c with gcc into libzero_oracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        extra = SANITIZE_FLAGS if os.environ.get("ORACLE_SANITIZE") == "1" else []
        subprocess.run(["gcc", *GCC_FLAGS, *extra, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build_library(force=False)
        L = ctypes.CDLL(_LIB)
        i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        L.oracle_plan.restype = i64
        L.oracle_plan.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
        L.oracle_pack_bucket.restype = None
        L.oracle_pack_bucket.argtypes = [vp, vp, i64, i64, vp, vp]
        L.oracle_reduce_column.restype = ctypes.c_float
        L.oracle_reduce_column.argtypes = [vp, i64, i64, i32]
        L.oracle_reduce_bucket.restype = None
        L.oracle_reduce_bucket.argtypes = [vp, vp, i64, i64, vp, i64, i32, vp, vp]
        L.oracle_overflow.restype = i32
        L.oracle_loss_scaler_update.restype = None
        L.oracle_loss_scaler_update.argtypes = [vp, i32]
        L.oracle_input_check.restype = i32
        L.oracle_input_check.argtypes = [vp, vp, i64, i64, vp, i32]
        L.oracle_overflow.argtypes = [vp, i64, vp, vp]
        L.oracle_adam_element.restype = None
        L.oracle_adam_element.argtypes = [ctypes.c_float, vp, vp, vp, i64, dbl, dbl, dbl, dbl, dbl]
        L.oracle_adam.restype = None
        L.oracle_adam.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, dbl, dbl, dbl, dbl, dbl, i32,
                                  vp, i32]
        L.oracle_unpack_bucket.restype = None
        L.oracle_unpack_bucket.argtypes = [vp, vp, i64, vp, vp]
        L.oracle_shard_init.restype = None
        L.oracle_shard_init.argtypes = [vp, vp, i64, i64, vp, i32, vp]
        L.oracle_pack_locate.restype = i32
        L.oracle_pack_locate.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        L.oracle_unpack_locate.restype = None
        L.oracle_unpack_locate.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_get_threads.restype = i32
        L.oracle_get_threads.argtypes = []
        L.oracle_model_state_bytes.restype = dbl
        L.oracle_model_state_bytes.argtypes = [dbl, dbl, i32]
        for name in ("oracle_convert_to_f32", "oracle_convert_from_f32"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [vp, vp, i64, i32]
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Host threads for the oracle's element loops (default 1).  Each loop over one
    parameter's columns is split into disjoint ranges; results are identical for any count."""
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _ptr_table(arrays) -> np.ndarray:
    """uint64 array of host addresses (0 for None)."""
    return np.array([0 if a is None else _ptr(a) for a in arrays], dtype=np.uint64)


@dataclass
class Plan:
    params: np.ndarray   # int64 [n, 9]
    buckets: np.ndarray  # int64 [n_buckets, 5]
    shard_len: int       # sum of row strides = length of every fp32 shard array
    nd: int
    rank: int

    @property
    def n(self) -> int:
        return self.params.shape[0]

    @property
    def n_buckets(self) -> int:
        return self.buckets.shape[0]

    def bucket_params(self, b: int) -> range:
        first, count = self.buckets[b, B_FIRST], self.buckets[b, B_COUNT]
        return range(int(first), int(first + count))


def plan(numels, nd: int, rank: int, bucket_bytes: int, groups=None) -> Plan:
    """groups: one int32 id per parameter (a bucket never spans a change of id), or None."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    n = numels.shape[0]
    if groups is not None:
        groups = np.ascontiguousarray(groups, dtype=np.int32)
        assert groups.shape == (n,)
    params = np.zeros((max(n, 1), 9), dtype=np.int64)
    buckets = np.zeros((max(n, 1), 5), dtype=np.int64)
    shard_len = np.zeros(1, dtype=np.int64)
    nb = lib().oracle_plan(_ptr(numels), None if groups is None else _ptr(groups), n, nd, rank, bucket_bytes,
                           _ptr(params), _ptr(buckets), _ptr(shard_len))
    if nb < 0:
        raise ValueError("oracle_plan: invalid arguments")
    return Plan(params[:n].copy(), buckets[:nb].copy(), int(shard_len[0]), nd, rank)


def pack_bucket(pl: Plan, b: int, grads, out: np.ndarray | None = None) -> np.ndarray:
    """grads: list (length n) of uint16 arrays or None.  Returns uint16 [nd, L_b]."""
    L = int(pl.buckets[b, B_STRIDE])
    if out is None:
        out = np.zeros((pl.nd, L), dtype=np.uint16)
    assert out.shape == (pl.nd, L) and out.dtype == np.uint16
    keep = [None if g is None else np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    table = _ptr_table(keep)
    lib().oracle_pack_bucket(_ptr(pl.params), _ptr(pl.buckets), pl.nd, b, _ptr(table), _ptr(out))
    return out


def reduce_column(vals: np.ndarray, dtype: int) -> np.float32:
    vals = np.ascontiguousarray(vals, dtype=np.uint16)
    return np.float32(lib().oracle_reduce_column(_ptr(vals), vals.shape[0], 1, dtype))


def reduce_bucket(pl: Plan, b: int, rows: np.ndarray, dtype: int, live: np.ndarray, g32: np.ndarray) -> None:
    """rows: uint16 [nd, row_stride]; writes g32 (float32 [shard_len]) in place."""
    assert rows.dtype == np.uint16 and rows.ndim == 2 and rows.shape[0] == pl.nd
    assert rows.shape[1] >= pl.buckets[b, B_STRIDE] and rows.flags["C_CONTIGUOUS"]
    assert g32.dtype == np.float32 and g32.shape == (pl.shard_len,)
    live = np.ascontiguousarray(live, dtype=np.uint8)
    lib().oracle_reduce_bucket(_ptr(pl.params), _ptr(pl.buckets), pl.nd, b, _ptr(rows), rows.shape[1], dtype,
                               _ptr(live), _ptr(g32))


def overflow(pl: Plan, g32: np.ndarray, live: np.ndarray) -> int:
    live = np.ascontiguousarray(live, dtype=np.uint8)
    return int(lib().oracle_overflow(_ptr(pl.params), pl.n, _ptr(g32), _ptr(live)))


def input_check(pl: Plan, b: int, grads, dtype: int) -> int:
    """Verdict of the fused path's input check over bucket b's gradients (list, None = no gradient)."""
    keep = [None if g is None else np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    table = _ptr_table(keep)
    return int(lib().oracle_input_check(_ptr(pl.params), _ptr(pl.buckets), pl.nd, b, _ptr(table), dtype))


class Scaler(ctypes.Structure):
    """The oracle's loss-scaler state (its own definition of the fields)."""
    _fields_ = [("scale", ctypes.c_float), ("good_steps", ctypes.c_int32), ("growth_interval", ctypes.c_int32),
                ("growth_factor", ctypes.c_float), ("backoff_factor", ctypes.c_float), ("min_scale", ctypes.c_float),
                ("max_scale", ctypes.c_float), ("overflows", ctypes.c_int32)]

    def as_tuple(self):
        return tuple(getattr(self, f) for f, _ in self._fields_)


def loss_scaler_update(s: Scaler, flag: int) -> None:
    """One step of the dynamic loss-scaling rule, in place."""
    lib().oracle_loss_scaler_update(ctypes.byref(s), int(flag))


@dataclass
class AdamHP:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    grad_scale: float = 1.0


def adam_element(g32: float, p32: float, m: float, v: float, t: int, hp: AdamHP):
    """One element; returns the new (p32, m, v) as float32."""
    P = np.array([p32], dtype=np.float32)
    M = np.array([m], dtype=np.float32)
    V = np.array([v], dtype=np.float32)
    lib().oracle_adam_element(float(np.float32(g32)), _ptr(P), _ptr(M), _ptr(V), t, hp.lr, hp.beta1, hp.beta2,
                              hp.eps, hp.grad_scale)
    return P[0], M[0], V[0]


def adam(pl: Plan, g32, p32, m, v, live, steps, hp: AdamHP, flag: int, arena: np.ndarray, dtype: int) -> None:
    """In place on p32, m, v (float32 [shard_len]), steps (int32 [n]) and arena
    (uint16 [nd * shard_len])."""
    for a in (g32, p32, m, v):
        assert a.dtype == np.float32 and a.shape == (pl.shard_len,) and a.flags["C_CONTIGUOUS"]
    assert steps.dtype == np.int32 and steps.shape == (pl.n,)
    assert arena.dtype == np.uint16 and arena.size == pl.nd * pl.shard_len and arena.flags["C_CONTIGUOUS"]
    live = np.ascontiguousarray(live, dtype=np.uint8)
    lib().oracle_adam(_ptr(pl.params), _ptr(pl.buckets), pl.n, pl.nd, pl.rank, _ptr(g32), _ptr(p32), _ptr(m),
                      _ptr(v), _ptr(live), _ptr(steps), hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale,
                      int(flag), _ptr(arena), dtype)


def unpack_bucket(pl: Plan, b: int, gathered: np.ndarray, outs) -> None:
    """gathered: uint16 [nd, L_b]; outs: list (length n) of uint16 arrays (written) or None."""
    assert gathered.dtype == np.uint16 and gathered.shape == (pl.nd, pl.buckets[b, B_STRIDE])
    gathered = np.ascontiguousarray(gathered)
    for o in outs:
        assert o is None or (o.dtype == np.uint16 and o.flags["C_CONTIGUOUS"])
    table = _ptr_table(outs)
    lib().oracle_unpack_bucket(_ptr(pl.params), _ptr(pl.buckets), b, _ptr(gathered), _ptr(table))


def shard_init(pl: Plan, masters, p32: np.ndarray, src_dtype: int = 0) -> None:
    """masters: list of float32 (src_dtype 0) or uint16 (BF16 / FP16) flat arrays, or None."""
    assert p32.dtype == np.float32 and p32.shape == (pl.shard_len,)
    want = np.float32 if src_dtype == 0 else np.uint16
    keep = [None if a is None else np.ascontiguousarray(a, dtype=want) for a in masters]
    table = _ptr_table(keep)
    lib().oracle_shard_init(_ptr(pl.params), _ptr(pl.buckets), pl.n, pl.n_buckets, _ptr(table), src_dtype,
                            _ptr(p32))


def pack_locate(pl: Plan, b: int, k: int, c: int):
    """(kind, i, e): kind 0 = row gap, 1 = gradient element e of parameter i, 2 = padding."""
    out = np.zeros(2, dtype=np.int64)
    kind = lib().oracle_pack_locate(_ptr(pl.params), _ptr(pl.buckets), b, k, c, out.ctypes.data,
                                    out.ctypes.data + 8)
    return int(kind), int(out[0]), int(out[1])


def unpack_locate(pl: Plan, i: int, e: int):
    """(row, col) of the bucket block that element e of parameter i is read from."""
    out = np.zeros(2, dtype=np.int64)
    lib().oracle_unpack_locate(_ptr(pl.params), i, e, out.ctypes.data, out.ctypes.data + 8)
    return int(out[0]), int(out[1])


def model_state_bytes(psi: float, nd: float, stage: int) -> float:
    return float(lib().oracle_model_state_bytes(psi, nd, stage))


def to_f32(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().oracle_convert_to_f32(_ptr(bits), _ptr(out), bits.size, dtype)
    return out


def from_f32(vals: np.ndarray, dtype: int) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(vals.shape, dtype=np.uint16)
    lib().oracle_convert_from_f32(_ptr(vals), _ptr(out), vals.size, dtype)
    return out
