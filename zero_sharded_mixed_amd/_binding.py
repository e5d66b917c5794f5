"""ctypes binding of libzero_shard.so — argument marshalling only.

Every function here has the name of the C entry point it calls (include/zero_shard.h) and
does nothing but turn torch tensors into device pointers, pick the stream and raise on a
non-zero status.  All arithmetic of the shard pipeline runs in the HIP kernels; there is no
CPU fallback: if the library is missing, the first call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_shard.so")
SMALL_GRID_LIB_PATH = os.path.join(_HERE, "libzero_shard_smallgrid.so")  # grids capped at a few blocks

ZERO_OK, ZERO_EINVAL, ZERO_ENOMEM, ZERO_EHIP, ZERO_ERANGE = 0, -1, -2, -3, -4
ZERO_BF16, ZERO_FP16 = 1, 2
STATUS_NAMES = {0: "ZERO_OK", -1: "ZERO_EINVAL", -2: "ZERO_ENOMEM", -3: "ZERO_EHIP", -4: "ZERO_ERANGE"}

# Every symbol the header declares (checked against the header by the ABI test).
EXPORTS = ("zero_plan_create", "zero_plan_create_grouped", "zero_plan_destroy", "zero_plan_get_summary",
           "zero_plan_param_info", "zero_plan_bucket_info", "zero_model_state_bytes", "zero_plan_model_state_bytes",
           "zero_pack_bucket", "zero_reduce_shard", "zero_overflow_check", "zero_adam_step", "zero_unpack",
           "zero_shard_init", "zero_pack_bucket_check", "zero_adam_prepare", "zero_reduce_adam_bucket",
           "zero_loss_scaler_init", "zero_loss_scaler_update", "zero_last_error", "zero_adam_step_noalloc",
           "zero_z3_layer_step", "zero_z3_step")
ADAM_NOALLOC_MAX_PARAMS = 131072  # ZERO_ADAM_NOALLOC_MAX_PARAMS
Z3_MAX_BUCKETS = 4                # ZERO_Z3_MAX_BUCKETS


class ZeroError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class zero_param_info(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("numel", "pad", "padded_numel", "shard_size", "shard_start", "shard_end",
                                             "shard_offset", "bucket", "bucket_col")]


class zero_bucket_info(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("first_param", "n_params", "row_elems", "row_stride", "shard_base",
                                             "block_offset")]


class zero_plan_summary(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("n_params", "nd", "rank", "n_buckets", "shard_numel", "shard_elems",
                                             "numel_total", "padded_total", "bucket_elems", "arena_numel")] + \
               [("dtype", ctypes.c_int32), ("device", ctypes.c_int32)]


class zero_loss_scaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("good_steps", ctypes.c_int32), ("growth_interval", ctypes.c_int32),
                ("growth_factor", ctypes.c_float), ("backoff_factor", ctypes.c_float), ("min_scale", ctypes.c_float),
                ("max_scale", ctypes.c_float), ("overflows", ctypes.c_int32)]


class zero_z3_pieces(ctypes.Structure):
    _fields_ = [("reduce_b0", ctypes.c_int64), ("reduce_n", ctypes.c_int64),
                ("rows", ctypes.c_void_p * Z3_MAX_BUCKETS), ("row_stride", ctypes.c_int64 * Z3_MAX_BUCKETS),
                ("live", ctypes.c_void_p), ("g32", ctypes.c_void_p),
                ("pack_b0", ctypes.c_int64), ("pack_n", ctypes.c_int64), ("grad_ptrs", ctypes.c_void_p),
                ("packed", ctypes.c_void_p * Z3_MAX_BUCKETS), ("check", ctypes.c_int32),
                ("gather_b0", ctypes.c_int64), ("gather_n", ctypes.c_int64),
                ("gathered", ctypes.c_void_p * Z3_MAX_BUCKETS), ("param_ptrs", ctypes.c_void_p),
                ("flag", ctypes.c_void_p)]


class zero_adam_hparams(ctypes.Structure):
    _fields_ = [(f, ctypes.c_double) for f in ("lr", "beta1", "beta2", "eps", "grad_scale")] + \
               [("loss_scaler", ctypes.c_void_p)]


_lib = None
LOSS_SCALER_BYTES = ctypes.sizeof(zero_loss_scaler)


def _scaler(plan: "Plan", t: Optional[torch.Tensor], what: str) -> Optional[int]:
    if t is None:
        return None
    if t.numel() * t.element_size() < LOSS_SCALER_BYTES:
        raise ValueError(f"{what}: loss scaler tensor too small")
    return _buf(plan, t, what + ": loss scaler", 0)


def lib() -> ctypes.CDLL:
    """Load libzero_shard.so (built in place by zero_sharded_mixed_amd/build.py)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route the binding's calls to another build of the same sources while the block runs (the
    tests run the build whose grids are capped at a few blocks through it); plans made inside
    are destroyed by the library that made them."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


_loaded = {}


def _load(path: str) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: the HIP library is not built "
                           "(python zero_sharded_mixed_amd/build.py); there is no fallback")
    L = ctypes.CDLL(path)
    i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
    sigs = {
        "zero_plan_create": (i32, [vp, i64, i32, i32, i64, i32, ctypes.POINTER(vp)]),
        "zero_plan_create_grouped": (i32, [vp, vp, i64, i32, i32, i64, i32, ctypes.POINTER(vp)]),
        "zero_plan_destroy": (None, [vp]),
        "zero_plan_get_summary": (i32, [vp, ctypes.POINTER(zero_plan_summary)]),
        "zero_plan_param_info": (i32, [vp, i64, ctypes.POINTER(zero_param_info)]),
        "zero_plan_bucket_info": (i32, [vp, i64, ctypes.POINTER(zero_bucket_info)]),
        "zero_model_state_bytes": (i32, [dbl, dbl, i32, ctypes.POINTER(dbl)]),
        "zero_plan_model_state_bytes": (i32, [vp, i32, ctypes.POINTER(dbl)]),
        "zero_pack_bucket": (i32, [vp, i64, vp, vp, vp]),
        "zero_reduce_shard": (i32, [vp, i64, vp, i64, vp, vp, vp, vp]),
        "zero_overflow_check": (i32, [vp, vp, vp, vp, vp]),
        "zero_adam_step": (i32, [vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(zero_adam_hparams), vp, vp, vp]),
        "zero_adam_step_noalloc": (i32, [vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(zero_adam_hparams), vp, vp, vp]),
        "zero_unpack": (i32, [vp, i64, vp, vp, vp]),
        "zero_z3_layer_step": (i32, [vp, i64, vp, i64, vp, vp, i64, vp, vp, i32, i64, vp, vp, vp, vp]),
        "zero_z3_step": (i32, [vp, ctypes.POINTER(zero_z3_pieces), vp]),
        "zero_shard_init": (i32, [vp, vp, i32, vp, vp]),
        "zero_pack_bucket_check": (i32, [vp, i64, vp, vp, vp, vp]),
        "zero_adam_prepare": (i32, [vp, vp, vp, ctypes.POINTER(zero_adam_hparams), vp, vp]),
        "zero_reduce_adam_bucket": (i32, [vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp]),
        "zero_loss_scaler_init": (i32, [ctypes.POINTER(zero_loss_scaler), vp, vp]),
        "zero_loss_scaler_update": (i32, [vp, vp, vp]),
        "zero_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _loaded[path] = L
    return L


def _check(status: int) -> None:
    if status != ZERO_OK:
        raise ZeroError(status, lib().zero_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _buf(plan: "Plan", t: Optional[torch.Tensor], what: str, min_elems: int, dtypes=None,
         elem_size: Optional[int] = None) -> Optional[int]:
    """Pointer of a buffer a kernel will read or write: on the plan's device, contiguous, of an
    allowed dtype (or element size) and holding at least min_elems elements.  Raises
    ValueError otherwise, before anything is launched.  None passes through (the library
    decides whether NULL is allowed)."""
    if t is None:
        return None
    if not t.is_cuda or t.device.index != plan.device:
        raise ValueError(f"{what}: tensor must live on cuda:{plan.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: contiguous tensor expected")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype} not in {tuple(dtypes)}")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{what}: {elem_size}-byte elements expected, got {t.dtype}")
    if t.numel() < min_elems:
        raise ValueError(f"{what}: {t.numel()} elements, at least {min_elems} needed")
    return t.data_ptr()


F32 = (torch.float32,)
I32 = (torch.int32,)
U8 = (torch.uint8, torch.bool)


def ptr_table(tensors: Sequence[Optional[torch.Tensor]], device=None) -> torch.Tensor:
    """Device int64 array of the tensors' data pointers (0 for None): a pointer table.

    The returned tensor holds references to the tensors it points at (attribute
    `zero_targets`), so their memory stays allocated for as long as the table object is alive:
    a kernel that reads through the table, at once or when a captured graph is replayed, never
    reads memory that the caching allocator has freed or handed back to the driver.  A slice or
    copy of the table is a new tensor object and carries neither the references nor the sizes
    below, so the entry points refuse it.  It also records every entry's element count and
    element size (`zero_numels`, `zero_elem_sizes`; 0 for None), which the entry points check
    against the plan before they launch."""
    keep = list(tensors)
    ptrs = [0 if t is None else _ptr(t) for t in keep]
    table = torch.tensor(ptrs, dtype=torch.int64, device=device or "cuda")
    table.zero_targets = keep
    table.zero_numels = np.array([0 if t is None else t.numel() for t in keep], dtype=np.int64)
    table.zero_elem_sizes = np.array([0 if t is None else t.element_size() for t in keep], dtype=np.int64)
    table.zero_devices = {t.device.index for t in keep if t is not None}
    return table


def _table(plan: "Plan", table: torch.Tensor, what: str, elem_size: int) -> int:
    """Pointer of a pointer table after checking, entry by entry, that every non-NULL entry
    of a parameter with elements is a buffer of elem_size-byte elements on the plan's device
    holding at least numel_i elements (a kernel reads or writes that many through it)."""
    numels = getattr(table, "zero_numels", None)
    if numels is None:
        raise ValueError(f"{what}: pointer table must come from ptr_table() (a slice or copy drops its sizes)")
    if table.numel() != plan.n or numels.shape[0] != plan.n:
        raise ValueError(f"{what}: pointer table has {table.numel()} entries, the plan {plan.n} parameters")
    # entries of parameters with no elements are never dereferenced
    present = (table.zero_elem_sizes != 0) & (plan.numels > 0)
    if np.any(table.zero_elem_sizes[present] != elem_size):
        raise ValueError(f"{what}: every buffer in the table must have {elem_size}-byte elements")
    short = present & (numels < plan.numels)
    if np.any(short):
        i = int(np.flatnonzero(short)[0])
        raise ValueError(f"{what}: entry {i} holds {int(numels[i])} elements, parameter {i} has {int(plan.numels[i])}")
    if table.zero_devices - {plan.device}:
        raise ValueError(f"{what}: every buffer in the table must live on cuda:{plan.device}")
    return _buf(plan, table, what + " table", plan.n, dtypes=(torch.int64,))


class Plan:
    """Owns a zero_plan*; destroyed with the object (or by close()).  Keeps the sizes the
    entry points' argument checks need: per-parameter numel, per-bucket row stride and block
    offset, the shard and arena lengths."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        self._lib = lib()  # the library that made the plan destroys it
        s = zero_plan_summary()
        _check(lib().zero_plan_get_summary(self._h, ctypes.byref(s)))
        self.n, self.nd, self.device = int(s.n_params), int(s.nd), int(s.device)
        self.n_buckets, self.shard_numel, self.arena_numel = int(s.n_buckets), int(s.shard_numel), int(s.arena_numel)
        info = zero_param_info()
        numels = np.zeros(self.n, dtype=np.int64)
        for i in range(self.n):
            _check(lib().zero_plan_param_info(self._h, i, ctypes.byref(info)))
            numels[i] = info.numel
        self.numels = numels
        bk = zero_bucket_info()
        self.row_stride, self.block_offset = [], []
        for b in range(self.n_buckets):
            _check(lib().zero_plan_bucket_info(self._h, b, ctypes.byref(bk)))
            self.row_stride.append(int(bk.row_stride))
            self.block_offset.append(int(bk.block_offset))

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("plan is closed")
        return self._h

    def block_elems(self, b: int) -> int:
        """Elements of bucket b's [Nd][L_b] block (0 for an index out of range: the library
        rejects the index)."""
        return self.nd * self.row_stride[b] if 0 <= b < self.n_buckets else 0

    def rows_elems(self, b: int, row_stride: int) -> int:
        """Elements a reduce of bucket b reads from its rows buffer."""
        if not 0 <= b < self.n_buckets or self.row_stride[b] == 0:
            return 0
        return (self.nd - 1) * max(int(row_stride), 0) + self.row_stride[b]

    def close(self) -> None:
        if self._h:
            self._lib.zero_plan_destroy(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def zero_plan_create(numels: Sequence[int], nd: int, rank: int, bucket_bytes: int, dtype: int) -> Plan:
    arr = (ctypes.c_int64 * max(len(numels), 1))(*[int(x) for x in numels])
    out = ctypes.c_void_p()
    _check(lib().zero_plan_create(arr, len(numels), nd, rank, bucket_bytes, dtype, ctypes.byref(out)))
    return Plan(out.value)


def zero_plan_create_grouped(numels: Sequence[int], groups: Optional[Sequence[int]], nd: int, rank: int,
                             bucket_bytes: int, dtype: int) -> Plan:
    arr = (ctypes.c_int64 * max(len(numels), 1))(*[int(x) for x in numels])
    if groups is not None and len(groups) != len(numels):
        raise ValueError("one group id per parameter")
    garr = None if groups is None else (ctypes.c_int32 * max(len(groups), 1))(*[int(x) for x in groups])
    out = ctypes.c_void_p()
    _check(lib().zero_plan_create_grouped(arr, garr, len(numels), nd, rank, bucket_bytes, dtype, ctypes.byref(out)))
    return Plan(out.value)


def zero_plan_destroy(plan: Plan) -> None:
    plan.close()


def zero_plan_get_summary(plan: Plan) -> zero_plan_summary:
    s = zero_plan_summary()
    _check(lib().zero_plan_get_summary(plan.handle, ctypes.byref(s)))
    return s


def zero_plan_param_info(plan: Plan, i: int) -> zero_param_info:
    s = zero_param_info()
    _check(lib().zero_plan_param_info(plan.handle, i, ctypes.byref(s)))
    return s


def zero_plan_bucket_info(plan: Plan, b: int) -> zero_bucket_info:
    s = zero_bucket_info()
    _check(lib().zero_plan_bucket_info(plan.handle, b, ctypes.byref(s)))
    return s


def zero_model_state_bytes(psi: float, nd: float, stage: int) -> float:
    out = ctypes.c_double()
    _check(lib().zero_model_state_bytes(psi, nd, stage, ctypes.byref(out)))
    return out.value


def zero_plan_model_state_bytes(plan: Plan, stage: int) -> float:
    out = ctypes.c_double()
    _check(lib().zero_plan_model_state_bytes(plan.handle, stage, ctypes.byref(out)))
    return out.value


def zero_pack_bucket(plan: Plan, b: int, grad_ptrs: torch.Tensor, packed: torch.Tensor, stream=None) -> None:
    _check(lib().zero_pack_bucket(plan.handle, b, _table(plan, grad_ptrs, "zero_pack_bucket: gradients", 2),
                                  _buf(plan, packed, "zero_pack_bucket: packed", plan.block_elems(b), elem_size=2),
                                  _stream(stream)))


def zero_reduce_shard(plan: Plan, b: int, rows: torch.Tensor, row_stride: int, live: torch.Tensor,
                      g32: torch.Tensor, flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """rows: 16-bit device tensor whose start is row 0; row k starts k*row_stride elements in."""
    _check(lib().zero_reduce_shard(plan.handle, b, _buf(plan, rows, "zero_reduce_shard: rows",
                                                        plan.rows_elems(b, row_stride), elem_size=2),
                                   row_stride, _buf(plan, live, "zero_reduce_shard: live", plan.n, U8),
                                   _buf(plan, g32, "zero_reduce_shard: g32", plan.shard_numel, F32),
                                   _buf(plan, flag, "zero_reduce_shard: flag", 1, I32), _stream(stream)))


def zero_overflow_check(plan: Plan, g32: torch.Tensor, live: torch.Tensor, flag: torch.Tensor, stream=None) -> None:
    _check(lib().zero_overflow_check(plan.handle, _buf(plan, g32, "zero_overflow_check: g32", plan.shard_numel, F32),
                                     _buf(plan, live, "zero_overflow_check: live", plan.n, U8),
                                     _buf(plan, flag, "zero_overflow_check: flag", 1, I32), _stream(stream)))


def zero_adam_step(plan: Plan, g32: torch.Tensor, p32: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
                   live: torch.Tensor, steps: torch.Tensor, lr: float, beta1: float, beta2: float, eps: float,
                   grad_scale: float, flag: Optional[torch.Tensor], arena: torch.Tensor, stream=None,
                   loss_scaler: Optional[torch.Tensor] = None) -> None:
    """loss_scaler: device tensor holding a zero_loss_scaler (see LOSS_SCALER_BYTES), or None."""
    S, w = plan.shard_numel, "zero_adam_step"
    hp = zero_adam_hparams(lr, beta1, beta2, eps, grad_scale, _scaler(plan, loss_scaler, w))
    _check(lib().zero_adam_step(plan.handle, _buf(plan, g32, w + ": g32", S, F32), _buf(plan, p32, w + ": p32", S, F32),
                                _buf(plan, m, w + ": m", S, F32), _buf(plan, v, w + ": v", S, F32),
                                _buf(plan, live, w + ": live", plan.n, U8), _buf(plan, steps, w + ": steps", plan.n, I32),
                                ctypes.byref(hp), _buf(plan, flag, w + ": flag", 1, I32),
                                _buf(plan, arena, w + ": arena", plan.arena_numel, elem_size=2), _stream(stream)))


def zero_adam_step_noalloc(plan: Plan, g32: torch.Tensor, p32: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
                           live: torch.Tensor, steps: torch.Tensor, lr: float, beta1: float, beta2: float,
                           eps: float, grad_scale: float, flag: Optional[torch.Tensor], arena: torch.Tensor,
                           stream=None, loss_scaler: Optional[torch.Tensor] = None) -> None:
    """zero_adam_step with its staging in the library's static device array (no allocation)."""
    S, w = plan.shard_numel, "zero_adam_step_noalloc"
    hp = zero_adam_hparams(lr, beta1, beta2, eps, grad_scale, _scaler(plan, loss_scaler, w))
    _check(lib().zero_adam_step_noalloc(plan.handle, _buf(plan, g32, w + ": g32", S, F32),
                                        _buf(plan, p32, w + ": p32", S, F32), _buf(plan, m, w + ": m", S, F32),
                                        _buf(plan, v, w + ": v", S, F32), _buf(plan, live, w + ": live", plan.n, U8),
                                        _buf(plan, steps, w + ": steps", plan.n, I32), ctypes.byref(hp),
                                        _buf(plan, flag, w + ": flag", 1, I32),
                                        _buf(plan, arena, w + ": arena", plan.arena_numel, elem_size=2),
                                        _stream(stream)))


def zero_unpack(plan: Plan, b: int, gathered: torch.Tensor, param_ptrs: torch.Tensor, stream=None) -> None:
    _check(lib().zero_unpack(plan.handle, b, _buf(plan, gathered, "zero_unpack: gathered", plan.block_elems(b),
                                                  elem_size=2),
                             _table(plan, param_ptrs, "zero_unpack: parameters", 2), _stream(stream)))


def zero_z3_step(plan: Plan, reduce_b0: int = 0, rows: Sequence = (), row_strides: Sequence = (),
                 live: Optional[torch.Tensor] = None, g32: Optional[torch.Tensor] = None, pack_b0: int = 0,
                 grad_ptrs: Optional[torch.Tensor] = None, packed: Sequence = (), check: bool = False,
                 gather_b0: int = 0, gathered: Sequence = (), param_ptrs: Optional[torch.Tensor] = None,
                 flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """One launch: the reduce of buckets reduce_b0 + j from rows[j] (row stride row_strides[j]),
    the pack of buckets pack_b0 + j into packed[j], the unpack of buckets gather_b0 + j from
    gathered[j] (empty sequences leave a kind out)."""
    w = "zero_z3_step"
    nr, nk, nu = len(rows), len(packed), len(gathered)
    if len(row_strides) != nr:
        raise ValueError(f"{w}: {nr} row buffers but {len(row_strides)} row strides")
    if max(nr, nk, nu) > Z3_MAX_BUCKETS:
        raise ValueError(f"{w}: at most {Z3_MAX_BUCKETS} buckets per piece")
    z = zero_z3_pieces()
    z.reduce_b0, z.reduce_n = reduce_b0, nr
    for j in range(nr):
        b = reduce_b0 + j
        z.rows[j] = _buf(plan, rows[j], f"{w}: rows of bucket {b}", plan.rows_elems(b, row_strides[j]), elem_size=2)
        z.row_stride[j] = int(row_strides[j])
    if nr:
        z.live = _buf(plan, live, w + ": live", plan.n, U8)
        z.g32 = _buf(plan, g32, w + ": g32", plan.shard_numel, F32)
    z.pack_b0, z.pack_n, z.check = pack_b0, nk, int(bool(check))
    for j in range(nk):
        z.packed[j] = _buf(plan, packed[j], f"{w}: packed block of bucket {pack_b0 + j}", plan.block_elems(pack_b0 + j),
                           elem_size=2)
    if nk:
        z.grad_ptrs = _table(plan, grad_ptrs, w + ": gradients", 2)
    z.gather_b0, z.gather_n = gather_b0, nu
    for j in range(nu):
        z.gathered[j] = _buf(plan, gathered[j], f"{w}: gathered block of bucket {gather_b0 + j}",
                             plan.block_elems(gather_b0 + j), elem_size=2)
    if nu:
        z.param_ptrs = _table(plan, param_ptrs, w + ": parameters", 2)
    z.flag = _buf(plan, flag, w + ": flag", 1, I32)
    _check(lib().zero_z3_step(plan.handle, ctypes.byref(z), _stream(stream)))


def zero_z3_layer_step(plan: Plan, reduce_b: int = -1, rows: Optional[torch.Tensor] = None, row_stride: int = 0,
                       live: Optional[torch.Tensor] = None, g32: Optional[torch.Tensor] = None, pack_b: int = -1,
                       grad_ptrs: Optional[torch.Tensor] = None, packed: Optional[torch.Tensor] = None,
                       check: bool = False, gather_b: int = -1, gathered: Optional[torch.Tensor] = None,
                       param_ptrs: Optional[torch.Tensor] = None, flag: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """reduce of bucket reduce_b, pack of bucket pack_b and unpack of bucket gather_b in one launch
    (an index of -1 leaves that piece out; its buffers are then not needed)."""
    w = "zero_z3_layer_step"
    r = reduce_b >= 0
    k = pack_b >= 0
    u = gather_b >= 0
    _check(lib().zero_z3_layer_step(
        plan.handle, reduce_b,
        _buf(plan, rows, w + ": rows", plan.rows_elems(reduce_b, row_stride), elem_size=2) if r else None, row_stride,
        _buf(plan, live, w + ": live", plan.n, U8) if r else None,
        _buf(plan, g32, w + ": g32", plan.shard_numel, F32) if r else None, pack_b,
        _table(plan, grad_ptrs, w + ": gradients", 2) if k else None,
        _buf(plan, packed, w + ": packed", plan.block_elems(pack_b), elem_size=2) if k else None, int(bool(check)),
        gather_b, _buf(plan, gathered, w + ": gathered", plan.block_elems(gather_b), elem_size=2) if u else None,
        _table(plan, param_ptrs, w + ": parameters", 2) if u else None,
        _buf(plan, flag, w + ": flag", 1, I32), _stream(stream)))


def zero_shard_init(plan: Plan, src_ptrs: torch.Tensor, src_dtype: int, p32: torch.Tensor, stream=None) -> None:
    _check(lib().zero_shard_init(plan.handle, _table(plan, src_ptrs, "zero_shard_init: sources",
                                                     4 if src_dtype == 0 else 2), src_dtype,
                                 _buf(plan, p32, "zero_shard_init: p32", plan.shard_numel, F32), _stream(stream)))


def zero_pack_bucket_check(plan: Plan, b: int, grad_ptrs: torch.Tensor, packed: torch.Tensor, flag: torch.Tensor,
                           stream=None) -> None:
    w = "zero_pack_bucket_check"
    _check(lib().zero_pack_bucket_check(plan.handle, b, _table(plan, grad_ptrs, w + ": gradients", 2),
                                        _buf(plan, packed, w + ": packed", plan.block_elems(b), elem_size=2),
                                        _buf(plan, flag, w + ": flag", 1, I32), _stream(stream)))


def zero_adam_prepare(plan: Plan, live: torch.Tensor, steps: torch.Tensor, lr: float, beta1: float, beta2: float,
                      eps: float, grad_scale: float, flag: Optional[torch.Tensor], stream=None,
                      loss_scaler: Optional[torch.Tensor] = None) -> None:
    w = "zero_adam_prepare"
    hp = zero_adam_hparams(lr, beta1, beta2, eps, grad_scale, _scaler(plan, loss_scaler, w))
    _check(lib().zero_adam_prepare(plan.handle, _buf(plan, live, w + ": live", plan.n, U8),
                                   _buf(plan, steps, w + ": steps", plan.n, I32), ctypes.byref(hp),
                                   _buf(plan, flag, w + ": flag", 1, I32), _stream(stream)))


def zero_reduce_adam_bucket(plan: Plan, b: int, rows: torch.Tensor, row_stride: int, live: torch.Tensor,
                            p32: torch.Tensor, m: torch.Tensor, v: torch.Tensor, flag: Optional[torch.Tensor],
                            arena: torch.Tensor, stream=None) -> None:
    """rows as in zero_reduce_shard; needs zero_adam_prepare earlier in the step on the same stream."""
    S, w = plan.shard_numel, "zero_reduce_adam_bucket"
    _check(lib().zero_reduce_adam_bucket(plan.handle, b, _buf(plan, rows, w + ": rows", plan.rows_elems(b, row_stride),
                                                              elem_size=2),
                                         row_stride, _buf(plan, live, w + ": live", plan.n, U8),
                                         _buf(plan, p32, w + ": p32", S, F32), _buf(plan, m, w + ": m", S, F32),
                                         _buf(plan, v, w + ": v", S, F32), _buf(plan, flag, w + ": flag", 1, I32),
                                         _buf(plan, arena, w + ": arena", plan.arena_numel, elem_size=2),
                                         _stream(stream)))




def zero_loss_scaler_init(cfg: zero_loss_scaler, scaler: torch.Tensor, stream=None) -> None:
    """scaler: device tensor of at least LOSS_SCALER_BYTES bytes (e.g. int32[8])."""
    if scaler.numel() * scaler.element_size() < LOSS_SCALER_BYTES:
        raise ValueError("loss scaler tensor too small")
    _check(lib().zero_loss_scaler_init(ctypes.byref(cfg), _ptr(scaler), _stream(stream)))


def zero_loss_scaler_update(flag: torch.Tensor, scaler: torch.Tensor, stream=None) -> None:
    if flag is not None and (flag.numel() < 1 or flag.dtype != torch.int32):
        raise ValueError("zero_loss_scaler_update: flag must be an int32 tensor of at least one element")
    if scaler is not None and scaler.numel() * scaler.element_size() < LOSS_SCALER_BYTES:
        raise ValueError("zero_loss_scaler_update: loss scaler tensor too small")
    _check(lib().zero_loss_scaler_update(_ptr(flag), _ptr(scaler), _stream(stream)))


def read_loss_scaler(scaler: torch.Tensor) -> zero_loss_scaler:
    """Host copy of a device scaler (synchronises)."""
    raw = scaler.detach().contiguous().view(torch.uint8)[:LOSS_SCALER_BYTES].cpu().numpy().tobytes()
    return zero_loss_scaler.from_buffer_copy(raw)


def zero_last_error() -> str:
    return lib().zero_last_error().decode(errors="replace")
