"""Helpers for the GPU parity tests: moving 16-bit bit patterns between numpy (the oracle's
side) and device tensors (the HIP side), comparisons at the stated tolerances, and ragged
plan generators.  Inputs are generated once and handed to both sides bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def to_np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def same_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Bit equality, except that any NaN equals any NaN (IEEE-754 leaves payloads open)."""
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))


def assert_same_f32(got: np.ndarray, want: np.ndarray, what: str) -> None:
    ok = same_f32(got, want)
    if not ok.all():
        bad = np.flatnonzero(~ok)
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} mismatches; first at {i}: got {got[i]!r} "
                             f"({got.view(np.uint32)[i]:#010x}) want {want[i]!r} ({want.view(np.uint32)[i]:#010x})")


def assert_close_f32(got: np.ndarray, want: np.ndarray, what: str, rel=1e-6, abs_=1e-7) -> None:
    """|got - want| <= abs + rel * |want| (the tolerance for Adam's fp32 state)."""
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    lim = abs_ + rel * np.abs(want.astype(np.float64))
    ok = err <= lim
    if not ok.all():
        i = np.flatnonzero(~ok)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} outside tolerance; first at {i}: got {got[i]!r} "
                             f"want {want[i]!r}")


def expected_arena(pl: oracle.Plan, oracle_arena: np.ndarray, got_p32: np.ndarray, ever: np.ndarray,
                   dtype: int) -> np.ndarray:
    """The arena the Adam step must leave: the oracle's everywhere, except at row r of every
    bucket in the columns of parameters that have taken a step, which hold the 16-bit RNE (by the
    oracle's conversion) of the kernel's own p32 -- the write is defined as that rounding, and
    the kernel's p32 is checked against the oracle's separately.  (Near zero the p32 tolerance
    can exceed a 16-bit ulp, so a 1-ulp bound on the 16-bit value against the oracle would not
    follow from it.)"""
    want = oracle_arena.copy()
    lp = oracle.from_f32(got_p32.astype(np.float32), dtype)
    for b in range(pl.n_buckets):
        O, L = int(pl.buckets[b, oracle.B_BASE]), int(pl.buckets[b, oracle.B_STRIDE])
        row = want[pl.nd * O + pl.rank * L: pl.nd * O + pl.rank * L + L]
        sel = ever[O:O + L]
        row[sel] = lp[O:O + L][sel]
    return want


def ordered16(h: np.ndarray) -> np.ndarray:
    """Integers in the order of the 16-bit float values (sign-magnitude to two's complement)."""
    h = h.astype(np.int64)
    return np.where(h < 0x8000, h, -(h & 0x7FFF))


def one_ulp_implied(p_ref: np.ndarray, dtype: int, rel: float = 1e-6, abs_: float = 1e-7) -> np.ndarray:
    """Where |p - p_ref| <= abs_ + rel |p_ref| forces RNE16(p) within one 16-bit ulp of
    RNE16(p_ref): the tolerance is at most half the smallest 16-bit ulp near p_ref (the ulp of
    |p_ref| / 2), so the interval crosses at most one rounding boundary.  False only near zero,
    where the absolute tolerance exceeds a 16-bit ulp."""
    a = np.abs(p_ref.astype(np.float64))
    mant, emin = (7, -126) if dtype == 1 else (10, -14)
    e = np.floor(np.log2(np.maximum(a / 2, 2.0 ** -160)))
    ulp = 2.0 ** (np.maximum(e, emin) - mant)
    return abs_ + rel * a <= ulp / 2


def assert_lp_within_ulp(got16: np.ndarray, want16: np.ndarray, p_ref: np.ndarray, dtype: int, what: str) -> None:
    """16-bit parameters within one ulp of the oracle's wherever the p32 tolerance implies it."""
    m = one_ulp_implied(p_ref, dtype)
    d = np.abs(ordered16(got16) - ordered16(want16))
    bad = m & (d > 1)
    if bad.any():
        i = np.flatnonzero(bad)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(bad)} beyond 1 ulp; first at {i}: got {got16[i]:#06x} "
                             f"want {want16[i]:#06x} (p_ref {p_ref[i]!r})")


def check_arena(pl: oracle.Plan, got_arena: np.ndarray, oracle_arena: np.ndarray, got_p32: np.ndarray,
                oracle_p32: np.ndarray, ever: np.ndarray, dtype: int, what: str) -> None:
    """The arena after Adam steps: bit-exact against the RNE of the kernel's own p32 where a
    parameter has stepped and against the oracle elsewhere (expected_arena), and within one
    ulp of the oracle's 16-bit parameters wherever the p32 tolerance implies it."""
    assert np.array_equal(got_arena, expected_arena(pl, oracle_arena, got_p32, ever, dtype)), what
    for b in range(pl.n_buckets):
        O, L = int(pl.buckets[b, oracle.B_BASE]), int(pl.buckets[b, oracle.B_STRIDE])
        at = pl.nd * O + pl.rank * L
        sel = ever[O:O + L]
        assert_lp_within_ulp(got_arena[at:at + L][sel], oracle_arena[at:at + L][sel], oracle_p32[O:O + L][sel], dtype,
                             f"{what} bucket {b}")


def ragged_numels(rng: np.random.Generator, n: int, nd: int, hi: int) -> list:
    """A ragged list that exercises every layout case: empty parameters, numel < nd, exact
    multiples of nd, primes, and log-uniform sizes up to hi."""
    out = []
    for _ in range(n):
        kind = rng.integers(0, 6)
        if kind == 0:
            out.append(0)
        elif kind == 1:
            out.append(int(rng.integers(1, max(2, nd))))
        elif kind == 2:
            out.append(nd * int(rng.integers(1, max(2, hi // max(nd, 1)))))
        else:
            out.append(int(np.exp(rng.uniform(0, np.log(hi)))))
    return out


def random_bits(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(0, 1 << 16, size=n, dtype=np.uint16)


def placed_views(arrays, rng: np.random.Generator, misalign: bool):
    """Copy uint16 arrays to the device, each in its own slot of one buffer; with misalign the
    slots start at random 2-byte offsets (not 16-byte aligned).  None stays None."""
    total = sum(0 if a is None else a.size + 16 for a in arrays) + 64
    buf = torch.zeros(total, dtype=torch.int16, device=DEV)
    views, pos = [], 8
    for a in arrays:
        if a is None:
            views.append(None)
            continue
        off = pos + (int(rng.integers(1, 8)) if misalign else 0)
        v = buf[off:off + a.size]
        if a.size:
            v.copy_(to_dev16(a))
        views.append(v)
        pos = ((off + a.size + 7) // 8 + 1) * 8
    return buf, views


def oracle_block(pl: oracle.Plan, flat: np.ndarray, b: int) -> np.ndarray:
    """View of bucket b's [nd, L_b] block inside an arena-shaped flat array."""
    off = pl.nd * pl.buckets[b, oracle.B_BASE]
    L = pl.buckets[b, oracle.B_STRIDE]
    return flat[off:off + pl.nd * L].reshape(pl.nd, L)


# ------------------------------------------------ sampling at full size ---------------
P_OFF, P_S, P_NUMEL, P_COL = oracle.P_OFFSET, oracle.P_SHARD, oracle.P_NUMEL, oracle.P_COL


def sample_columns(pl, rng, count, extra_params=300):
    """Shard columns inside parameter slices: uniform ones plus the first and last slice column
    of some parameters (boundaries of parameters, buckets and padding)."""
    s = pl.params[:, P_S]
    cum = np.cumsum(s)
    pick = rng.integers(0, cum[-1], size=count)
    i = np.searchsorted(cum, pick, side="right")
    j = pick - (cum[i] - s[i])
    cols = pl.params[i, P_OFF] + j
    nz = np.flatnonzero(s > 0)
    chosen = rng.choice(nz, size=min(extra_params, nz.size), replace=False)
    edges = np.concatenate([pl.params[chosen, P_OFF], pl.params[chosen, P_OFF] + s[chosen] - 1])
    return np.unique(np.concatenate([cols, edges]))


def column_owner(pl, cols):
    """(param, index of the column inside the param's slice) for shard columns."""
    ends = pl.params[:, P_OFF] + pl.params[:, P_S]
    i = np.searchsorted(ends, cols, side="right")
    return i, cols - pl.params[i, P_OFF]


def gather_params(tensors, idx_i, idx_e, fill=0):
    """Values tensors[i][e] for parallel index arrays (device gathers, one per parameter), on
    the host; `fill` where e is past the parameter's end (padding) or the tensor is None."""
    dt = next(t.dtype for t in tensors if t is not None)
    out = torch.full((idx_i.size,), fill, dtype=dt)
    for i in np.unique(idx_i):
        t = tensors[i]
        if t is None:
            continue
        sel = np.flatnonzero(idx_i == i)
        e = idx_e[sel]
        ok = e < t.numel()
        if ok.any():
            out[torch.from_numpy(sel[ok])] = t[torch.from_numpy(e[ok]).to(t.device)].cpu()
    return out


def bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def row_zero_mask(pl, b, live):
    """Positions of one rank row (rank r's row of bucket b) that a real packer sends as +0 or
    leaves unwritten: padding of each parameter, dead parameters, and the row gap."""
    L = int(pl.buckets[b, oracle.B_STRIDE])
    keep = np.zeros(L, dtype=bool)
    r = pl.rank
    for i in pl.bucket_params(b):
        if not live[i]:
            continue
        c, s_, n = pl.params[i, P_COL], pl.params[i, P_S], pl.params[i, P_NUMEL]
        real = max(0, min(s_, n - r * s_))
        keep[c:c + real] = True
    return ~keep
