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


def ordered16(h: np.ndarray) -> np.ndarray:
    """Integers in the order of the 16-bit float values (sign-magnitude to two's complement)."""
    h = h.astype(np.int64)
    return np.where(h < 0x8000, h, -(h & 0x7FFF))


def assert_within_ulp16(got: np.ndarray, want: np.ndarray, what: str, ulps: int = 1) -> None:
    d = np.abs(ordered16(got) - ordered16(want))
    if (d > ulps).any():
        i = np.flatnonzero(d > ulps)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(d > ulps)} beyond {ulps} ulp; first at {i}: "
                             f"got {got[i]:#06x} want {want[i]:#06x}")


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
