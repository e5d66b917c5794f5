"""Pins of the oracle's Nd-way shard reduce (the arithmetic of the reduce-scatter in the
ColossalAI "low level zero" issue, Design / BWD) against exact arithmetic: integer-valued
sums, correctly rounded two-term sums, the recursive-summation error bound, an ordering
example whose answer IEEE-754 fixes, and library conversions for Nd = 1."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, FP16, B_BASE, B_STRIDE, P_COL, P_OFFSET, P_SHARD


def bits_of(values, dtype):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16 if dtype == BF16 else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_of(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16 if dtype == BF16 else torch.float16)
    return t.float().numpy()


@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_integer_sums_are_exact(dtype):
    rng = np.random.default_rng(dtype)
    hi = 256 if dtype == BF16 else 2048  # integers exactly representable in the 16-bit type
    for nd in (1, 2, 8, 64, 1024):
        vals = rng.integers(-hi, hi + 1, size=nd)
        got = oracle.reduce_column(bits_of(vals.astype(np.float32), dtype), dtype)
        assert got == np.float32(vals.sum())  # |sum| < 2^24: every partial sum is exact


@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_nd1_is_the_exact_conversion(dtype):
    allbits = np.arange(1 << 16, dtype=np.uint16)
    ref = f32_of(allbits, dtype)
    got = np.array([oracle.reduce_column(allbits[i:i + 1], dtype) for i in range(0, 1 << 16, 97)])
    r = ref[::97]
    same = (got.view(np.uint32) == r.view(np.uint32)) | (np.isnan(got) & np.isnan(r))
    assert np.all(same)


@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_two_term_sum_is_correctly_rounded(dtype):
    """a + b of two 16-bit values is exact in double; one rounding to fp32 is the IEEE sum."""
    rng = np.random.default_rng(5)
    a = bits_of(rng.standard_normal(3000).astype(np.float32) * 3, dtype)
    b = bits_of(rng.standard_normal(3000).astype(np.float32) * 1e-3, dtype)
    fa, fb = f32_of(a, dtype), f32_of(b, dtype)
    for i in range(3000):
        exact = float(fa[i]) + float(fb[i])
        assert oracle.reduce_column(np.array([a[i], b[i]]), dtype) == np.float32(exact)


def test_fixed_ascending_order():
    """1 + 2^-24 + 2^-24 in fp32: ascending order rounds each tiny addend away (ties to
    even keep 1.0); adding the two tiny terms first gives 1 + 2^-23.  The reduce must take
    rank 0 first and then ranks 1, 2, ... in order."""
    for dtype in (BF16, FP16):
        one, tiny = bits_of([1.0, 2.0 ** -24], dtype)
        assert oracle.reduce_column(np.array([one, tiny, tiny]), dtype) == np.float32(1.0)
        assert oracle.reduce_column(np.array([tiny, tiny, one]), dtype) == np.float32(1.0 + 2.0 ** -23)


@pytest.mark.parametrize("nd", [8, 64, 1024])
def test_error_bound_of_recursive_summation(nd):
    """|fl(sum) - sum| <= gamma_{nd-1} * sum |x_k| with gamma_m = m u / (1 - m u), u = 2^-24."""
    rng = np.random.default_rng(nd)
    u = 2.0 ** -24
    g = (nd - 1) * u / (1 - (nd - 1) * u)
    for trial in range(200):
        bits = bits_of(rng.standard_normal(nd).astype(np.float32), BF16)
        f = f32_of(bits, BF16).astype(np.float64)
        got = float(oracle.reduce_column(bits, BF16))
        assert abs(got - math.fsum(f)) <= g * np.abs(f).sum() + 1e-300


def test_fp16_subnormals_are_kept():
    sub = np.arange(1, 1024, dtype=np.uint16)  # every positive fp16 subnormal
    for s in sub[::37]:
        got = oracle.reduce_column(np.array([s, s]), FP16)
        assert got == np.float32(2 * int(s) * 2.0 ** -24)


def test_non_finite_inputs_propagate():
    for dtype in (BF16, FP16):
        inf, ninf, one = bits_of([math.inf, -math.inf, 1.0], dtype)
        nan = bits_of([math.nan], dtype)[0]
        assert math.isinf(oracle.reduce_column(np.array([one, inf, one]), dtype))
        assert math.isnan(oracle.reduce_column(np.array([inf, one, ninf]), dtype))
        assert math.isnan(oracle.reduce_column(np.array([one, nan]), dtype))


def test_bucket_reduce_writes_live_columns_only():
    rng = np.random.default_rng(12)
    nd = 8
    numels = [100, 33, 250, 8, 77]
    pl = oracle.plan(numels, nd, 4, 0)
    L = pl.buckets[0, B_STRIDE]
    rows = bits_of(rng.standard_normal(nd * L).astype(np.float32), BF16).reshape(nd, L)
    live = np.array([1, 0, 1, 1, 0], dtype=np.uint8)
    g32 = np.full(pl.shard_len, -7.0, dtype=np.float32)
    oracle.reduce_bucket(pl, 0, rows, BF16, live, g32)
    for i in range(len(numels)):
        off, col, s = pl.params[i, P_OFFSET], pl.params[i, P_COL], pl.params[i, P_SHARD]
        for j in range(s):
            want = oracle.reduce_column(rows[:, col + j], BF16) if live[i] else np.float32(-7.0)
            assert g32[off + j] == want
    assert np.all(g32[pl.buckets[0, B_BASE] + pl.buckets[0, 2]:] == -7.0)  # the gap is not written


def test_overflow_flag():
    nd = 4
    numels = [40, 40, 40]
    pl = oracle.plan(numels, nd, 0, 0)
    g32 = np.zeros(pl.shard_len, dtype=np.float32)
    live = np.ones(3, dtype=np.uint8)
    assert oracle.overflow(pl, g32, live) == 0
    for bad in (np.inf, -np.inf, np.nan):
        g = g32.copy()
        g[pl.params[1, P_OFFSET] + 3] = bad
        assert oracle.overflow(pl, g, live) == 1
        live2 = live.copy()
        live2[1] = 0
        assert oracle.overflow(pl, g, live2) == 0  # a dead parameter's slot does not count
    g = g32.copy()
    g[pl.params[2, P_OFFSET]] = np.float32(3.4e38)  # large but finite
    assert oracle.overflow(pl, g, live) == 0


def test_negative_zero_is_kept():
    """IEEE-754: (-0) + (-0) = -0 under round to nearest.  The sum starts from rank 0's
    value, not from +0, so a column of negative zeros reduces to -0."""
    for dtype in (BF16, FP16):
        nz = bits_of([-0.0], dtype)[0]
        for nd in (1, 2, 8):
            got = oracle.reduce_column(np.full(nd, nz), dtype)
            assert np.array([got], np.float32).view(np.uint32)[0] == 0x80000000
