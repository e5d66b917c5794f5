"""Pins of the oracle's input check (the fused path's overflow verdict, taken from the
gradients before the reduce): exact rational arithmetic over every 16-bit pattern, the
guarantee it exists for (no flagged input -> every fp32 sum finite), and what it must ignore
(parameters without a gradient, other buckets, padding)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle

BF16, FP16 = 1, 2
TWO_126 = Fraction(2) ** 126


def exact_value(bits: int, dtype: int):
    """The value of a 16-bit pattern, from the format definitions via numpy's bit views; None
    for inf and NaN."""
    if dtype == BF16:
        x = np.array([bits << 16], np.uint32).view(np.float32)[0]
    else:
        x = np.array([bits], np.uint16).view(np.float16)[0]
    return Fraction(float(x)) if np.isfinite(x) else None


def one_param_verdict(vals: np.ndarray, nd: int, dtype: int) -> int:
    pl = oracle.plan([vals.size], nd, 0, 0)
    return oracle.input_check(pl, 0, [vals.astype(np.uint16)], dtype)


@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("nd", [1, 3, 8, 1000, 65535])
def test_every_pattern_against_exact_arithmetic(nd, dtype):
    bits = np.arange(1 << 16, dtype=np.int64)
    vals = [exact_value(int(b), dtype) for b in bits]
    bad = np.array([v is None or abs(v) * nd > TWO_126 for v in vals])
    # all patterns that pass, in one parameter: no flag
    assert one_param_verdict(bits[~bad], nd, dtype) == 0
    # every failing pattern on its own (there are few per format at most sizes), else a sample
    failing = bits[bad]
    rng = np.random.default_rng(nd * 7 + dtype)
    pick = failing if failing.size <= 600 else np.concatenate(
        [np.sort(failing)[:100], rng.choice(failing, 400, replace=False)])
    for b in pick:
        vec = np.array([0, int(b), 0x3F80 if dtype == BF16 else 0x3C00], np.uint16)
        assert one_param_verdict(vec, nd, dtype) == 1, hex(int(b))


def test_bound_is_inclusive_at_a_power_of_two():
    # Nd = 8: 2^126 / 8 = 2^123, a bf16 value (0x7D00); the next bf16 value up is flagged
    assert exact_value(0x7D00, BF16) == Fraction(2) ** 123
    assert one_param_verdict(np.array([0x7D00, 0xFD00], np.uint16), 8, BF16) == 0
    assert one_param_verdict(np.array([0x7D01], np.uint16), 8, BF16) == 1
    assert one_param_verdict(np.array([0xFD01], np.uint16), 8, BF16) == 1


def test_non_finite_always_flagged_and_fp16_never_reaches_the_bound():
    for dtype, pats in ((BF16, (0x7F80, 0xFF80, 0x7FC0, 0xFFC1)), (FP16, (0x7C00, 0xFC00, 0x7E00, 0x7C01))):
        for p in pats:
            assert one_param_verdict(np.array([p], np.uint16), 1, dtype) == 1
    # the largest finite fp16 value (65504) is far below 2^126 / 65535
    assert one_param_verdict(np.array([0x7BFF, 0xFBFF], np.uint16), 65535, FP16) == 0


def test_clear_verdict_means_finite_sums():
    """The guarantee: if no input of any rank is flagged, every fp32 sum of Nd of them in the
    reduce's order is finite -- checked at the worst case (every value at the largest allowed
    magnitude, one sign), while values just past the largest bf16 makes the sum overflow."""
    for nd in (1, 2, 3, 8, 64, 1000, 65535):
        allowed = [b for b in range(0x7F80) if exact_value(b, BF16) * nd <= TWO_126]
        top = max(allowed, key=lambda b: exact_value(b, BF16))
        for sign in (0, 0x8000):
            col = np.full(nd, top | sign, np.uint16)
            s = oracle.reduce_column(col, BF16)
            assert np.isfinite(s), (nd, hex(top))
    # without the check: eight copies of the largest finite bf16 overflow fp32
    assert np.isinf(oracle.reduce_column(np.full(8, 0x7F7F, np.uint16), BF16))
    assert one_param_verdict(np.array([0x7F7F], np.uint16), 8, BF16) == 1


def test_ignores_dead_parameters_other_buckets_and_padding():
    numels = [10, 7, 300, 5]
    nd = 4
    pl = oracle.plan(numels, nd, 1, 2 * 16)  # capacity 16 padded elements -> several buckets
    assert pl.n_buckets >= 3
    inf = np.uint16(0x7F80)
    grads = [np.full(x, 0x3F80, np.uint16) for x in numels]
    grads[1][3] = inf
    b1 = int(pl.params[1, oracle.P_BUCKET])
    for b in range(pl.n_buckets):
        assert oracle.input_check(pl, b, grads, BF16) == int(b == b1)
    dead = list(grads)
    dead[1] = None
    assert all(oracle.input_check(pl, b, dead, BF16) == 0 for b in range(pl.n_buckets))
    # param 1 (7 elements, padded to 8): its padding element is not a gradient element; the
    # array handed over has exactly numel entries, so an inf just past them is never read
    g1 = np.full(8, 0x3F80, np.uint16)
    g1[7] = inf
    grads2 = list(grads)
    grads2[1] = g1[:7]
    assert oracle.input_check(pl, b1, grads2, BF16) == 0
