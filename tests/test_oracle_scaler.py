"""Pins of the oracle's dynamic loss-scaling rule: a closed form over the lengths of the runs of
clean steps, the clamps, and the invariants the rule keeps."""
import numpy as np
import pytest

import oracle


def fresh(scale=1.0, interval=3, growth=2.0, backoff=0.5, lo=2.0 ** -60, hi=2.0 ** 60):
    return oracle.Scaler(scale, 0, interval, growth, backoff, lo, hi, 0)


def closed_form(flags, interval, s0=1.0):
    """Power-of-two factors, no clamping: every maximal run of L clean steps grows the scale
    floor(L / interval) times, every overflow halves it, and the count left over is the
    trailing run's length mod interval."""
    runs, cur = [], 0
    for f in flags:
        if f:
            runs.append(cur)
            cur = 0
        else:
            cur += 1
    grows = sum(r // interval for r in runs) + cur // interval
    n_over = int(sum(flags))
    return s0 * 2.0 ** (grows - n_over), cur % interval, n_over


@pytest.mark.parametrize("interval", [1, 2, 3, 7, 50])
def test_closed_form_over_random_sequences(interval):
    rng = np.random.default_rng(interval)
    for trial in range(40):
        n = int(rng.integers(0, 56))  # at most 55 doublings or halvings: inside the 2^±60 clamps
        p = rng.uniform(0.0, 0.5)
        flags = (rng.random(n) < p).astype(int)
        s = fresh(interval=interval)
        for f in flags:
            oracle.loss_scaler_update(s, f)
        scale, good, over = closed_form(flags, interval)
        assert (s.scale, s.good_steps, s.overflows) == (scale, good, over), (interval, trial)


def test_worked_sequence():
    # 2^16, interval 2: clean, clean (grow to 2^17), overflow (2^16), clean, overflow (2^15)
    s = fresh(scale=2.0 ** 16, interval=2)
    seen = []
    for f in (0, 0, 1, 0, 1):
        oracle.loss_scaler_update(s, f)
        seen.append((s.scale, s.good_steps, s.overflows))
    assert seen == [(2.0 ** 16, 1, 0), (2.0 ** 17, 0, 0), (2.0 ** 16, 0, 1), (2.0 ** 16, 1, 1), (2.0 ** 15, 0, 2)]


def test_clamps():
    s = fresh(scale=2.0 ** 24, interval=1, lo=1.0, hi=2.0 ** 24)
    for _ in range(5):
        oracle.loss_scaler_update(s, 0)
        assert s.scale == 2.0 ** 24 and s.good_steps == 0
    s = fresh(scale=4.0, interval=1, lo=1.0, hi=2.0 ** 24)
    for k in range(6):
        oracle.loss_scaler_update(s, 1)
        assert s.scale == max(1.0, 4.0 / 2 ** (k + 1)) and s.overflows == k + 1


def test_other_factors_multiply_in_binary32():
    # growth 3, back-off 1/4: 3^a 4^-b is exact in binary32 while 3^a < 2^24
    s = fresh(scale=1.0, interval=1, growth=3.0, backoff=0.25)
    for f in (0, 0, 0, 1, 0, 1, 1, 0, 0):
        oracle.loss_scaler_update(s, f)
    assert s.scale == 3.0 ** 6 * 0.25 ** 3 and s.overflows == 3
    # a factor whose products round: 1.1 (binary32) applied once, against numpy's binary32 product
    s = fresh(scale=3.0, interval=1, growth=float(np.float32(1.1)))
    oracle.loss_scaler_update(s, 0)
    assert s.scale == float(np.float32(3.0) * np.float32(1.1))


def test_invariants_hold():
    rng = np.random.default_rng(5)
    s = fresh(scale=2.0 ** 10, interval=4, lo=2.0 ** 5, hi=2.0 ** 14)
    for f in (rng.random(2000) < 0.2):
        oracle.loss_scaler_update(s, int(f))
        assert 2.0 ** 5 <= s.scale <= 2.0 ** 14
        assert 0 <= s.good_steps < 4
