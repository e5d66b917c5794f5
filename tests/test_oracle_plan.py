"""Pins of the oracle's plan (padding, shards, buckets, layout) against what the pages and
plain arithmetic fix: the briefia.fr "Implémentation simplifiée" formulas, the even split of
the ColossalAI "low level zero" issue (Overview / Goal / INIT), brute force, invariants."""
import numpy as np
import pytest

import oracle
from oracle import (B_BASE, B_COUNT, B_FIRST, B_ROW, B_STRIDE, P_BUCKET, P_COL, P_END, P_NUMEL, P_OFFSET, P_PAD,
                    P_PADDED, P_SHARD, P_START)


def brute_pad(numel, nd):
    """Smallest non-negative pad with (numel + pad) divisible by nd, found by search."""
    pad = 0
    while (numel + pad) % nd != 0:
        pad += 1
    return pad


@pytest.mark.parametrize("nd", [1, 2, 3, 8, 64, 1024])
def test_pad_and_shard_brute_force(nd):
    numels = np.arange(0, 3 * nd + 1, dtype=np.int64)
    for rank in sorted({0, nd // 2, nd - 1}):
        pl = oracle.plan(numels, nd, rank, 0)
        for i, x in enumerate(numels):
            p = pl.params[i]
            pad = brute_pad(int(x), nd)
            assert p[P_NUMEL] == x and p[P_PAD] == pad and p[P_PADDED] == x + pad
            assert p[P_SHARD] * nd == x + pad
            assert p[P_START] == rank * p[P_SHARD] and p[P_END] == p[P_START] + p[P_SHARD]


def test_shards_tile_every_parameter_exactly():
    rng = np.random.default_rng(1)
    for nd in (1, 3, 8, 64, 1000):
        numels = rng.integers(0, 5000, size=40)
        plans = [oracle.plan(numels, nd, r, 0) for r in range(nd)]
        for i, x in enumerate(numels):
            covered = np.zeros(plans[0].params[i, P_PADDED], dtype=np.int64)
            for pl in plans:
                covered[pl.params[i, P_START]:pl.params[i, P_END]] += 1
            assert np.all(covered == 1)  # rank rows partition [0, padded) with no overlap


def test_every_rank_gets_the_same_share():
    """The issue's goal: every rank holds a similar amount; with per-parameter even sharding
    it is exactly equal, and 5 parameters on 8 ranks leave no rank empty (the Overview's
    counter-example of whole-parameter assignment)."""
    numels = np.array([1000, 37, 4096, 5, 123457])
    shares = {oracle.plan(numels, 8, r, 0).params[:, P_SHARD].sum() for r in range(8)}
    assert len(shares) == 1 and shares.pop() > 0
    pl = oracle.plan(numels, 8, 7, 0)
    assert np.all(pl.params[:, P_SHARD] >= 1)


def test_mlp_model_worked_numbers():
    """MlpModel of the issue's Optim section at world_size 8, rank 3: every shard is the
    parameter's size / 8, starts at 3 * shard, and the shard slices follow list order."""
    numels = [256 * 128, 256, 256 * 256, 256, 512 * 256, 512]
    pl = oracle.plan(numels, 8, 3, 0)
    assert list(pl.params[:, P_SHARD]) == [4096, 32, 8192, 32, 16384, 64]
    assert list(pl.params[:, P_START]) == [12288, 96, 24576, 96, 49152, 192]
    assert list(pl.params[:, P_OFFSET]) == [0, 4096, 4128, 12320, 12352, 28736]
    assert list(pl.params[:, P_PAD]) == [0] * 6
    assert pl.n_buckets == 1 and pl.shard_len == 28800


def _check_buckets(pl, numels, capacity):
    padded = pl.params[:, P_PADDED]
    nxt = 0
    for b in range(pl.n_buckets):
        first, count = pl.buckets[b, B_FIRST], pl.buckets[b, B_COUNT]
        assert first == nxt and count >= 1
        nxt = first + count
        total = padded[first:first + count].sum()
        if capacity is None:
            continue
        assert total <= capacity or count == 1  # only a lone parameter may exceed the capacity
        if b + 1 < pl.n_buckets:  # maximal: the next parameter would not have fitted
            assert total + padded[first + count] > capacity
    assert nxt == len(numels)
    for i in range(len(numels)):
        b = pl.params[i, P_BUCKET]
        assert pl.buckets[b, B_FIRST] <= i < pl.buckets[b, B_FIRST] + pl.buckets[b, B_COUNT]


def test_bucket_greedy_rule():
    rng = np.random.default_rng(2)
    for trial in range(50):
        numels = rng.integers(0, 3000, size=rng.integers(1, 60))
        nd = int(rng.choice([1, 2, 7, 8, 64]))
        cap_elems = int(rng.integers(1, 8000))
        pl = oracle.plan(numels, nd, 0, 2 * cap_elems)
        _check_buckets(pl, numels, cap_elems)
    pl = oracle.plan(rng.integers(0, 3000, size=30), 8, 0, 0)
    assert pl.n_buckets == 1


def test_row_and_shard_layout():
    rng = np.random.default_rng(3)
    for trial in range(30):
        numels = rng.integers(0, 5000, size=rng.integers(1, 50))
        nd = int(rng.choice([1, 3, 8, 64]))
        pl = oracle.plan(numels, nd, int(rng.integers(0, nd)), 2 * int(rng.integers(1, 20000)))
        base = 0
        for b in range(pl.n_buckets):
            bk = pl.buckets[b]
            idx = list(pl.bucket_params(b))
            assert bk[B_ROW] == pl.params[idx, P_SHARD].sum()
            assert bk[B_STRIDE] % 8 == 0 and bk[B_ROW] <= bk[B_STRIDE] < bk[B_ROW] + 8
            assert bk[B_BASE] == base
            base += bk[B_STRIDE]
            col = 0
            for i in idx:
                assert pl.params[i, P_COL] == col and pl.params[i, P_OFFSET] == bk[B_BASE] + col
                col += pl.params[i, P_SHARD]
        assert pl.shard_len == base


def test_rank_shard_contents_do_not_depend_on_bucket_size():
    """Concatenating the live part of row r of every bucket gives the same list of
    parameter slices [p_0r, p_1r, ...] whatever the bucket capacity."""
    rng = np.random.default_rng(4)
    numels = rng.integers(0, 4000, size=40)
    ref = None
    for cap in (0, 2, 2000, 20000, 10 ** 9):
        pl = oracle.plan(numels, 8, 5, cap)
        order = []
        for i in range(len(numels)):
            off, s = pl.params[i, P_OFFSET], pl.params[i, P_SHARD]
            order.append((i, pl.params[i, P_START], s))
            assert off + s <= pl.shard_len
        ref = ref or order
        assert order == ref


@pytest.mark.parametrize("args", [([], 8, 0, 0), ([5], 0, 0, 0), ([5], 8, 8, 0), ([5], 8, -1, 0), ([-1], 8, 0, 0),
                                  ([5], 8, 0, -2)])
def test_invalid_arguments(args):
    with pytest.raises(ValueError):
        oracle.plan(*args)


def test_bucket_filled_exactly_stays_one_bucket():
    """A bucket is full when adding the next parameter would exceed the capacity; a run that
    reaches the capacity exactly still fits."""
    pl = oracle.plan([4, 4, 1], 1, 0, 2 * 8)
    assert pl.n_buckets == 2 and list(pl.buckets[:, B_COUNT]) == [2, 1]
    pl = oracle.plan([3, 5], 1, 0, 2 * 8)
    assert pl.n_buckets == 1
    pl = oracle.plan([10, 0, 2], 1, 0, 2 * 8)  # an oversize parameter is alone, even before an empty one
    assert list(pl.buckets[:, B_COUNT]) == [1, 2]


# ------------------------------------------------------ grouped plans (ZeRO-3 units) --

def _runs(groups):
    """[start, end) of every maximal run of equal ids."""
    out, a = [], 0
    for i in range(1, len(groups) + 1):
        if i == len(groups) or groups[i] != groups[i - 1]:
            out.append((a, i))
            a = i
    return out


@pytest.mark.parametrize("nd,cap", [(1, 0), (3, 2 * 500), (8, 2 * 4000), (8, 0), (64, 2 * 30000)])
def test_grouped_plan_is_the_concatenation_of_per_group_plans(nd, cap):
    """A grouped plan is the plans of each run of equal ids laid one after the other: buckets,
    columns and every field the same, bucket indices and shard offsets shifted by what the
    earlier runs hold (an independent restatement: each run planned on its own)."""
    rng = np.random.default_rng(nd * 7 + cap)
    for trial in range(6):
        n = int(rng.integers(1, 60))
        numels = rng.integers(0, 5000, size=n)
        groups = np.cumsum(rng.random(n) < 0.25).astype(np.int32)
        if trial == 5:
            groups = (np.arange(n) // 3 % 2).astype(np.int32)  # ids that come back: runs, not sets
        pl = oracle.plan(numels, nd, nd - 1, cap, groups)
        bshift = pshift = 0
        for a, e in _runs(groups):
            sub = oracle.plan(numels[a:e], nd, nd - 1, cap)
            got = pl.params[a:e].copy()
            want = sub.params.copy()
            want[:, P_BUCKET] += bshift
            want[:, P_OFFSET] += pshift
            assert np.array_equal(got, want), (trial, a, e)
            gb = pl.buckets[bshift:bshift + sub.n_buckets].copy()
            wb = sub.buckets.copy()
            wb[:, B_FIRST] += a
            wb[:, B_BASE] += pshift
            assert np.array_equal(gb, wb), (trial, a, e)
            bshift += sub.n_buckets
            pshift += sub.shard_len
        assert bshift == pl.n_buckets and pshift == pl.shard_len


def test_grouped_plan_special_cases():
    numels = [100, 7, 3000, 0, 45, 45]
    # one group: the ungrouped plan
    a = oracle.plan(numels, 8, 2, 2 * 1000)
    b = oracle.plan(numels, 8, 2, 2 * 1000, np.zeros(6, np.int32))
    assert np.array_equal(a.params, b.params) and np.array_equal(a.buckets, b.buckets)
    # every parameter its own group: one bucket each, whatever the capacity
    for cap in (0, 2, 10 ** 9):
        c = oracle.plan(numels, 8, 2, cap, np.arange(6, dtype=np.int32))
        assert c.n_buckets == 6 and list(c.buckets[:, B_COUNT]) == [1] * 6
    # unbounded capacity: exactly the runs of equal ids
    d = oracle.plan(numels, 8, 2, 0, np.array([5, 5, 1, 1, 1, 5], np.int32))
    assert list(d.buckets[:, B_FIRST]) == [0, 2, 5] and list(d.buckets[:, B_COUNT]) == [2, 3, 1]
