"""Pins of the oracle's pack and unpack: the regroup/flatten example of the ColossalAI issue
"[zero] improving compatibility of low level zero" (Design, BWD) stored under tests/golden,
an independent reshape-based restatement of that procedure, identity, zero padding and
the layer-drop rule (Design, Optim)."""
import os
import re

import numpy as np
import pytest

import oracle
from oracle import B_ROW, B_STRIDE, P_COL, P_NUMEL, P_PADDED, P_SHARD

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_regroup():
    numels, nd, rows = None, None, {}
    for line in open(os.path.join(GOLDEN, "llz_bwd_regroup.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("numels"):
            numels = [int(x) for x in line.split()[1:]]
        elif line.startswith("nd"):
            nd = int(line.split()[1])
        else:
            k, body = line.split(":")
            rows[int(k.split()[1])] = body.split()
    return numels, nd, rows


def test_golden_regroup_example():
    numels, nd, rows = _load_regroup()
    pl = oracle.plan(numels, nd, 0, 0)
    grads = [np.arange(1 + 100 * i, 1 + 100 * i + n, dtype=np.uint16) for i, n in enumerate(numels)]
    packed = oracle.pack_bucket(pl, 0, grads)
    S = pl.buckets[0, B_ROW]
    for k in range(nd):
        expect = []
        for tok in rows[k]:
            m = re.fullmatch(r"g(\d+)\[(\d+)\]", tok)
            expect.append(0 if tok == "0" else int(grads[int(m.group(1))][int(m.group(2))]))
        assert list(packed[k, :S]) == expect
        assert np.all(packed[k, S:] == 0)  # row gap


def reshape_pack(numels, nd, grads):
    """The issue's BWD procedure with numpy primitives: pad each gradient with zeros, view
    it as [nd, -1], collect row k of every gradient and flatten them in list order."""
    rows = [[] for _ in range(nd)]
    for n, g in zip(numels, grads):
        padded = np.concatenate([g, np.zeros((-n) % nd, dtype=np.uint16)])
        view = padded.reshape(nd, -1)
        for k in range(nd):
            rows[k].append(view[k])
    return np.stack([np.concatenate(r) for r in rows]) if numels else None


def random_bits(rng, n):
    return rng.integers(0, 1 << 16, size=n, dtype=np.uint16)  # every pattern, NaN payloads included


@pytest.mark.parametrize("nd", [1, 2, 3, 8, 64])
def test_pack_matches_reshape_restatement(nd):
    rng = np.random.default_rng(nd)
    numels = [int(x) for x in rng.integers(0, 700, size=25)]
    pl = oracle.plan(numels, nd, 0, 0)
    grads = [random_bits(rng, n) for n in numels]
    packed = oracle.pack_bucket(pl, 0, grads)
    S = pl.buckets[0, B_ROW]
    assert np.array_equal(packed[:, :S], reshape_pack(numels, nd, grads))


def test_nd1_pack_is_concatenation():
    rng = np.random.default_rng(7)
    numels = [5, 0, 17, 3]
    grads = [random_bits(rng, n) for n in numels]
    pl = oracle.plan(numels, 1, 0, 0)
    packed = oracle.pack_bucket(pl, 0, grads)
    assert np.array_equal(packed[0, :sum(numels)], np.concatenate(grads))


def test_padding_slots_are_zero_and_dead_columns_untouched():
    rng = np.random.default_rng(8)
    nd = 8
    numels = [13, 64, 1, 100, 7]
    pl = oracle.plan(numels, nd, 2, 0)
    grads = [random_bits(rng, n) | np.uint16(1) for n in numels]  # no zero bit patterns
    grads[3] = None  # a parameter without a gradient
    sentinel = np.full((nd, pl.buckets[0, B_STRIDE]), 0xBEEF, dtype=np.uint16)
    packed = oracle.pack_bucket(pl, 0, grads, out=sentinel)
    for i, n in enumerate(numels):
        s, col = pl.params[i, P_SHARD], pl.params[i, P_COL]
        block = packed[:, col:col + s].reshape(-1)  # row-major = the padded flat parameter
        if grads[i] is None:
            assert np.all(block == 0xBEEF)
        else:
            assert np.array_equal(block[:n], grads[i]) and np.all(block[n:] == 0)


@pytest.mark.parametrize("nd,cap", [(1, 0), (3, 0), (8, 3000), (64, 50000), (1024, 0)])
def test_unpack_inverts_pack(nd, cap):
    rng = np.random.default_rng(nd + cap)
    numels = [int(x) for x in rng.integers(0, 3000, size=30)]
    pl = oracle.plan(numels, nd, nd - 1, cap)
    grads = [random_bits(rng, n) for n in numels]
    for b in range(pl.n_buckets):
        packed = oracle.pack_bucket(pl, b, grads)
        outs = [np.full(n, 0xDEAD, dtype=np.uint16) if i in pl.bucket_params(b) else None
                for i, n in enumerate(numels)]
        oracle.unpack_bucket(pl, b, packed, outs)
        for i in pl.bucket_params(b):
            assert np.array_equal(outs[i], grads[i])


def test_unpack_matches_reshape_restatement():
    """Unpack read the page's way: block[:, col:col+s] is the [nd, s] view of the padded
    parameter; flatten it and drop the padding."""
    rng = np.random.default_rng(9)
    nd = 8
    numels = [int(x) for x in rng.integers(0, 500, size=12)]
    pl = oracle.plan(numels, nd, 1, 0)
    block = random_bits(rng, nd * pl.buckets[0, B_STRIDE]).reshape(nd, -1)
    outs = [np.zeros(n, dtype=np.uint16) for n in numels]
    oracle.unpack_bucket(pl, 0, block, outs)
    for i, n in enumerate(numels):
        col, s = pl.params[i, P_COL], pl.params[i, P_SHARD]
        assert np.array_equal(outs[i], block[:, col:col + s].reshape(-1)[:n])


def test_locate_agrees_with_pack_and_unpack():
    rng = np.random.default_rng(10)
    nd = 16
    numels = [int(x) for x in rng.integers(0, 400, size=20)]
    pl = oracle.plan(numels, nd, 3, 2000)
    grads = [random_bits(rng, n) for n in numels]
    for b in range(pl.n_buckets):
        packed = oracle.pack_bucket(pl, b, grads)
        L = pl.buckets[b, B_STRIDE]
        for k in range(nd):
            for c in range(L):
                kind, i, e = oracle.pack_locate(pl, b, k, c)
                want = grads[i][e] if kind == 1 else 0
                assert packed[k, c] == want
    for i, n in enumerate(numels):
        for e in range(n):
            row, col = oracle.unpack_locate(pl, i, e)
            assert row * pl.params[i, P_SHARD] + (col - pl.params[i, P_COL]) == e
            assert row < nd and pl.params[i, P_PADDED] == pl.params[i, P_SHARD] * nd
            assert e < pl.params[i, P_NUMEL]


def test_shard_init_is_row_r_of_the_padded_master():
    """INIT of the issue and the briefia.fr snippet: p32 is a clone of row r of the
    zero-padded flat parameter."""
    rng = np.random.default_rng(11)
    nd, r = 8, 6
    numels = [int(x) for x in rng.integers(0, 300, size=15)]
    pl = oracle.plan(numels, nd, r, 1000)
    masters = [rng.standard_normal(n).astype(np.float32) for n in numels]
    p32 = np.full(pl.shard_len, np.nan, dtype=np.float32)
    oracle.shard_init(pl, masters, p32)
    for i, n in enumerate(numels):
        s, off = pl.params[i, P_SHARD], pl.params[i, 6]
        padded = np.concatenate([masters[i], np.zeros((-n) % nd, dtype=np.float32)])
        assert np.array_equal(p32[off:off + s], padded.reshape(nd, -1)[r])
    for b in range(pl.n_buckets):
        base = pl.buckets[b, 4]
        assert np.all(p32[base + pl.buckets[b, B_ROW]:base + pl.buckets[b, B_STRIDE]] == 0)
