"""Randomised end-to-end parity through the C ABI: seeded random plans (Nd from 1 to 1031, odd
ones included; any rank; bucket capacities from one element to one bucket; optional group ids;
bf16 or fp16; tiny, empty and multi-tile parameters; dead parameters; misaligned per-parameter
buffers), each run through the whole step on the unfused path — plan tables, pack, Nd-way
reduce with the fused flag, Adam, unpack — and on the fused path — checked pack, reduce + Adam —
against the oracle: bit for bit for the plan, pack, reduce, flag and unpack; Adam within its
tolerance; the fused path bit-identical to the unfused one."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_amd as Z
from gpu_harness import (DEV, assert_close_f32, assert_same_f32, check_arena, oracle_block, placed_views,
                         random_bits, say, to_dev16, to_np16, to_np32)

pytestmark = pytest.mark.gpu
BF16, FP16 = Z.ZERO_BF16, Z.ZERO_FP16
SENT16 = 0x5A5A
NDS = [1, 2, 3, 5, 7, 8, 13, 16, 31, 64, 100, 257, 1024, 1031]


def random_case(seed):
    rng = np.random.default_rng(10_000 + seed)
    nd = int(rng.choice(NDS))
    rank = int(rng.integers(0, nd))
    n = int(rng.integers(1, 120))
    kinds = rng.choice(4, size=n, p=[0.3, 0.35, 0.3, 0.05])  # few multi-tile parameters
    numels = []
    for k in kinds:
        if k == 0:
            numels.append(int(rng.integers(0, 2 * nd + 2)))        # empty, below Nd, about Nd
        elif k == 1:
            numels.append(int(rng.integers(0, 3000)))
        elif k == 2:
            numels.append(int(rng.integers(3000, 40000)))
        else:
            numels.append(int(nd * 2048 * int(rng.integers(1, 3)) + int(rng.integers(-3, 4)) * nd
                              + int(rng.integers(0, nd))))         # whole tiles, ragged tail
    numels = [max(0, x) for x in numels]
    total = sum(numels)
    cap = int(rng.choice([0, 2, 2 * max(1, total // 7), 2 * max(1, total // 2), 2 * int(rng.integers(1, 5000))]))
    groups = None
    if rng.random() < 0.4:
        groups = np.cumsum(rng.random(n) < 0.15).astype(np.int32)
    dtype = BF16 if rng.random() < 0.5 else FP16
    return rng, nd, rank, numels, cap, groups, dtype


# seeds whose plans cover Nd = 3, 13, 1031, 8, 257, 31, 100, 16, 1024, 64 and 1
SMALL_GRID_SEEDS = [0, 1, 2, 4, 9, 10, 11, 12, 15, 16, 61]


def finite_bits(rng, n, dtype):
    return random_bits(rng, n) & np.uint16(0xBFFF if dtype == BF16 else 0xBBFF)


@pytest.mark.parametrize("seed", range(64))
def test_random_plan_whole_step(seed):
    rng, nd, rank, numels, cap, groups, dtype = random_case(seed)
    say(f"sweep seed={seed} nd={nd} rank={rank} n={len(numels)} total={sum(numels)} cap={cap} "
        f"groups={'yes' if groups is not None else 'no'} dtype={dtype}")
    gl = None if groups is None else [int(x) for x in groups]
    A = Z.ShardStep(numels, nd, rank, cap, dtype, groups=gl)   # unfused
    F = Z.ShardStep(numels, nd, rank, cap, dtype, groups=gl)   # fused
    pl = oracle.plan(numels, nd, rank, cap, groups)
    S = pl.shard_len
    # plan tables
    assert (A.summary.n_buckets, A.summary.shard_numel) == (pl.n_buckets, S)
    for i in range(len(numels)):
        info = Z.zero_plan_param_info(A.plan, i)
        assert [info.numel, info.pad, info.padded_numel, info.shard_size, info.shard_start, info.shard_end,
                info.shard_offset, info.bucket, info.bucket_col] == list(pl.params[i]), i
    for b in range(pl.n_buckets):
        bk = Z.zero_plan_bucket_info(A.plan, b)
        assert [bk.first_param, bk.n_params, bk.row_elems, bk.row_stride, bk.shard_base] == list(pl.buckets[b])

    # state: p32 N(0, 0.02), m = v = 0, step counts 0..2, all-gather block of finite patterns
    p32 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    steps = rng.integers(0, 3, size=len(numels)).astype(np.int32)
    arena = finite_bits(rng, nd * S, dtype)
    for X in (A, F):
        X.p32.copy_(torch.from_numpy(p32))
        X.steps.copy_(torch.from_numpy(steps))
        X.arena.copy_(to_dev16(arena))
    live = (rng.random(len(numels)) > 0.2).astype(np.uint8)
    for X in (A, F):
        X.live.copy_(torch.from_numpy(live))

    # this rank's gradients, dead ones absent, at random (mis)alignments
    grads = [finite_bits(rng, x, dtype) if l else None for x, l in zip(numels, live)]
    _buf, views = placed_views(grads, rng, misalign=bool(rng.random() < 0.5))
    ptrs = Z.ptr_table(views)
    A.packed.fill_(SENT16)
    A.pack(ptrs)
    F.packed.fill_(SENT16)
    F.flag.zero_()
    F.pack(ptrs, check=True)
    torch.cuda.synchronize()
    got_a, got_f = to_np16(A.packed), to_np16(F.packed)
    assert np.array_equal(got_a, got_f)  # the checked pack writes the same bits
    want_flag = 0
    rows = []
    for b in range(pl.n_buckets):
        want = np.full((nd, pl.buckets[b, oracle.B_STRIDE]), SENT16, dtype=np.uint16)
        oracle.pack_bucket(pl, b, grads, out=want)
        assert np.array_equal(oracle_block(pl, got_a, b), want), f"pack bucket {b}"
        want_flag |= oracle.input_check(pl, b, grads, dtype)
        # the Nd ranks' rows r of bucket b: the others random, this rank's from its own pack
        L = int(pl.buckets[b, oracle.B_STRIDE])
        r_rows = finite_bits(rng, nd * L, dtype).reshape(nd, L)
        r_rows[rank] = want[rank]
        rows.append(r_rows)
    assert int(F.flag.item()) == want_flag == 0
    rdev = [to_dev16(r.reshape(-1)) if r.size else torch.zeros(8, dtype=torch.int16, device=DEV) for r in rows]

    def rows_of(b):
        return rdev[b], int(pl.buckets[b, oracle.B_STRIDE])

    # unfused: reduce (+ flag), Adam
    A.flag.zero_()
    A.g32.fill_(-5.0)
    A.reduce(rows_of)
    g32 = np.full(S, -5.0, np.float32)
    for b in range(pl.n_buckets):
        oracle.reduce_bucket(pl, b, rows[b], dtype, live, g32)
    torch.cuda.synchronize()
    assert_same_f32(to_np32(A.g32), g32, "g32")
    flag = oracle.overflow(pl, g32, live)
    assert int(A.flag.item()) == flag == 0
    hp = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=1.0 / nd)
    A.adam(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
    # fused: reduce + Adam per bucket
    F.reduce_adam(rows_of, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
    oracle.adam(pl, g32, p32, m, v, live, steps, hp, 0, arena, dtype)
    torch.cuda.synchronize()
    for ta, tf in ((A.p32, F.p32), (A.m, F.m), (A.v, F.v)):
        assert torch.equal(ta.view(torch.int32), tf.view(torch.int32))
    assert torch.equal(A.steps, F.steps) and torch.equal(A.arena, F.arena)
    assert np.array_equal(to_np32(A.steps), steps)
    assert_close_f32(to_np32(A.p32), p32, "p32")
    assert_close_f32(to_np32(A.m), m, "m")
    assert_close_f32(to_np32(A.v), v, "v", abs_=8 * 2.0 ** -149, rel=2e-6)
    ever = np.zeros(S, dtype=bool)
    for i in np.flatnonzero(live):
        o, s_ = pl.params[i, oracle.P_OFFSET], pl.params[i, oracle.P_SHARD]
        ever[o:o + s_] = True
    got_arena = to_np16(A.arena)
    check_arena(pl, got_arena, arena, to_np32(A.p32), p32, ever, dtype, "arena")

    # unpack the (device) all-gather blocks into fresh, possibly misaligned outputs
    skip = rng.random(len(numels)) < 0.1
    outs = [None if sk else np.full(x, SENT16, dtype=np.uint16) for x, sk in zip(numels, skip)]
    _obuf, oviews = placed_views(outs, rng, misalign=bool(rng.random() < 0.5))
    A.unpack(Z.ptr_table(oviews))
    torch.cuda.synchronize()
    for b in range(pl.n_buckets):
        oracle.unpack_bucket(pl, b, oracle_block(pl, got_arena, b).copy(), outs)
    for i, (o, vw) in enumerate(zip(outs, oviews)):
        if o is not None:
            assert np.array_equal(to_np16(vw), o), f"unpack param {i}"


@pytest.mark.parametrize("seed", range(24))
def test_random_plan_overflow_skips(seed):
    """The same random plans with one inf or NaN planted in this rank's own row of a live
    gradient: the checked pack flags it (the oracle's input check), the unfused reduce flags it
    (the oracle's overflow of the sums), and both paths then skip the step, leaving p32, m, v, the
    step counts and the all-gather block bit for bit as they were."""
    rng, nd, rank, numels, cap, groups, dtype = random_case(seed + 500)
    pl = oracle.plan(numels, nd, rank, cap, groups)
    S = pl.shard_len
    # a live parameter with at least one real element in row `rank`
    cand = [i for i, x in enumerate(numels) if x > rank * pl.params[i, oracle.P_SHARD]]
    if not cand:
        pytest.skip("no parameter has a real element in this rank's row")
    i = int(rng.choice(cand))
    s_i = int(pl.params[i, oracle.P_SHARD])
    j = int(rng.integers(0, min(s_i, numels[i] - rank * s_i)))
    bad = int(rng.choice([0x7F80, 0xFF80, 0x7FC0] if dtype == BF16 else [0x7C00, 0xFC00, 0x7E00]))
    say(f"overflow sweep seed={seed} nd={nd} rank={rank} n={len(numels)} param={i} col={j} bits={bad:#x}")
    gl = None if groups is None else [int(x) for x in groups]
    A = Z.ShardStep(numels, nd, rank, cap, dtype, groups=gl)
    F = Z.ShardStep(numels, nd, rank, cap, dtype, groups=gl)
    live = (rng.random(len(numels)) > 0.2).astype(np.uint8)
    live[i] = 1
    p32 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    arena = finite_bits(rng, nd * S, dtype)
    steps = rng.integers(0, 3, size=len(numels)).astype(np.int32)
    for X in (A, F):
        X.p32.copy_(torch.from_numpy(p32))
        X.m.copy_(torch.from_numpy(p32 * 0.5))
        X.v.copy_(torch.from_numpy(np.abs(p32)))
        X.steps.copy_(torch.from_numpy(steps))
        X.arena.copy_(to_dev16(arena))
        X.live.copy_(torch.from_numpy(live))
    before = [t.clone() for t in (A.p32, A.m, A.v, A.steps, A.arena)]
    grads = [finite_bits(rng, x, dtype) if l else None for x, l in zip(numels, live)]
    grads[i][rank * s_i + j] = bad
    _buf, views = placed_views(grads, rng, misalign=bool(rng.random() < 0.5))
    ptrs = Z.ptr_table(views)
    A.pack(ptrs)
    F.flag.zero_()
    F.pack(ptrs, check=True)
    got = to_np16(A.packed)
    rows, want_check = [], 0
    for b in range(pl.n_buckets):
        L = int(pl.buckets[b, oracle.B_STRIDE])
        r_rows = finite_bits(rng, nd * L, dtype).reshape(nd, L)
        r_rows[rank] = oracle_block(pl, got, b)[rank]
        rows.append(r_rows)
        want_check |= oracle.input_check(pl, b, grads, dtype)
    rdev = [to_dev16(r.reshape(-1)) if r.size else torch.zeros(8, dtype=torch.int16, device=DEV) for r in rows]

    def rows_of(b):
        return rdev[b], int(pl.buckets[b, oracle.B_STRIDE])

    A.flag.zero_()
    A.reduce(rows_of)
    g32 = np.zeros(S, np.float32)
    for b in range(pl.n_buckets):
        oracle.reduce_bucket(pl, b, rows[b], dtype, live, g32)
    torch.cuda.synchronize()
    assert want_check == 1 and int(F.flag.item()) == 1
    assert oracle.overflow(pl, g32, live) == 1 and int(A.flag.item()) == 1
    assert_same_f32(to_np32(A.g32), g32, "g32")
    hp = (1e-3, 0.9, 0.999, 1e-8, 1.0 / nd)
    A.adam(*hp)
    F.reduce_adam(rows_of, *hp)
    torch.cuda.synchronize()
    for X in (A, F):
        for t, t0 in zip((X.p32, X.m, X.v, X.steps, X.arena), before):
            assert torch.equal(t, t0)


@pytest.mark.parametrize("seed", range(16))
def test_random_zero3_schedule(seed):
    """Random layered models (1 to 12 layers of 1 to 6 parameters, empty ones included) through
    ZeRO-3's schedule (one stream, prefetch, or the fused layer steps): every gather (forward and backward) against the
    oracle's unpack, the gather order, each layer's packed gradients, the reduced shard and flag,
    then Adam, against the oracle."""
    rng = np.random.default_rng(20_000 + seed)
    nd = int(rng.choice(NDS))
    rank = int(rng.integers(0, nd))
    n_layers = int(rng.integers(1, 13))
    numels, groups = [], []
    for layer in range(n_layers):
        for _ in range(int(rng.integers(1, 7))):
            k = rng.random()
            numels.append(0 if k < 0.1 else int(rng.integers(1, 2 * nd + 2)) if k < 0.4 else
                          int(rng.integers(1, 30000)))
            groups.append(layer)
    dtype = BF16 if rng.random() < 0.5 else FP16
    mode = ("one-stream", "prefetch", "fused")[int(rng.integers(0, 3))]
    prefetch = mode == "prefetch"
    batch = int(rng.integers(1, Z.Z3_MAX_BUCKETS + 1)) if mode == "fused" else 1
    say(f"zero3 sweep seed={seed} nd={nd} rank={rank} layers={n_layers} n={len(numels)} {mode} batch={batch}")
    st = Z.ShardStep(numels, nd, rank, 0, dtype, groups=groups)
    pl = oracle.plan(numels, nd, rank, 0, np.array(groups, np.int32))
    assert pl.n_buckets == n_layers
    S = pl.shard_len
    lp = [finite_bits(rng, x, dtype) for x in numels]
    arena = np.zeros(nd * S, np.uint16)
    for b in range(pl.n_buckets):
        oracle_block(pl, arena, b)[:] = oracle.pack_bucket(pl, b, lp)
    st.arena.copy_(to_dev16(arena))
    p32 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    st.p32.copy_(torch.from_numpy(p32))
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    steps = np.zeros(len(numels), np.int32)
    live = (rng.random(len(numels)) > 0.2).astype(np.uint8)
    st.live.copy_(torch.from_numpy(live))
    z3 = Z.Zero3Schedule(st, prefetch=prefetch, fused=mode == "fused", batch=batch)

    def check_gather(lid, params):
        outs = [np.zeros(x, np.uint16) for x in numels]
        oracle.unpack_bucket(pl, lid, oracle_block(pl, arena, lid).copy(), outs)
        for i, view in zip(z3.layers[lid], params):
            got = to_np16(view)
            assert np.array_equal(got, outs[i]) and np.array_equal(got, lp[i]), (lid, i)

    grads = [finite_bits(rng, x, dtype) if l else None for x, l in zip(numels, live)]
    gptrs = Z.ptr_table([None if g is None else to_dev16(g) for g in grads])
    rows = [finite_bits(rng, nd * int(pl.buckets[b, oracle.B_STRIDE]), dtype).reshape(nd, -1)
            for b in range(pl.n_buckets)]
    want_packed = []
    for b in range(pl.n_buckets):
        want = np.full((nd, pl.buckets[b, oracle.B_STRIDE]), SENT16, dtype=np.uint16)
        oracle.pack_bucket(pl, b, grads, out=want)
        want_packed.append(want)
        rows[b][rank] = want[rank]
    rdev = [to_dev16(r.reshape(-1)) if r.size else torch.zeros(8, dtype=torch.int16, device=DEV) for r in rows]
    out = torch.full_like(st.packed, SENT16)
    st.flag.zero_()
    st.g32.fill_(-3.0)
    z3.forward(check_gather)
    z3.backward(lambda lid: gptrs, lambda lid: (rdev[lid], int(pl.buckets[lid, oracle.B_STRIDE])), check_gather,
                out=out)
    last = z3.batches[-1][1] - z3.batches[-1][0]  # the last batch is not gathered twice
    assert z3.order == list(range(n_layers)) + list(range(n_layers - last - 1, -1, -1))
    torch.cuda.synchronize()
    got_out = to_np16(out)
    for b in range(pl.n_buckets):
        assert np.array_equal(oracle_block(pl, got_out, b), want_packed[b]), f"packed layer {b}"
    g32 = np.full(S, -3.0, np.float32)
    for b in range(pl.n_buckets):
        oracle.reduce_bucket(pl, b, rows[b], dtype, live, g32)
    assert_same_f32(to_np32(st.g32), g32, "g32")
    assert int(st.flag.item()) == oracle.overflow(pl, g32, live) == 0
    hp = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=1.0 / nd)
    st.adam(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
    oracle.adam(pl, g32, p32, m, v, live, steps, hp, 0, arena, dtype)
    torch.cuda.synchronize()
    assert np.array_equal(to_np32(st.steps), steps)
    assert_close_f32(to_np32(st.p32), p32, "p32")
    assert_close_f32(to_np32(st.m), m, "m")
    assert_close_f32(to_np32(st.v), v, "v", abs_=8 * 2.0 ** -149, rel=2e-6)
    ever = np.zeros(S, dtype=bool)
    for i in np.flatnonzero(live):
        o, s_ = pl.params[i, oracle.P_OFFSET], pl.params[i, oracle.P_SHARD]
        ever[o:o + s_] = True
    check_arena(pl, to_np16(st.arena), arena, to_np32(st.p32), p32, ever, dtype, "arena")


@pytest.mark.parametrize("seed", SMALL_GRID_SEEDS)
def test_random_plan_whole_step_small_grids(seed):
    """The same parity with the library built with every grid capped at 37 blocks: each block
    then takes many tiles, row groups and chunk groups in turn (the pack restages its LDS for
    every mixed tile, the fused kernel reuses its LDS across tiles), so what is checked here is
    the kernels' loops over their work items, which the one-shot grids never iterate."""
    with Z._binding.library(Z._binding.SMALL_GRID_LIB_PATH):
        test_random_plan_whole_step(seed)
