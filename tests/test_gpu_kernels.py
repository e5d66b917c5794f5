"""Parity of every HIP kernel with the oracle on small ragged plans (several tiles each, ragged
tails, empty parameters, numel < Nd, dead parameters, misaligned per-parameter buffers),
called through the C ABI.  Pack, unpack, plan, shard init and reduce are compared bit for bit
(NaN equals NaN); Adam's fp32 state within |d| <= 1e-7 + 1e-6 |ref| and the 16-bit parameters
within 1 ulp."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_amd as Z
from gpu_harness import (DEV, assert_close_f32, assert_same_f32, check_arena, oracle_block, placed_views,
                         ragged_numels, random_bits, say, to_dev16, to_np16, to_np32)

pytestmark = pytest.mark.gpu

BF16, FP16 = Z.ZERO_BF16, Z.ZERO_FP16
SENT16 = 0x5A5A

CASES = [  # (nd, rank, n_params, max numel, bucket bytes, seed)
    (1, 0, 40, 30000, 0, 1),
    (3, 2, 60, 20000, 2 * 9000, 2),
    (8, 3, 80, 70000, 2 * 60000, 3),
    (64, 63, 120, 200000, 2 * 400000, 4),
    (1024, 517, 150, 300000, 2 * 2_000_000, 5),
]


def make(case):
    nd, rank, n, hi, cap, seed = case
    rng = np.random.default_rng(seed)
    numels = ragged_numels(rng, n, nd, hi)
    say(f"case nd={nd} rank={rank} n={n} cap={cap} total={sum(numels)}")
    step = Z.ShardStep(numels, nd, rank, cap, BF16)
    return rng, numels, step, oracle.plan(numels, nd, rank, cap)


@pytest.mark.parametrize("case", CASES)
def test_plan_tables(case):
    _, numels, st, pl = make(case)
    s = st.summary
    assert (s.n_params, s.nd, s.rank, s.n_buckets, s.shard_numel) == (len(numels), pl.nd, pl.rank, pl.n_buckets,
                                                                     pl.shard_len)
    assert s.padded_total == pl.params[:, oracle.P_PADDED].sum() and s.numel_total == sum(numels)
    assert s.shard_elems == pl.params[:, oracle.P_SHARD].sum() and s.arena_numel == pl.nd * pl.shard_len
    for i in range(len(numels)):
        info = Z.zero_plan_param_info(st.plan, i)
        got = [info.numel, info.pad, info.padded_numel, info.shard_size, info.shard_start, info.shard_end,
               info.shard_offset, info.bucket, info.bucket_col]
        assert got == list(pl.params[i]), i
    for b in range(pl.n_buckets):
        bk = Z.zero_plan_bucket_info(st.plan, b)
        assert [bk.first_param, bk.n_params, bk.row_elems, bk.row_stride, bk.shard_base] == list(pl.buckets[b])
        assert bk.block_offset == pl.nd * pl.buckets[b, oracle.B_BASE]


@pytest.mark.parametrize("bucket_bytes", [0, 2, 2 * 1000, 2 * 123457])
def test_plan_tables_bucket_sizes(bucket_bytes):
    rng = np.random.default_rng(bucket_bytes)
    numels = ragged_numels(rng, 300, 8, 50000)
    plan = Z.zero_plan_create(numels, 8, 5, bucket_bytes, FP16)
    pl = oracle.plan(numels, 8, 5, bucket_bytes)
    for i in range(len(numels)):
        info = Z.zero_plan_param_info(plan, i)
        assert (info.shard_offset, info.bucket, info.bucket_col) == tuple(pl.params[i, [6, 7, 8]])
    assert Z.zero_plan_get_summary(plan).n_buckets == pl.n_buckets


def test_plan_of_empty_parameters():
    plan = Z.zero_plan_create([0, 0, 0], 4, 1, 0, BF16)
    s = Z.zero_plan_get_summary(plan)
    assert s.shard_numel == 0 and s.n_buckets == 1 and s.padded_total == 0


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("misalign", [False, True])
def test_pack(case, misalign):
    rng, numels, st, pl = make(case)
    grads = [random_bits(rng, x) for x in numels]  # every bit pattern, NaN payloads included
    dead = rng.random(len(numels)) < 0.2
    src = [None if d else g for g, d in zip(grads, dead)]
    _buf, views = placed_views(src, rng, misalign)
    st.packed.fill_(SENT16)
    st.pack(Z.ptr_table(views))
    torch.cuda.synchronize()
    got = to_np16(st.packed)
    for b in range(pl.n_buckets):
        want = np.full((pl.nd, pl.buckets[b, oracle.B_STRIDE]), SENT16, dtype=np.uint16)
        oracle.pack_bucket(pl, b, src, out=want)
        assert np.array_equal(oracle_block(pl, got, b), want), f"bucket {b}"


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("misalign", [False, True])
def test_unpack(case, misalign):
    rng, numels, st, pl = make(case)
    gathered = random_bits(rng, pl.nd * pl.shard_len)
    skip = rng.random(len(numels)) < 0.15
    outs = [None if s else np.full(x, SENT16, dtype=np.uint16) for x, s in zip(numels, skip)]
    _buf, views = placed_views(outs, rng, misalign)
    st.unpack(Z.ptr_table(views), src=to_dev16(gathered))
    torch.cuda.synchronize()
    for b in range(pl.n_buckets):
        oracle.unpack_bucket(pl, b, oracle_block(pl, gathered, b).copy(), outs)
    for i, (o, v) in enumerate(zip(outs, views)):
        if o is not None:
            assert np.array_equal(to_np16(v), o), f"param {i}"


def special_rows(rng, nd, L, dtype):
    """16-bit rows: normal values with some subnormals, signed zeros, infinities and NaNs."""
    t = torch.randn(nd * L, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
    h = to_np16(t.to(torch.bfloat16 if dtype == BF16 else torch.float16).to(DEV))
    pos = rng.choice(h.size, size=max(1, h.size // 500), replace=False)
    specials = np.array([0x0001, 0x8001, 0x03FF, 0x8000, 0x0000] if dtype == FP16 else
                        [0x0001, 0x8001, 0x007F, 0x8000, 0x0000], dtype=np.uint16)
    h[pos] = specials[rng.integers(0, specials.size, size=pos.size)]
    pos = rng.choice(h.size, size=max(1, h.size // 20000), replace=False)
    nonfinite = np.array([0x7C00, 0xFC00, 0x7E00] if dtype == FP16 else [0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16)
    h[pos] = nonfinite[rng.integers(0, 3, size=pos.size)]
    return h.reshape(nd, L)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_reduce_and_fused_flag(case, dtype):
    nd, rank, n, hi, cap, seed = case
    rng = np.random.default_rng(seed + 100)
    numels = ragged_numels(rng, n, nd, hi)
    st = Z.ShardStep(numels, nd, rank, cap, dtype)
    pl = oracle.plan(numels, nd, rank, cap)
    live = (rng.random(len(numels)) > 0.25).astype(np.uint8)
    st.live.copy_(torch.from_numpy(live))
    st.g32.fill_(-7.0)
    want = np.full(pl.shard_len, -7.0, dtype=np.float32)
    for b in range(pl.n_buckets):
        L = int(pl.buckets[b, oracle.B_STRIDE])
        extra = 8 * int(rng.integers(0, 3))  # row stride above L_b
        rows = special_rows(rng, nd, L + extra, dtype) if L else np.zeros((nd, extra), np.uint16)
        oracle.reduce_bucket(pl, b, np.ascontiguousarray(rows), dtype, live, want)
        st_rows = to_dev16(rows.reshape(-1)) if rows.size else torch.zeros(8, dtype=torch.int16, device=DEV)
        Z.zero_reduce_shard(st.plan, b, st_rows, L + extra, st.live, st.g32, st.flag)
    torch.cuda.synchronize()
    assert_same_f32(to_np32(st.g32), want, "g32")
    assert int(st.flag.item()) == oracle.overflow(pl, want, live)
    # the standalone check agrees with the fused one
    st.flag.zero_()
    st.overflow_check()
    assert int(st.flag.item()) == oracle.overflow(pl, want, live)


@pytest.mark.parametrize("nd", [15, 16, 17, 40])
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_reduce_row_forms_around_nd_16(nd, dtype):
    """The reduce runs one kernel below Nd = 16 (one group of rows in flight on every tile) and
    another from Nd = 16 (one group on tiles inside one parameter, two on the others); both sides
    of that switch, with partial last groups (Nd = 15, 17, 40) and whole tiles next to mixed ones,
    match the oracle bit for bit."""
    rng = np.random.default_rng(nd)
    numels = [nd * 2048 * 3 + 5, 7, nd * 2048 - 3, nd * 4096, 100003] + ragged_numels(rng, 30, nd, 90000)
    st = Z.ShardStep(numels, nd, nd - 2, 0, dtype)
    pl = oracle.plan(numels, nd, nd - 2, 0)
    live = np.ones(len(numels), dtype=np.uint8)
    live[1::4] = 0
    st.live.copy_(torch.from_numpy(live))
    st.g32.fill_(-7.0)
    want = np.full(pl.shard_len, -7.0, dtype=np.float32)
    for b in range(pl.n_buckets):
        L = int(pl.buckets[b, oracle.B_STRIDE])
        rows = special_rows(rng, nd, L + 8, dtype)
        oracle.reduce_bucket(pl, b, np.ascontiguousarray(rows), dtype, live, want)
        Z.zero_reduce_shard(st.plan, b, to_dev16(rows.reshape(-1)), L + 8, st.live, st.g32, st.flag)
    torch.cuda.synchronize()
    say(f"reduce row forms nd={nd} dtype={dtype} shard={pl.shard_len}")
    assert_same_f32(to_np32(st.g32), want, "g32")
    assert int(st.flag.item()) == oracle.overflow(pl, want, live)


def test_reduce_exact_order_example():
    """Rows 1, 2^-24, 2^-24 must reduce to 1.0 (ascending order, seeded with rank 0)."""
    st = Z.ShardStep([3 * 64], 3, 0, 0, BF16)
    one, tiny = 0x3F80, 0x3380  # bf16 bits of 1.0 and 2^-24
    rows = np.array([[one] * 64, [tiny] * 64, [tiny] * 64], dtype=np.uint16)
    Z.zero_reduce_shard(st.plan, 0, to_dev16(rows.reshape(-1)), 64, st.live, st.g32)
    assert np.all(to_np32(st.g32)[:64] == 1.0)


def test_overflow_check_injections():
    rng = np.random.default_rng(9)
    numels = ragged_numels(rng, 200, 8, 40000)
    st = Z.ShardStep(numels, 8, 2, 2 * 50000, FP16)
    pl = oracle.plan(numels, 8, 2, 2 * 50000)
    live = (rng.random(len(numels)) > 0.3).astype(np.uint8)
    st.live.copy_(torch.from_numpy(live))
    base = rng.standard_normal(pl.shard_len).astype(np.float32)
    for trial in range(6):
        g = base.copy()
        if trial > 0:
            pos = rng.choice(pl.shard_len, size=trial, replace=False)
            g[pos] = np.array([np.inf, -np.inf, np.nan])[rng.integers(0, 3, size=trial)]
        st.g32.copy_(torch.from_numpy(g))
        st.flag.zero_()
        st.overflow_check()
        assert int(st.flag.item()) == oracle.overflow(pl, g, live), trial


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("src_dtype", [0, BF16, FP16])
def test_shard_init(case, src_dtype):
    rng, numels, st, pl = make(case)
    if src_dtype == 0:
        masters = [rng.standard_normal(x).astype(np.float32) for x in numels]
        dev = [torch.from_numpy(a).to(DEV) for a in masters]
    else:
        masters = [random_bits(rng, x) & np.uint16(0xBFFF) for x in numels]  # finite patterns
        dev = [to_dev16(a) for a in masters]
    skip = rng.random(len(numels)) < 0.1
    masters = [None if s else a for a, s in zip(masters, skip)]
    dev = [None if s else t for t, s in zip(dev, skip)]
    st.p32.fill_(3.25)
    st.init_master(Z.ptr_table(dev), src_dtype)
    want = np.full(pl.shard_len, 3.25, dtype=np.float32)
    oracle.shard_init(pl, masters, want, src_dtype)
    torch.cuda.synchronize()
    assert_same_f32(to_np32(st.p32), want, "p32")


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_adam_steps(case, dtype):
    nd, rank, n, hi, cap, seed = case
    rng = np.random.default_rng(seed + 200)
    numels = ragged_numels(rng, n, nd, hi)
    st = Z.ShardStep(numels, nd, rank, cap, dtype)
    pl = oracle.plan(numels, nd, rank, cap)
    S = pl.shard_len
    p32 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    steps = rng.integers(0, 3, size=len(numels)).astype(np.int32)
    arena = random_bits(rng, nd * S) & np.uint16(0xBFFF)
    for t, a in ((st.p32, p32), (st.m, m), (st.v, v)):
        t.copy_(torch.from_numpy(a))
    st.steps.copy_(torch.from_numpy(steps))
    st.arena.copy_(to_dev16(arena))
    hp = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=1.0 / 8)
    ever = np.zeros(S, dtype=bool)  # columns of parameters that have taken a step
    for step in range(4):
        live = (rng.random(len(numels)) > 0.3).astype(np.uint8)
        g32 = (rng.standard_normal(S) * 1e-2).astype(np.float32)
        g32[rng.random(S) < 0.05] = 0.0
        flag = 1 if step == 2 else 0  # one skipped step
        st.live.copy_(torch.from_numpy(live))
        st.g32.copy_(torch.from_numpy(g32))
        st.flag.fill_(flag)
        before = [to_np32(t) for t in (st.p32, st.m, st.v)]
        st.adam(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
        oracle.adam(pl, g32, p32, m, v, live, steps, hp, flag, arena, dtype)
        torch.cuda.synchronize()
        assert np.array_equal(to_np32(st.steps), steps)
        assert_close_f32(to_np32(st.p32), p32, f"p32 step {step}")
        assert_close_f32(to_np32(st.m), m, f"m step {step}")
        assert_close_f32(to_np32(st.v), v, f"v step {step}", abs_=0.0, rel=2e-6)
        # a parameter without a gradient (and every parameter on a skipped step) keeps its state
        # bit for bit; so do the row gaps
        keep = np.ones(S, dtype=bool)
        if not flag:
            for i in np.flatnonzero(live):
                o, s = pl.params[i, oracle.P_OFFSET], pl.params[i, oracle.P_SHARD]
                keep[o:o + s] = False
        ever |= ~keep
        got_arena = to_np16(st.arena)
        check_arena(pl, got_arena, arena, to_np32(st.p32), p32, ever, dtype, f"arena {step}")
        for name, old, t in zip("pmv", before, (st.p32, st.m, st.v)):
            assert np.array_equal(old[keep].view(np.uint32), to_np32(t)[keep].view(np.uint32)), name


def test_adam_first_step_closed_form():
    """From m = v = 0 the first step moves p by lr * g / (|g| + eps) (a closed form, not the
    oracle): checks the kernel's bias correction on its own."""
    S = 4096
    st = Z.ShardStep([S], 1, 0, 0, BF16)
    rng = np.random.default_rng(11)
    p0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    g = (rng.standard_normal(S) * 1e-3).astype(np.float32)
    st.p32.copy_(torch.from_numpy(p0))
    st.g32.copy_(torch.from_numpy(g))
    st.adam(1e-3, 0.9, 0.999, 1e-8, 1.0)
    g64 = g.astype(np.float64)
    assert_close_f32(to_np32(st.p32), (p0 - 1e-3 * g64 / (np.abs(g64) + 1e-8)).astype(np.float32), "p1",
                     rel=1e-6, abs_=1e-9)
