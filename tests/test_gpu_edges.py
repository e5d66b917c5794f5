"""Edge cases of the shard pipeline on the GPU, through the C ABI: an empty shard, one
parameter past 2^32 elements (64-bit indexing everywhere), the largest Nd, a step in which no
parameter has a gradient, argument rejection by every hot call, and bit-for-bit determinism
of repeated runs."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_amd as Z
from zero_sharded_mixed_amd import _binding as B
from gpu_harness import (DEV, assert_close_f32, assert_same_f32, ragged_numels, random_bits, to_dev16, to_np16,
                         to_np32)

pytestmark = pytest.mark.gpu
BF16, FP16 = Z.ZERO_BF16, Z.ZERO_FP16
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=0.5)


def test_empty_shard_every_entry_point():
    st = Z.ShardStep([0, 0, 0, 0], 4, 1, 0, BF16)
    assert st.summary.shard_numel == 0 and st.summary.arena_numel == 0
    dummy = torch.zeros(64, dtype=torch.int16, device=DEV)
    g32 = torch.zeros(8, dtype=torch.float32, device=DEV)
    ptrs = Z.ptr_table([dummy[:0]] * 4)
    Z.zero_shard_init(st.plan, ptrs, 0, g32)
    Z.zero_pack_bucket(st.plan, 0, ptrs, dummy)
    Z.zero_reduce_shard(st.plan, 0, dummy, 0, st.live, g32, st.flag)
    Z.zero_overflow_check(st.plan, g32, st.live, st.flag)
    Z.zero_adam_step(st.plan, g32, g32, g32, g32, st.live, st.steps, **HP, flag=st.flag, arena=dummy)
    Z.zero_unpack(st.plan, 0, dummy, ptrs)
    torch.cuda.synchronize()
    assert int(st.flag.item()) == 0
    assert torch.all(st.steps == 1)  # live parameters count a step even when they hold no elements
    assert torch.all(dummy == 0) and torch.all(g32 == 0)


def test_parameter_past_two_to_the_32():
    """One parameter of 2^32 + 5 elements at Nd = 2: shard offsets, row strides and element
    indices all pass 2^31 and 2^32."""
    n = (1 << 32) + 5
    nd, r = 2, 1
    st = Z.ShardStep([n], nd, r, 0, BF16)
    pl = oracle.plan([n], nd, r, 0)
    s_ = pl.params[0, oracle.P_SHARD]
    L = int(pl.buckets[0, oracle.B_STRIDE])
    assert s_ == (n + 1) // 2 and L == ((s_ + 7) // 8) * 8
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    g = torch.randint(-32768, 32767, (n,), generator=gen, dtype=torch.int16, device=DEV)
    g.bitwise_and_(~0x4000)  # clear the top exponent bit: finite bf16 patterns only
    st.pack(Z.ptr_table([g]))
    # sampled positions, the end of each row included
    rng = np.random.default_rng(6)
    ks = np.concatenate([rng.integers(0, nd, 200), [0, 1, 1, 1]])
    cs = np.concatenate([rng.integers(0, L, 200), [s_ - 1, s_ - 1, s_ - 2, L - 1]])
    for k, c in zip(ks, cs):
        kind, i, e = oracle.pack_locate(pl, 0, int(k), int(c))
        want = int(g[e].item()) & 0xFFFF if kind == 1 else 0
        assert int(st.packed[int(k) * L + int(c)].item()) & 0xFFFF == want, (k, c)
    # reduce and Adam near the end of the shard
    Z.zero_reduce_shard(st.plan, 0, st.packed, L, st.live, st.g32, st.flag)
    assert int(st.flag.item()) == 0
    cols = np.concatenate([rng.integers(0, s_, 200), [s_ - 1, s_ - 2, 0]])
    rows = to_np16(st.packed.view(nd, L)[:, torch.from_numpy(cols).to(DEV)].contiguous())
    want_g = np.array([oracle.reduce_column(rows[:, t], BF16) for t in range(cols.size)], np.float32)
    assert_same_f32(to_np32(st.g32[torch.from_numpy(cols).to(DEV)]), want_g, "g32")
    st.p32.fill_(0.25)
    st.adam(**{k: v for k, v in HP.items()})
    for t, col in enumerate(cols[:50]):
        p, m, v = oracle.adam_element(want_g[t], np.float32(0.25), np.float32(0), np.float32(0), 1,
                                      oracle.AdamHP(**HP))
        assert_close_f32(to_np32(st.p32[int(col):int(col) + 1]), np.array([p], np.float32), "p32")
    # unpack of a gathered block of random bits, checked at the top of the parameter
    gathered = torch.randint(-32768, 32767, (nd * L,), generator=gen, dtype=torch.int16, device=DEV)
    out = torch.zeros(n, dtype=torch.int16, device=DEV)
    Z.zero_unpack(st.plan, 0, gathered, Z.ptr_table([out]))
    for e in [0, 1, s_ - 1, s_, n - 2, n - 1, (1 << 32) - 1, 1 << 32]:
        row, col = oracle.unpack_locate(pl, 0, int(e))
        assert int(out[e].item()) == int(gathered[row * L + col].item()), e
    del g, gathered, out, st
    torch.cuda.empty_cache()


def test_largest_nd():
    nd, r = 65535, 40000
    rng = np.random.default_rng(7)
    numels = [int(x) for x in rng.integers(0, 400_000, size=12)] + [nd - 1, nd, 1]
    st = Z.ShardStep(numels, nd, r, 0, FP16)
    pl = oracle.plan(numels, nd, r, 0)
    L = int(pl.buckets[0, oracle.B_STRIDE])
    grads = [random_bits(rng, x) for x in numels]
    st.pack(Z.ptr_table([to_dev16(g) for g in grads]))
    want = oracle.pack_bucket(pl, 0, grads)
    assert np.array_equal(to_np16(st.packed).reshape(nd, L), want)
    rows = (random_bits(rng, nd * L) & np.uint16(0x3BFF)).reshape(nd, L)  # finite fp16
    Z.zero_reduce_shard(st.plan, 0, to_dev16(rows.reshape(-1)), L, st.live, st.g32, st.flag)
    g32 = np.zeros(pl.shard_len, np.float32)
    oracle.reduce_bucket(pl, 0, rows, FP16, np.ones(len(numels), np.uint8), g32)
    assert_same_f32(to_np32(st.g32), g32, "g32")
    assert int(st.flag.item()) == 0


def test_step_without_any_gradient():
    rng = np.random.default_rng(8)
    numels = ragged_numels(rng, 50, 8, 30000)
    st = Z.ShardStep(numels, 8, 2, 2 * 20000, BF16)
    st.live.zero_()
    st.g32.fill_(float("nan"))  # would poison anything that read it
    st.p32.normal_()
    before = [t.clone() for t in (st.p32, st.m, st.v, st.arena, st.steps)]
    rows = torch.full((8 * int(st.summary.shard_numel) + 64,), 0x7C00, dtype=torch.int16, device=DEV)
    st.reduce(lambda b: (rows[8 * st.buckets[b].shard_base:], int(st.buckets[b].row_stride)))
    st.overflow_check()
    st.adam(**HP)
    torch.cuda.synchronize()
    assert int(st.flag.item()) == 0  # nothing live: nothing to overflow
    for a, t in zip(before, (st.p32, st.m, st.v, st.arena, st.steps)):
        assert torch.equal(a.view(torch.int8) if a.dtype != torch.int32 else a,
                           t.view(torch.int8) if t.dtype != torch.int32 else t)
    assert torch.all(torch.isnan(st.g32))  # the reduce wrote no dead column


def _status(call):
    try:
        call()
    except Z.ZeroError as e:
        return e.status
    return B.ZERO_OK


def test_hot_calls_reject_bad_arguments():
    st = Z.ShardStep([1000, 37, 5000], 8, 3, 0, BF16)
    L = int(st.buckets[0].row_stride)
    buf = torch.zeros(8 * L + 64, dtype=torch.int16, device=DEV)
    ptrs = Z.ptr_table([torch.zeros(x, dtype=torch.int16, device=DEV) for x in (1000, 37, 5000)])
    f = torch.zeros(int(st.summary.shard_numel) + 8, dtype=torch.float32, device=DEV)
    E = B.ZERO_EINVAL
    assert _status(lambda: Z.zero_pack_bucket(st.plan, 1, ptrs, buf)) == E          # bucket out of range
    assert _status(lambda: Z.zero_pack_bucket(st.plan, -1, ptrs, buf)) == E
    assert _status(lambda: Z.zero_pack_bucket(st.plan, 0, ptrs, buf[1:])) == E      # misaligned block
    assert _status(lambda: Z.zero_reduce_shard(st.plan, 0, buf, L - 8, st.live, f)) == E  # stride < L_b
    assert _status(lambda: Z.zero_reduce_shard(st.plan, 0, buf, L + 4, st.live, f)) == E  # stride % 8
    assert _status(lambda: Z.zero_reduce_shard(st.plan, 0, buf[1:], L, st.live, f)) == E  # misaligned rows
    assert _status(lambda: Z.zero_reduce_shard(st.plan, 0, buf, L, st.live, f[1:])) == E  # misaligned g32
    assert _status(lambda: Z.zero_overflow_check(st.plan, f[2:], st.live, st.flag)) == E
    for bad in (dict(beta1=1.0), dict(beta2=-0.1), dict(lr=float("inf")), dict(eps=float("nan"))):
        hp = dict(HP, **bad)
        assert _status(lambda: Z.zero_adam_step(st.plan, f, f, f, f, st.live, st.steps, **hp, flag=None,
                                                arena=st.arena)) == E
    assert _status(lambda: Z.zero_adam_step(st.plan, f[1:], f, f, f, st.live, st.steps, **HP, flag=None,
                                            arena=st.arena)) == E
    assert _status(lambda: Z.zero_unpack(st.plan, 0, buf[3:], ptrs)) == E
    assert _status(lambda: Z.zero_shard_init(st.plan, ptrs, 7, f)) == E
    L_ = B.lib()
    assert L_.zero_pack_bucket(st.plan.handle, 0, None, ctypes.c_void_p(buf.data_ptr()), None) == E
    assert Z.zero_last_error().startswith("zero_pack_bucket")
    torch.cuda.synchronize()
    assert int(st.steps.sum().item()) == 0  # nothing ran


def test_repeated_runs_are_bit_identical():
    """Same inputs, same outputs, bit for bit: no kernel depends on timing or scheduling."""
    rng = np.random.default_rng(9)
    numels = ragged_numels(rng, 120, 64, 200000)
    outs = []
    grads = [random_bits(rng, x) & np.uint16(0xBFFF) for x in numels]
    rows = None
    for rep in range(2):
        st = Z.ShardStep(numels, 64, 17, 2 * 300000, BF16)
        if rows is None:
            rows = [(random_bits(rng, 64 * int(bk.row_stride)) & np.uint16(0xBBFF)) for bk in st.buckets]
        st.p32.copy_(torch.linspace(-0.05, 0.05, st.p32.numel(), device=DEV))
        st.pack(Z.ptr_table([to_dev16(g) for g in grads]))
        rdev = [to_dev16(r_) for r_ in rows]
        st.reduce(lambda b: (rdev[b], int(st.buckets[b].row_stride)))
        st.adam(**HP)
        params = [torch.zeros(x, dtype=torch.int16, device=DEV) for x in numels]
        st.unpack(Z.ptr_table(params))
        torch.cuda.synchronize()
        outs.append([to_np16(st.packed), to_np32(st.g32).view(np.uint32), to_np32(st.p32).view(np.uint32),
                     to_np32(st.m).view(np.uint32), to_np32(st.v).view(np.uint32), to_np16(st.arena),
                     np.concatenate([to_np16(p) for p in params])])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_empty_buckets_and_shards_take_null_buffers():
    """A bucket holding only empty parameters (here closed off by a one-element capacity) has
    empty rows; its block is a zero-length tensor whose data pointer is NULL.  Every per-bucket
    call accepts that and does nothing, and the whole step runs through ShardStep, unfused and
    fused, with the other buckets matching the oracle.  A model of only empty parameters runs
    every call with NULL shard buffers."""
    numels, nd, rank = [100, 0, 0, 50], 4, 1
    st = Z.ShardStep(numels, nd, rank, 2, BF16)
    pl = oracle.plan(numels, nd, rank, 2)
    assert [int(bk.row_stride) for bk in st.buckets] == [32, 0, 16]  # the two empty ones share a bucket
    assert st.block(st.packed, 1).numel() == 0
    L_ = B.lib()
    for b in (1,):  # NULL buffers on an empty bucket: nothing to do, no error
        assert L_.zero_pack_bucket(st.plan.handle, b, None, None, None) == B.ZERO_OK
        assert L_.zero_pack_bucket_check(st.plan.handle, b, None, None, None, None) == B.ZERO_OK
        assert L_.zero_unpack(st.plan.handle, b, None, None, None) == B.ZERO_OK
        assert L_.zero_reduce_shard(st.plan.handle, b, None, 0, None, None, None, None) == B.ZERO_OK
        assert L_.zero_reduce_adam_bucket(st.plan.handle, b, None, 0, None, None, None, None, None, None,
                                          None) == B.ZERO_OK
    rng = np.random.default_rng(12)
    grads = [(rng.standard_normal(x) * 1e-2).astype(np.float32) for x in numels]
    g16 = [torch.from_numpy(g).to(torch.bfloat16).to(DEV) for g in grads]
    host = [to_np16(t) for t in g16]
    st.pack(Z.ptr_table(g16))
    want = np.zeros(int(st.summary.arena_numel), np.uint16)
    for b in range(pl.n_buckets):
        L = int(pl.buckets[b, oracle.B_STRIDE])
        if L:
            off = nd * int(pl.buckets[b, oracle.B_BASE])
            want[off:off + nd * L] = oracle.pack_bucket(pl, b, host).reshape(-1)
    torch.cuda.synchronize()
    assert np.array_equal(to_np16(st.packed), want)
    F = Z.ShardStep(numels, nd, rank, 2, BF16)
    F.pack(Z.ptr_table(g16), check=True)
    rows_of = lambda b: (st.block(st.packed, b), int(st.buckets[b].row_stride))  # noqa: E731
    st.reduce(rows_of)
    st.adam(**HP)
    F.reduce_adam(rows_of, **HP)
    g32 = np.zeros(pl.shard_len, np.float32)
    live = np.ones(len(numels), np.uint8)
    for b in range(pl.n_buckets):
        L = int(pl.buckets[b, oracle.B_STRIDE])
        off = nd * int(pl.buckets[b, oracle.B_BASE])
        oracle.reduce_bucket(pl, b, want[off:off + nd * L].reshape(nd, L), BF16, live, g32)
    st.unpack(Z.ptr_table(g16))
    torch.cuda.synchronize()
    assert_same_f32(to_np32(st.g32), g32, "g32")
    assert torch.equal(st.p32, F.p32) and torch.equal(st.arena, F.arena)
    assert torch.all(st.steps == 1) and int(st.flag.item()) == int(F.flag.item()) == 0
    # a model of only empty parameters: every shard buffer has no elements (NULL pointers)
    E = Z.ShardStep([0, 0, 0], 8, 5, 0, FP16)
    assert E.p32.numel() == 0 and E.packed.numel() == 0
    empty = Z.ptr_table([E.packed] * 3)
    E.init_master(empty, 0)
    E.pack(empty, check=True)
    E.reduce(lambda b: (E.packed, 0))
    E.overflow_check()
    E.adam(**HP)
    E.reduce_adam(lambda b: (E.packed, 0), **HP)
    E.unpack(empty)
    torch.cuda.synchronize()
    assert torch.all(E.steps == 2) and int(E.flag.item()) == 0

