"""The fused path on the GPU, through the C ABI: the checked pack (packed bits and input
verdict against the oracle, injections in every code path of the pack), the fused reduce +
Adam (bit-identical to zero_reduce_shard + zero_adam_step on the same rows and against the
oracle within the Adam tolerance), skipping on a set flag, argument rejection, and the full-size
workloads in the launch configuration bench.py times."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import zero_sharded_mixed_amd as Z
from gpu_harness import (DEV, assert_close_f32, bits16, check_arena, column_owner, gather_params, placed_views,
                         ragged_numels, random_bits, row_zero_mask, sample_columns, say, to_dev16, to_np16, to_np32)

pytestmark = pytest.mark.gpu
BF16, FP16 = Z.ZERO_BF16, Z.ZERO_FP16
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=1.0 / 8)
# v's bound: 2e-6 relative, with a floor of 8 units of fp32's subnormal spacing 2^-149 (the
# random-bit gradients here reach down to 2^-126, where g * g is subnormal and every fp32 operation
# rounds at that fixed absolute spacing)
V_ABS = 8 * 2.0 ** -149
P_OFF, P_S, P_NUMEL = oracle.P_OFFSET, oracle.P_SHARD, oracle.P_NUMEL

CASES = [  # (nd, rank, bucket bytes, seed)
    (1, 0, 0, 1),
    (3, 2, 2 * 9000, 2),
    (8, 3, 2 * 60000, 3),
    (64, 63, 2 * 400000, 4),
    (1024, 517, 2 * 2_000_000, 5),
]


def layout_numels(rng, nd):
    """Large parameters (whole tiles: the uniform path of the pack), a ragged middle (tiles
    with a few parameters: the staged path) and a run of 400 parameters of at most 5 columns
    (more than 256 parameters in one tile: the generic path)."""
    big = [nd * 2048 * 3 + 5, nd * 2048 + nd * 3]
    mid = ragged_numels(rng, 60, nd, 30000)
    tiny = [int(x) for x in rng.integers(1, 5 * nd + 1, size=400)]
    return big[:1] + mid[:30] + tiny + mid[30:] + big[1:]


def finite_bits(rng, n, dtype):
    """Random finite 16-bit patterns of magnitude below 2 (bf16) or 1 (fp16)."""
    return random_bits(rng, n) & np.uint16(0xBFFF if dtype == BF16 else 0xBBFF)


def largest_allowed(nd):
    """The largest positive bf16 pattern with |x| * nd <= 2^126 (exact arithmetic)."""
    lim = Fraction(2) ** 126
    best = 0
    for b in range(0x7F80):
        x = Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))
        if x * nd <= lim:
            best = b
    return best


# ------------------------------------------------------------------- checked pack ------

@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_checked_pack(case, dtype):
    nd, rank, cap, seed = case
    rng = np.random.default_rng(seed + 300)
    numels = layout_numels(rng, nd)
    say(f"checked pack nd={nd} rank={rank} dtype={dtype} n={len(numels)}")
    st = Z.ShardStep(numels, nd, rank, cap, dtype)
    pl = oracle.plan(numels, nd, rank, cap)
    grads = [finite_bits(rng, x, dtype) for x in numels]
    dead = rng.random(len(numels)) < 0.2
    dev = [to_dev16(g) for g in grads]
    ptrs = Z.ptr_table([None if d else t for d, t in zip(dead, dev)])
    host = [None if d else g for d, g in zip(dead, grads)]
    # clean inputs: same bits as the unchecked pack, flag clear
    for b in range(pl.n_buckets):
        st.flag.zero_()
        blk = st.block(st.packed, b)
        blk.fill_(0x5A5A)
        Z.zero_pack_bucket_check(st.plan, b, ptrs, blk, st.flag)
        want = oracle.pack_bucket(pl, b, host)
        got = to_np16(blk).reshape(want.shape)
        for i in pl.bucket_params(b):
            if host[i] is not None:
                c, s_ = pl.params[i, oracle.P_COL], pl.params[i, P_S]
                assert np.array_equal(got[:, c:c + s_], want[:, c:c + s_]), (b, i)
        assert np.array_equal(got[:, pl.buckets[b, oracle.B_ROW]:], want[:, pl.buckets[b, oracle.B_ROW]:])
        assert int(st.flag.item()) == oracle.input_check(pl, b, host, dtype) == 0
    # injections: one value per trial into a live (or, for some trials, a dead) parameter
    top = largest_allowed(nd)
    specials = ([0x7F80, 0xFF80, 0x7FC0, top + 1, top, top | 0x8000, (top + 1) | 0x8000] if dtype == BF16 else
                [0x7C00, 0xFC00, 0x7E01, 0x7BFF, 0xFBFF])
    nonempty = [i for i in range(len(numels)) if numels[i] > 0]
    groups = {"big": [0, len(numels) - 1], "tiny": list(range(31, 431)), "mid": nonempty}
    trials = 0
    for gname, pool in groups.items():
        pool = [i for i in pool if numels[i] > 0]
        for _ in range(6):
            i = int(rng.choice(pool))
            e = int(rng.integers(0, numels[i]))
            val = int(rng.choice(specials))
            old = grads[i][e]
            grads[i][e] = val
            dev[i][e] = int(np.uint16(val).view(np.int16))
            b = int(pl.params[i, oracle.P_BUCKET])
            st.flag.zero_()
            Z.zero_pack_bucket_check(st.plan, b, ptrs, st.block(st.packed, b), st.flag)
            want_flag = oracle.input_check(pl, b, host, dtype)
            assert int(st.flag.item()) == want_flag, (gname, i, e, hex(val), dead[i])
            if dead[i]:
                assert want_flag == 0
            want = oracle.pack_bucket(pl, b, host)
            got = to_np16(st.block(st.packed, b)).reshape(want.shape)
            if not dead[i]:
                c, s_ = pl.params[i, oracle.P_COL], pl.params[i, P_S]
                assert np.array_equal(got[:, c:c + s_], want[:, c:c + s_])
            grads[i][e] = old
            dev[i][e] = int(np.uint16(old).view(np.int16))
            trials += 1
    assert trials == 18


@pytest.mark.parametrize("case", [CASES[2], CASES[3]])
def test_checked_pack_misaligned_gradients(case):
    """Gradients at odd 2-byte offsets (realigned loads, staged and element paths): the same
    bits as the oracle's pack and the same verdict, clean and with one injection per trial."""
    nd, rank, cap, seed = case
    rng = np.random.default_rng(seed + 500)
    numels = layout_numels(rng, nd)
    st = Z.ShardStep(numels, nd, rank, cap, BF16)
    pl = oracle.plan(numels, nd, rank, cap)
    grads = [finite_bits(rng, x, BF16) for x in numels]
    buf, views = placed_views(grads, rng, misalign=True)
    ptrs = Z.ptr_table(views)
    for trial in range(4):
        inj = None
        if trial:
            i = int(rng.choice([j for j in range(len(numels)) if numels[j] > 0]))
            e = int(rng.integers(0, numels[i]))
            inj = (i, e, grads[i][e])
            grads[i][e] = 0x7FC0
            views[i][e] = int(np.uint16(0x7FC0).view(np.int16))
        for b in range(pl.n_buckets):
            st.flag.zero_()
            Z.zero_pack_bucket_check(st.plan, b, ptrs, st.block(st.packed, b), st.flag)
            want = oracle.pack_bucket(pl, b, grads)
            got = to_np16(st.block(st.packed, b)).reshape(want.shape)
            assert np.array_equal(got, want), (trial, b)
            assert int(st.flag.item()) == oracle.input_check(pl, b, grads, BF16), (trial, b)
        if inj:
            i, e, old = inj
            grads[i][e] = old
            views[i][e] = int(np.uint16(old).view(np.int16))
    del buf


def test_checked_pack_bound_at_nd8():
    """2^123 = 2^126 / 8 passes, the next bf16 value flags: the kernel's bound is the oracle's."""
    st = Z.ShardStep([4096 * 8, 37], 8, 1, 0, BF16)
    for val, want in ((0x7D00, 0), (0xFD00, 0), (0x7D01, 1), (0xFD01, 1), (0x7F7F, 1)):
        g = torch.full((4096 * 8,), 0x3F80, dtype=torch.int16, device=DEV)
        g[4096 + 17] = int(np.uint16(val).view(np.int16))
        g2 = torch.full((37,), 0x3F80, dtype=torch.int16, device=DEV)
        st.flag.zero_()
        Z.zero_pack_bucket_check(st.plan, 0, Z.ptr_table([g, g2]), st.block(st.packed, 0), st.flag)
        assert int(st.flag.item()) == want, hex(val)
        g2[36] = int(np.uint16(val).view(np.int16))
        g[4096 + 17] = 0x3F80
        st.flag.zero_()
        Z.zero_pack_bucket_check(st.plan, 0, Z.ptr_table([g, g2]), st.block(st.packed, 0), st.flag)
        assert int(st.flag.item()) == want, hex(val)


# --------------------------------------------------------------- fused reduce + Adam --

def rows_for(rng, pl, b, own_row, dtype, extra):
    """A bucket's Nd rows (row_stride L_b + extra): this rank's own packed row and finite
    random rows for the others."""
    L = int(pl.buckets[b, oracle.B_STRIDE])
    rows = finite_bits(rng, pl.nd * (L + extra), dtype).reshape(pl.nd, L + extra)
    rows[pl.rank, :L] = own_row
    return rows


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_fused_matches_unfused_and_oracle(case, dtype):
    nd, rank, cap, seed = case
    rng = np.random.default_rng(seed + 400)
    numels = layout_numels(rng, nd)
    say(f"fused nd={nd} rank={rank} dtype={dtype} n={len(numels)}")
    A = Z.ShardStep(numels, nd, rank, cap, dtype)   # unfused
    F = Z.ShardStep(numels, nd, rank, cap, dtype)   # fused
    pl = oracle.plan(numels, nd, rank, cap)
    S = pl.shard_len
    p32 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    steps = rng.integers(0, 3, size=len(numels)).astype(np.int32)
    arena = random_bits(rng, nd * S) & np.uint16(0xBFFF)
    for X in (A, F):
        X.p32.copy_(torch.from_numpy(p32))
        X.steps.copy_(torch.from_numpy(steps))
        X.arena.copy_(to_dev16(arena))
        X.g32.fill_(float("nan"))
    hp = oracle.AdamHP(**HP)
    ever = np.zeros(S, dtype=bool)  # columns of parameters that have taken a step
    for step in range(4):
        live = (rng.random(len(numels)) > 0.25).astype(np.uint8)
        inject = step == 2  # an inf in this rank's own gradient: both paths must skip the step
        grads = [finite_bits(rng, x, dtype) if l else None for x, l in zip(numels, live)]
        if inject:
            # into this rank's own slice (row r), which this rank's unfused reduce sees too; in a
            # real job the rank owning another slice would flag it and the flags are ORed
            s_ = pl.params[:, P_S]
            own = [j for j in range(len(numels)) if live[j] and numels[j] > rank * s_[j]]
            i = int(rng.choice(own))
            e = rank * int(s_[i]) + int(rng.integers(0, min(int(s_[i]), numels[i] - rank * int(s_[i]))))
            grads[i][e] = 0x7F80 if dtype == BF16 else 0x7C00
        ptrs = Z.ptr_table([None if g is None else to_dev16(g) for g in grads])
        for X in (A, F):
            X.live.copy_(torch.from_numpy(live))
            X.flag.zero_()
        A.pack(ptrs)
        F.pack(ptrs, check=True)
        assert torch.equal(A.packed, F.packed)
        assert int(F.flag.item()) == max(oracle.input_check(pl, b, grads, dtype) for b in range(pl.n_buckets)) \
            == int(inject)
        rows = []
        g32 = np.zeros(S, np.float32)
        for b in range(pl.n_buckets):
            extra = 8 * int(rng.integers(0, 3))
            rows.append(rows_for(rng, pl, b, oracle.pack_bucket(pl, b, grads)[rank], dtype, extra))
            oracle.reduce_bucket(pl, b, rows[b], dtype, live, g32)
        rdev = [to_dev16(r_.reshape(-1)) if r_.size else torch.zeros(8, dtype=torch.int16, device=DEV) for r_ in rows]
        A.reduce(lambda b: (rdev[b], rows[b].shape[1]))
        A.adam(**HP)
        F.reduce_adam(lambda b: (rdev[b], rows[b].shape[1]), **HP)
        flag = oracle.overflow(pl, g32, live)
        assert int(A.flag.item()) == flag == int(inject)
        oracle.adam(pl, g32, p32, m, v, live, steps, hp, flag, arena, dtype)
        torch.cuda.synchronize()
        for name, ta, tf in (("p32", A.p32, F.p32), ("m", A.m, F.m), ("v", A.v, F.v)):
            assert torch.equal(ta.view(torch.int32), tf.view(torch.int32)), f"{name} step {step}"
        assert torch.equal(A.arena, F.arena) and torch.equal(A.steps, F.steps), step
        assert bool(torch.isnan(F.g32).all())  # the fused path never writes the fp32 gradient
        assert np.array_equal(to_np32(F.steps), steps)
        assert_close_f32(to_np32(F.p32), p32, f"p32 step {step}")
        assert_close_f32(to_np32(F.m), m, f"m step {step}")
        assert_close_f32(to_np32(F.v), v, f"v step {step}", abs_=V_ABS, rel=2e-6)
        if not flag:
            for i in np.flatnonzero(live):
                ever[pl.params[i, P_OFF]:pl.params[i, P_OFF] + pl.params[i, P_S]] = True
        got_arena = to_np16(F.arena)
        check_arena(pl, got_arena, arena, to_np32(F.p32), p32, ever, dtype, f"arena {step}")


def test_fused_without_flag_steps_regardless():
    """d_flag = NULL: the step is taken even when the pack's verdict is set, as with
    zero_adam_step and a NULL flag."""
    rng = np.random.default_rng(21)
    numels = layout_numels(rng, 8)
    A = Z.ShardStep(numels, 8, 5, 2 * 50000, BF16)
    F = Z.ShardStep(numels, 8, 5, 2 * 50000, BF16)
    pl = oracle.plan(numels, 8, 5, 2 * 50000)
    rows = [finite_bits(rng, 8 * int(pl.buckets[b, oracle.B_STRIDE]), BF16) for b in range(pl.n_buckets)]
    rdev = [to_dev16(r_) for r_ in rows]
    for X in (A, F):
        X.p32.copy_(torch.linspace(-1, 1, X.p32.numel(), device=DEV))
        X.flag.fill_(1)
    A.reduce(lambda b: (rdev[b], int(pl.buckets[b, oracle.B_STRIDE])), fused_check=False)
    A.adam(**HP, use_flag=False)
    F.reduce_adam(lambda b: (rdev[b], int(pl.buckets[b, oracle.B_STRIDE])), **HP, use_flag=False)
    for ta, tf in ((A.p32, F.p32), (A.m, F.m), (A.v, F.v)):
        assert torch.equal(ta.view(torch.int32), tf.view(torch.int32))
    assert torch.equal(A.arena, F.arena) and torch.equal(A.steps, F.steps)
    assert int(F.steps.min().item()) == 1


def test_fused_skips_on_set_flag():
    rng = np.random.default_rng(22)
    numels = layout_numels(rng, 8)
    F = Z.ShardStep(numels, 8, 0, 0, FP16)
    F.p32.normal_()
    F.m.normal_()
    F.v.uniform_()
    F.arena.random_(-30000, 30000)
    before = [t.clone() for t in (F.p32, F.m, F.v, F.arena, F.steps)]
    rows = torch.zeros(8 * int(F.buckets[0].row_stride), dtype=torch.int16, device=DEV)
    F.flag.fill_(1)
    F.reduce_adam(lambda b: (rows, int(F.buckets[0].row_stride)), **HP)
    torch.cuda.synchronize()
    for a, t in zip(before, (F.p32, F.m, F.v, F.arena, F.steps)):
        assert torch.equal(a, t)


def _status(call):
    try:
        call()
    except Z.ZeroError as e:
        return e.status
    return Z.ZERO_OK


def test_fused_calls_reject_bad_arguments():
    st = Z.ShardStep([1000, 37, 5000], 8, 3, 0, BF16)
    L = int(st.buckets[0].row_stride)
    buf = torch.zeros(8 * L + 64, dtype=torch.int16, device=DEV)
    ptrs = Z.ptr_table([torch.zeros(x, dtype=torch.int16, device=DEV) for x in (1000, 37, 5000)])
    f = torch.zeros(int(st.summary.shard_numel) + 8, dtype=torch.float32, device=DEV)
    E = Z.ZERO_EINVAL
    assert _status(lambda: Z.zero_pack_bucket_check(st.plan, 1, ptrs, buf, st.flag)) == E
    assert _status(lambda: Z.zero_pack_bucket_check(st.plan, 0, ptrs, buf[1:], st.flag)) == E
    assert _status(lambda: Z.zero_pack_bucket_check(st.plan, 0, ptrs, buf, None)) == E
    assert _status(lambda: Z.zero_adam_prepare(st.plan, st.live, st.steps, **dict(HP, beta1=1.0), flag=None)) == E
    assert _status(lambda: Z.zero_adam_prepare(st.plan, st.live, st.steps, **dict(HP, lr=float("nan")),
                                               flag=None)) == E
    ra = Z.zero_reduce_adam_bucket
    assert _status(lambda: ra(st.plan, 1, buf, L, st.live, f, f, f, None, st.arena)) == E        # bucket
    assert _status(lambda: ra(st.plan, 0, buf, L - 8, st.live, f, f, f, None, st.arena)) == E    # stride < L_b
    assert _status(lambda: ra(st.plan, 0, buf, L + 4, st.live, f, f, f, None, st.arena)) == E    # stride % 8
    assert _status(lambda: ra(st.plan, 0, buf[1:], L, st.live, f, f, f, None, st.arena)) == E    # rows
    assert _status(lambda: ra(st.plan, 0, buf, L, st.live, f[1:], f, f, None, st.arena)) == E    # p32
    big = torch.zeros(int(st.summary.arena_numel) + 64, dtype=torch.int16, device=DEV)
    assert _status(lambda: ra(st.plan, 0, buf, L, st.live, f, f, f, None, big[3:])) == E         # arena
    assert _status(lambda: ra(st.plan, 0, buf, L, None, f, f, f, None, st.arena)) == E           # live
    # buffers too small for what the kernels would touch are refused before any launch
    with pytest.raises(ValueError, match="arena"):
        ra(st.plan, 0, buf, L, st.live, f, f, f, None, st.arena[8:])
    with pytest.raises(ValueError, match="rows"):
        ra(st.plan, 0, buf[:7 * L + L - 8], L, st.live, f, f, f, None, st.arena)
    with pytest.raises(ValueError, match="entry 1"):
        Z.zero_pack_bucket_check(st.plan, 0, Z.ptr_table([ptrs.zero_targets[0], buf[:36], ptrs.zero_targets[2]]),
                                 buf, st.flag)
    with pytest.raises(ValueError, match="ptr_table"):
        Z.zero_pack_bucket_check(st.plan, 0, ptrs.clone(), buf, st.flag)
    torch.cuda.synchronize()
    assert int(st.steps.sum().item()) == 0 and int(st.flag.item()) == 0


# ------------------------------------------------------------------- full-size lists --

def run_fused_fullsize(config, n_steps=2, n_samples=8000):
    """Both paths on one workload at its real size: this rank's gradients packed with the
    check, the other ranks' rows from the row generator; the unfused path is the reference bit
    for bit, and sampled columns are checked against the oracle."""
    w = W.workload(config)
    nd, r = w.nd, w.rank
    rng = np.random.default_rng(2000 + config)
    say(f"[fused config {config}] {w.name}: n={w.n} nd={nd} rank={r}")
    pl = oracle.plan(w.numels, nd, r, w.bucket_bytes)
    A = Z.ShardStep(w.numels, nd, r, w.bucket_bytes, w.dtype)
    F = Z.ShardStep(w.numels, nd, r, w.bucket_bytes, w.dtype)
    hp = oracle.AdamHP(lr=w.lr, beta1=w.betas[0], beta2=w.betas[1], eps=w.eps, grad_scale=w.grad_scale)
    masters = W.masters(w, DEV)
    A.init_master(Z.ptr_table(masters), 0)
    F.p32.copy_(A.p32)
    cols = sample_columns(pl, rng, n_samples)
    ci, cj = column_owner(pl, cols)
    ce = r * pl.params[ci, P_S] + cj
    cols_dev = torch.from_numpy(cols).to(DEV)
    o_p32 = gather_params(masters, ci, ce, 0.0).numpy().astype(np.float32)
    o_p32[ce >= pl.params[ci, P_NUMEL]] = 0.0
    del masters
    o_m = np.zeros_like(o_p32)
    o_v = np.zeros_like(o_p32)
    o_t = np.zeros(pl.n, np.int64)
    for step in range(n_steps):
        live = W.live_mask(w, step)
        say(f"[fused config {config}] step {step}: live {int(live.sum())}/{w.n}")
        own = [t if l else None for t, l in zip(W.grads(w, step, r, DEV), live)]
        ptrs = Z.ptr_table(own)
        for X in (A, F):
            X.live.copy_(torch.from_numpy(live))
            X.flag.zero_()
        A.pack(ptrs)
        F.pack(ptrs, check=True)
        assert torch.equal(A.packed, F.packed)
        own_flag = int(F.flag.item())
        assert own_flag == 0  # the generated gradients are finite and far below the bound
        recv = []
        for b in range(pl.n_buckets):
            L = int(pl.buckets[b, oracle.B_STRIDE])
            blk = W.remote_rows(w, step, b, L, DEV).view(torch.int16)
            zero = torch.from_numpy(row_zero_mask(pl, b, live)).to(DEV)
            blk.masked_fill_(zero.unsqueeze(0), 0)
            blk[r].copy_(A.own_row(A.packed, b))
            recv.append(blk)
        # another rank's gradient overflowed on odd steps of the lists that inject: its own
        # check set its flag, and the all-reduce of the flags brings it here
        pos, _ = W.injections(w, step, 1)
        if pos.size:
            F.flag.fill_(1)
            A.flag.fill_(1)
        rows_of = lambda b: (recv[b].view(-1), int(pl.buckets[b, oracle.B_STRIDE]))
        A.reduce(rows_of)
        A.adam(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
        F.reduce_adam(rows_of, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
        torch.cuda.synchronize()
        for name, ta, tf in (("p32", A.p32, F.p32), ("m", A.m, F.m), ("v", A.v, F.v)):
            assert torch.equal(ta.view(torch.int32), tf.view(torch.int32)), f"{name} step {step}"
        assert torch.equal(A.arena, F.arena) and torch.equal(A.steps, F.steps), step
        # oracle on the sampled columns
        flag = int(F.flag.item())
        if not flag:
            cb = pl.params[ci, oracle.P_BUCKET]
            cc = pl.params[ci, oracle.P_COL] + cj
            rows = np.zeros((nd, cols.size), np.uint16)
            for b in np.unique(cb):
                sel = np.flatnonzero(cb == b)
                rows[:, sel] = bits16(recv[b][:, torch.from_numpy(cc[sel]).to(DEV)].cpu())
            # this rank's row at the sampled columns comes from its own gradients, not the GPU
            real = (ce < pl.params[ci, P_NUMEL]) & (live[ci] == 1)
            rows[r] = np.where(real, bits16(gather_params(own, ci, ce, 0)), 0)
            o_t[live == 1] += 1
            for s_i in np.flatnonzero(live[ci] == 1):
                g = oracle.reduce_column(rows[:, s_i], w.dtype)
                o_p32[s_i], o_m[s_i], o_v[s_i] = oracle.adam_element(g, o_p32[s_i], o_m[s_i], o_v[s_i],
                                                                     int(o_t[ci[s_i]]), hp)
        assert np.array_equal(to_np32(F.steps).astype(np.int64), o_t), f"steps {step}"
        assert_close_f32(to_np32(F.p32[cols_dev]), o_p32, f"p32 step {step}")
        assert_close_f32(to_np32(F.m[cols_dev]), o_m, f"m step {step}")
        assert_close_f32(to_np32(F.v[cols_dev]), o_v, f"v step {step}", rel=2e-6, abs_=0.0)
        del own, ptrs, recv
    say(f"[fused config {config}] ok")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_fused_fullsize_workload(config):
    try:
        run_fused_fullsize(config)
    finally:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
