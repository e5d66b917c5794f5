"""The five workloads on the GPU, through the C ABI, against the oracle.

MlpModel (small): every stage, every element, over its 3 steps.  The four large lists run at
their real sizes, in the launch configuration bench.py times (one block per tile, every bucket),
and are checked on sampled outputs the oracle computes one by one: the plan tables in full;
p32 init, pack, reduce, overflow flag, Adam state and 16-bit parameters, unpack at sampled
positions (with every parameter's first and last slice column, row boundaries and injected
positions among them).  The oracle's inputs always come from the seeded generators, never from
a GPU output: a sampled column's rows are gathered from the source gradients, and the oracle
carries the sampled columns' Adam state from step to step itself."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import zero_sharded_mixed_amd as Z
from gpu_harness import (DEV, assert_close_f32, assert_lp_within_ulp, assert_same_f32, bits16, check_arena,
                         column_owner, gather_params, oracle_block, row_zero_mask, sample_columns, say, to_np16,
                         to_np32)

pytestmark = pytest.mark.gpu
P_OFF, P_S, P_NUMEL, P_COL, P_BUCKET, P_START = (oracle.P_OFFSET, oracle.P_SHARD, oracle.P_NUMEL, oracle.P_COL,
                                                 oracle.P_BUCKET, oracle.P_START)


def tdtype(w):
    return torch.bfloat16 if w.dtype == W.BF16 else torch.float16


def check_plan(st, pl):
    s = st.summary
    assert (s.n_buckets, s.shard_numel) == (pl.n_buckets, pl.shard_len)
    for i in range(pl.n):
        info = Z.zero_plan_param_info(st.plan, i)
        assert [info.numel, info.pad, info.padded_numel, info.shard_size, info.shard_start, info.shard_end,
                info.shard_offset, info.bucket, info.bucket_col] == list(pl.params[i]), i
    for b in range(pl.n_buckets):
        bk = Z.zero_plan_bucket_info(st.plan, b)
        assert [bk.first_param, bk.n_params, bk.row_elems, bk.row_stride, bk.shard_base] == list(pl.buckets[b])


# ------------------------------------------------------------------------- MlpModel ----

def test_mlp_model_every_element_three_steps():
    w = W.workload(1)
    nd, r = w.nd, w.rank
    st = Z.ShardStep(w.numels, nd, r, w.bucket_bytes, w.dtype)
    pl = oracle.plan(w.numels, nd, r, w.bucket_bytes)
    check_plan(st, pl)
    masters = W.masters(w, "cpu")
    st.init_master(Z.ptr_table([m.to(DEV) for m in masters]), 0)
    p32 = np.zeros(pl.shard_len, np.float32)
    oracle.shard_init(pl, [m.numpy() for m in masters], p32)
    assert_same_f32(to_np32(st.p32), p32, "p32 init")
    lp = [m.to(torch.bfloat16) for m in masters]
    lp_dev = [t.to(DEV) for t in lp]
    lp_ptrs = Z.ptr_table(lp_dev)
    st.pack(lp_ptrs, out=st.arena)
    arena = np.zeros(nd * pl.shard_len, np.uint16)
    for b in range(pl.n_buckets):
        oracle_block(pl, arena, b)[:] = oracle.pack_bucket(pl, b, [to_np16(t) for t in lp])
    assert np.array_equal(to_np16(st.arena), arena)
    m = np.zeros_like(p32)
    v = np.zeros_like(p32)
    steps = np.zeros(pl.n, np.int32)
    hp = oracle.AdamHP(lr=w.lr, beta1=w.betas[0], beta2=w.betas[1], eps=w.eps, grad_scale=w.grad_scale)
    ever = np.zeros(pl.shard_len, dtype=bool)  # columns of parameters that have taken a step
    packed_all = torch.zeros((nd, int(st.summary.arena_numel)), dtype=torch.int16, device=DEV)
    flat = packed_all.view(-1)
    for step in range(w.steps):
        live = W.live_mask(w, step)
        assert live[2] == 0 and live[3] == 0  # drop_linear never has a gradient
        st.live.copy_(torch.from_numpy(live))
        rows = [np.zeros((nd, pl.buckets[b, oracle.B_STRIDE]), np.uint16) for b in range(pl.n_buckets)]
        for k in range(nd):
            g = [t if l else None for t, l in zip(W.grads(w, step, k, "cpu"), live)]
            st.pack(Z.ptr_table([None if t is None else t.to(DEV) for t in g]), out=packed_all[k])
            for b in range(pl.n_buckets):
                want = oracle.pack_bucket(pl, b, [None if t is None else to_np16(t) for t in g])
                got = oracle_block(pl, to_np16(packed_all[k]), b)
                for i in pl.bucket_params(b):
                    if live[i]:
                        c, s_ = pl.params[i, P_COL], pl.params[i, P_S]
                        assert np.array_equal(got[:, c:c + s_], want[:, c:c + s_]), (step, k, i)
                rows[b][k] = want[r]
        st.flag.zero_()
        stride = int(st.summary.arena_numel)
        st.reduce(lambda b: (flat[st.buckets[b].block_offset + r * st.buckets[b].row_stride:], stride))
        g32 = np.zeros(pl.shard_len, np.float32)
        for b in range(pl.n_buckets):
            oracle.reduce_bucket(pl, b, rows[b], w.dtype, live, g32)
        got_g = to_np32(st.g32)
        for i in np.flatnonzero(live):
            o, s_ = pl.params[i, P_OFF], pl.params[i, P_S]
            assert_same_f32(got_g[o:o + s_], g32[o:o + s_], f"g32 step {step} param {i}")
        flag = oracle.overflow(pl, g32, live)
        assert int(st.flag.item()) == flag == 0
        before = [to_np32(t) for t in (st.p32, st.m, st.v)]
        st.adam(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
        oracle.adam(pl, g32, p32, m, v, live, steps, hp, flag, arena, w.dtype)
        assert np.array_equal(to_np32(st.steps), steps)
        assert_close_f32(to_np32(st.p32), p32, f"p32 step {step}")
        assert_close_f32(to_np32(st.m), m, f"m step {step}")
        assert_close_f32(to_np32(st.v), v, f"v step {step}")
        for i in np.flatnonzero(live):
            ever[pl.params[i, P_OFF]:pl.params[i, P_OFF] + pl.params[i, P_S]] = True
        check_arena(pl, to_np16(st.arena), arena, to_np32(st.p32), p32, ever, w.dtype, f"arena {step}")
        for i in (2, 3):  # the dropped layer: p32 / m / v bit-identical
            o, s_ = pl.params[i, P_OFF], pl.params[i, P_S]
            for old, t in zip(before, (st.p32, st.m, st.v)):
                assert np.array_equal(old[o:o + s_].view(np.uint32), to_np32(t)[o:o + s_].view(np.uint32))
        st.unpack(lp_ptrs)
        outs = [np.zeros(int(x), np.uint16) for x in w.numels]
        got_arena = to_np16(st.arena)
        for b in range(pl.n_buckets):
            oracle.unpack_bucket(pl, b, oracle_block(pl, got_arena, b).copy(), outs)
        for i, t in enumerate(lp_dev):
            assert np.array_equal(to_np16(t), outs[i]), (step, i)


# ----------------------------------------------------------------- full-size workloads --

def run_fullsize(config, max_steps=None, n_samples=20000):
    w = W.workload(config)
    nd, r = w.nd, w.rank
    steps_to_run = w.steps if max_steps is None else min(w.steps, max_steps)
    rng = np.random.default_rng(1000 + config)
    say(f"[config {config}] {w.name}: n={w.n} nd={nd} rank={r}")
    pl = oracle.plan(w.numels, nd, r, w.bucket_bytes)
    st = Z.ShardStep(w.numels, nd, r, w.bucket_bytes, w.dtype)
    check_plan(st, pl)
    tdt = tdtype(w)
    hp = oracle.AdamHP(lr=w.lr, beta1=w.betas[0], beta2=w.betas[1], eps=w.eps, grad_scale=w.grad_scale)

    cols = sample_columns(pl, rng, n_samples)
    ci, cj = column_owner(pl, cols)
    ce = r * pl.params[ci, P_S] + cj                     # element of the padded parameter
    cb = pl.params[ci, P_BUCKET]
    cc = pl.params[ci, P_COL] + cj                       # column inside the bucket row

    # p32 init: row r of the zero-padded fp32 master
    masters = W.masters(w, DEV)
    st.init_master(Z.ptr_table(masters), 0)
    o_p32 = gather_params(masters, ci, ce, 0.0).numpy().astype(np.float32)
    o_p32[ce >= pl.params[ci, P_NUMEL]] = 0.0
    assert_same_f32(to_np32(st.p32[torch.from_numpy(cols).to(DEV)]), o_p32, "p32 init")
    lp = [m.to(tdt) for m in masters]
    del masters
    lp_ptrs = Z.ptr_table(lp)
    o_lp_before = bits16(gather_params(lp, ci, ce, 0))   # published parameters at the sampled positions
    st.pack(lp_ptrs, out=st.arena)                       # every rank holds the full model
    o_m = np.zeros_like(o_p32)
    o_v = np.zeros_like(o_p32)
    o_t = np.zeros(pl.n, np.int64)
    cols_dev = torch.from_numpy(cols).to(DEV)
    arena_rowr = torch.from_numpy(nd * pl.buckets[cb, oracle.B_BASE] + r * pl.buckets[cb, oracle.B_STRIDE] + cc).to(DEV)
    packed_all = None
    if w.emulation == "full":
        packed_all = torch.zeros((nd, int(st.summary.arena_numel)), dtype=torch.int16, device=DEV)

    for step in range(steps_to_run):
        live = W.live_mask(w, step)
        st.live.copy_(torch.from_numpy(live))
        say(f"[config {config}] step {step}: live {int(live.sum())}/{w.n}")
        # rows[k][s] = virtual rank k's row-r value at sampled column s (from the source gradients)
        rows = np.zeros((nd, cols.size), np.uint16)
        real = (ce < pl.params[ci, P_NUMEL]) & (live[ci] == 1)
        own = None
        for k in (range(nd) if w.emulation == "full" else [r]):
            g = [t if l else None for t, l in zip(W.grads(w, step, k, DEV), live)]
            vals = bits16(gather_params(g, ci, ce, 0))
            rows[k] = np.where(real, vals, 0)
            if w.emulation == "full":
                st.pack(Z.ptr_table(g), out=packed_all[k])
            if k == r:
                own = g
            else:
                del g
        # the pack of this rank's own gradients, checked at sampled (bucket, row, column)
        st.packed.fill_(0x5A5A)
        own_ptrs = Z.ptr_table(own)
        st.pack(own_ptrs)
        pb = rng.integers(0, pl.n_buckets, size=4000)
        pk = rng.integers(0, nd, size=4000)
        pc = np.array([rng.integers(0, pl.buckets[b, oracle.B_STRIDE]) if pl.buckets[b, oracle.B_STRIDE] else 0
                       for b in pb])
        loc = [oracle.pack_locate(pl, int(b), int(k), int(c)) for b, k, c in zip(pb, pk, pc)]
        kind = np.array([x[0] for x in loc])
        li, le = np.array([x[1] for x in loc]), np.array([x[2] for x in loc])
        src = bits16(gather_params(own, np.where(kind == 1, li, 0), np.where(kind == 1, le, 0), 0))
        expect = np.where(kind == 1, src, 0).astype(np.uint16)
        dead = (kind != 0) & (live[np.where(kind != 0, li, 0)] == 0)
        flat_idx = nd * pl.buckets[pb, oracle.B_BASE] + pk * pl.buckets[pb, oracle.B_STRIDE] + pc
        got = bits16(st.packed[torch.from_numpy(flat_idx).to(DEV)].cpu())
        assert np.array_equal(got[~dead], expect[~dead]), f"pack step {step}"
        assert np.all(got[dead] == 0x5A5A), f"pack wrote a dead slot, step {step}"

        # the other ranks' rows r
        injected = np.zeros(cols.size, dtype=bool)
        if w.emulation == "full":
            flat = packed_all.view(-1)
            stride = int(st.summary.arena_numel)
            rows_of = lambda b: (flat[st.buckets[b].block_offset + r * st.buckets[b].row_stride:], stride)
        else:
            recv = []
            for b in range(pl.n_buckets):
                L = int(pl.buckets[b, oracle.B_STRIDE])
                blk = W.remote_rows(w, step, b, L, DEV).view(torch.int16)
                zero = torch.from_numpy(row_zero_mask(pl, b, live)).to(DEV)
                blk.masked_fill_(zero.unsqueeze(0), 0)
                blk[r].copy_(st.own_row(st.packed, b))
                recv.append(blk)
            # inf / NaN injections on odd steps at live positions of other ranks' rows; some
            # land on sampled columns so that the oracle sees them
            pos, vals = W.injections(w, step, int(real.sum()) * (nd - 1))
            if pos.size:
                live_cols = np.flatnonzero(real)
                kk = pos // live_cols.size
                sc_idx = live_cols[pos % live_cols.size]
                kk = np.where(kk < r, kk, kk + 1)
                vb = bits16(vals)
                for k, s_i, val in zip(kk, sc_idx, vb):
                    recv[cb[s_i]][k, cc[s_i]] = int(np.int16(np.uint16(val).view(np.int16)))
                    injected[s_i] = True
            for b in range(pl.n_buckets):  # sampled columns of the generated rows
                sel = np.flatnonzero(cb == b)
                if sel.size:
                    vals_b = bits16(recv[b][:, torch.from_numpy(cc[sel]).to(DEV)].cpu())
                    for k in range(nd):
                        if k != r:
                            rows[k, sel] = vals_b[k]
            rows_of = lambda b: (recv[b].view(-1), int(pl.buckets[b, oracle.B_STRIDE]))

        st.flag.zero_()
        st.reduce(rows_of)
        o_g = np.array([oracle.reduce_column(rows[:, s_i], w.dtype) for s_i in range(cols.size)], np.float32)
        got_g = to_np32(st.g32[cols_dev])
        lv = live[ci] == 1
        assert_same_f32(got_g[lv], o_g[lv], f"g32 step {step}")
        flag = int(st.flag.item())
        # the flag: any non-finite live value of the full shard (a property at any size), and
        # what the recipe fixes (injections -> set; none of these lists overflows on its own)
        live_cols_all = torch.zeros(pl.shard_len, dtype=torch.bool, device=DEV)
        for i in np.flatnonzero(live):
            live_cols_all[pl.params[i, P_OFF]:pl.params[i, P_OFF] + pl.params[i, P_S]] = True
        any_bad = bool((~torch.isfinite(st.g32) & live_cols_all).any().item())
        assert flag == int(any_bad), f"flag step {step}"
        assert flag == int(bool(injected.any())), f"flag recipe step {step}"
        if injected.any():
            assert np.all(~np.isfinite(got_g[injected]))

        # Adam, with the oracle carrying the sampled columns' state
        st.adam(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale)
        if not flag:
            o_t[live == 1] += 1
            for s_i in np.flatnonzero(lv):
                o_p32[s_i], o_m[s_i], o_v[s_i] = oracle.adam_element(o_g[s_i], o_p32[s_i], o_m[s_i], o_v[s_i],
                                                                     int(o_t[ci[s_i]]), hp)
        assert np.array_equal(to_np32(st.steps).astype(np.int64), o_t), f"steps {step}"
        assert_close_f32(to_np32(st.p32[cols_dev]), o_p32, f"p32 step {step}")
        assert_close_f32(to_np32(st.m[cols_dev]), o_m, f"m step {step}")
        assert_close_f32(to_np32(st.v[cols_dev]), o_v, f"v step {step}")
        assert_close_f32(to_np32(st.v[cols_dev]), o_v, f"v step {step} (relative)", rel=2e-6, abs_=0.0)
        got_lp = bits16(st.arena[arena_rowr].cpu())
        ever_live = o_t[ci] > 0
        # the 16-bit parameter is the RNE of the kernel's own p32 (checked against the oracle above)
        got_p = to_np32(st.p32[cols_dev])
        assert np.array_equal(got_lp[ever_live], oracle.from_f32(got_p[ever_live], w.dtype)), f"lp step {step}"
        assert_lp_within_ulp(got_lp[ever_live], oracle.from_f32(o_p32[ever_live], w.dtype), o_p32[ever_live], w.dtype,
                             f"lp step {step}")
        assert np.array_equal(got_lp[~ever_live], o_lp_before[~ever_live]), f"untouched lp step {step}"
        del own, own_ptrs
        if w.emulation != "full":
            del recv

    # unpack at full size, from a gathered arena of random bits
    gen = torch.Generator(device=DEV)
    gen.manual_seed(W.seed_of(config, 99, 0, W.SLOT_ROWS))
    gathered = torch.randint(-32768, 32767, (int(st.summary.arena_numel),), generator=gen, dtype=torch.int16,
                             device=DEV)
    st.unpack(lp_ptrs, src=gathered)
    ui = rng.integers(0, pl.n, size=6000)
    ui = ui[pl.params[ui, P_NUMEL] > 0]
    ue = (rng.random(ui.size) * pl.params[ui, P_NUMEL]).astype(np.int64)
    ue = np.concatenate([ue, np.zeros(ui.size, np.int64), pl.params[ui, P_NUMEL] - 1,
                         np.minimum(pl.params[ui, P_S], pl.params[ui, P_NUMEL] - 1)])  # first, last, row boundary
    ui = np.concatenate([ui] * 4)
    rc = [oracle.unpack_locate(pl, int(i), int(e)) for i, e in zip(ui, ue)]
    gi = (nd * pl.buckets[pl.params[ui, P_BUCKET], oracle.B_BASE] + np.array([x[0] for x in rc]) *
          pl.buckets[pl.params[ui, P_BUCKET], oracle.B_STRIDE] + np.array([x[1] for x in rc]))
    want = bits16(gathered[torch.from_numpy(gi).to(DEV)].cpu())
    got = bits16(gather_params(lp, ui, ue, 0))
    assert np.array_equal(got, want), "unpack"
    say(f"[config {config}] ok")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_fullsize_workload(config):
    try:
        run_fullsize(config)
    finally:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_fullsize_injected_inf_skips_both_paths():
    """The 7.5B paper-style list (fp16 gradients, loss scale 2^16, Nd = 64, rank 63) at its real
    size, in the launch configuration bench.py times, with one +inf planted in this rank's
    gradient at an element of its own row r.  The oracle's verdict for that step is "skip"
    (the reduced column is non-finite; its input check flags the gradient too).  The unfused
    path (pack -> reduce with the fused check -> Adam) and the fused path (checked pack ->
    reduce + Adam) both raise the flag, and neither changes p32, m, v, the step counts or the
    all-gather arena: every array bit-identical to its state before the step."""
    w = W.workload(4)
    nd, r = w.nd, w.rank
    pl = oracle.plan(w.numels, nd, r, w.bucket_bytes)
    X = Z.ShardStep(w.numels, nd, r, w.bucket_bytes, w.dtype)
    masters = W.masters(w, DEV)
    X.init_master(Z.ptr_table(masters), 0)
    lp = W.to_16bit(masters, w.dtype)
    del masters
    X.pack(Z.ptr_table(lp), out=X.arena)
    del lp
    live = W.live_mask(w, 0)
    X.live.copy_(torch.from_numpy(live))
    g = W.grads(w, 0, r, DEV)
    i = [n for n, _ in w.params].index("h.0.qkv.weight")
    s_i, col = int(pl.params[i, P_S]), int(pl.params[i, P_COL])
    j = 12345
    e = r * s_i + j                                       # element j of rank r's row of parameter i
    assert e < pl.params[i, P_NUMEL]
    g[i][e] = float("inf")
    b = int(pl.params[i, P_BUCKET])
    # the oracle's verdicts: its input check over the bucket's gradients, and the reduce of the
    # planted column (the other ranks' values from the row generator)
    host = [bits16(t.cpu()) if pl.params[k, P_BUCKET] == b else None for k, t in enumerate(g)]
    assert oracle.input_check(pl, b, host, w.dtype) == 1
    del host
    own = Z.ptr_table(g)
    X.pack(own)
    recv = []
    for bb in range(pl.n_buckets):
        L = int(pl.buckets[bb, oracle.B_STRIDE])
        blk = W.remote_rows(w, 0, bb, L, DEV).view(torch.int16)
        blk.masked_fill_(torch.from_numpy(row_zero_mask(pl, bb, live)).to(DEV).unsqueeze(0), 0)
        blk[r].copy_(X.own_row(X.packed, bb))
        recv.append(blk)
    column = bits16(recv[b][:, col + j].cpu())
    assert column[r] == 0x7C00  # the packed row carries the +inf
    g32 = np.zeros(pl.shard_len, np.float32)
    g32[int(pl.params[i, P_OFF]) + j] = oracle.reduce_column(column, w.dtype)
    only = np.zeros(pl.n, np.uint8)
    only[i] = 1
    assert oracle.overflow(pl, g32, only) == 1
    rows_of = lambda bb: (recv[bb].view(-1), int(pl.buckets[bb, oracle.B_STRIDE]))
    before = {k: t.clone() for k, t in (("p32", X.p32), ("m", X.m), ("v", X.v), ("steps", X.steps),
                                        ("arena", X.arena))}

    def unchanged(what):
        for k, t in (("p32", X.p32), ("m", X.m), ("v", X.v), ("steps", X.steps), ("arena", X.arena)):
            assert torch.equal(t.view(torch.int32) if t.dtype == torch.float32 else t,
                               before[k].view(torch.int32) if t.dtype == torch.float32 else before[k]), (what, k)

    hp = (w.lr, w.betas[0], w.betas[1], w.eps, w.grad_scale)
    X.flag.zero_()
    X.reduce(rows_of)
    X.adam(*hp)
    torch.cuda.synchronize()
    assert int(X.flag.item()) == 1
    assert not np.isfinite(to_np32(X.g32[int(pl.params[i, P_OFF]) + j:int(pl.params[i, P_OFF]) + j + 1])[0])
    unchanged("unfused")
    X.flag.zero_()
    X.pack(own, out=torch.empty_like(X.packed), check=True)
    assert int(X.flag.item()) == 1
    X.reduce_adam(rows_of, *hp)
    torch.cuda.synchronize()
    unchanged("fused")
    del recv, g, own, X, before
    torch.cuda.empty_cache()
