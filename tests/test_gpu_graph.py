"""The hot calls inside a HIP graph: they allocate nothing, never synchronise and clear nothing
with a memset (the flag is cleared by a fill kernel), so one whole step — pack, reduce with
the fused check, Adam, unpack, or the fused path — can be captured and replayed.  Each replay,
with eager work, synchronisations and a release of the allocator's cache between replays, must
leave exactly the state the same number of eager steps leaves.

This rank's gradients are reachable only through their pointer table, as in a caller that
keeps the table and drops its own list: the table holds the tensors, so releasing the cache
(which torch.cuda.graph also does when capture begins) cannot unmap memory a replay reads."""
import pytest
import torch

import workloads as W
import zero_sharded_mixed_amd as Z
from gpu_harness import DEV, say

pytestmark = pytest.mark.gpu

_SETUPS = {}


def setup_workload(cfg):
    """MlpModel (one bucket) or the GPT-2 1.5B-shaped list (four 500M-element buckets), full
    emulation: every virtual rank's gradients packed into its own rows beforehand.  "1-nd64" is
    the MlpModel at 64 virtual ranks, rank 17: the reduce's many-row kernel, launched with its
    LDS reservation, inside the graph."""
    if cfg in _SETUPS:
        return _SETUPS[cfg]
    if cfg == "1-nd64":
        w = W.workload(1)
        w.nd, w.rank = 64, 17
    else:
        w = W.workload(cfg)
    say(f"graph setup: {w.name}, Nd={w.nd}, rank {w.rank}")
    st = Z.ShardStep(w.numels, w.nd, w.rank, w.bucket_bytes, w.dtype)
    masters = W.masters(w, DEV)
    st.init_master(Z.ptr_table(masters), 0)
    lp = [m.to(torch.bfloat16) for m in masters]
    del masters
    lp_ptrs = Z.ptr_table(lp)
    st.pack(lp_ptrs, out=st.arena)
    live = W.live_mask(w, 0)
    st.live.copy_(torch.from_numpy(live))
    rows = torch.zeros((w.nd, int(st.summary.arena_numel)), dtype=torch.int16, device=DEV)
    own_ptrs = None
    for k in range(w.nd):
        table = Z.ptr_table([t if l else None for t, l in zip(W.grads(w, 0, k, DEV), live)])
        st.pack(table, out=rows[k])
        if k == w.rank:
            own_ptrs = table  # the only reference to this rank's gradients
    torch.cuda.synchronize()
    _SETUPS[cfg] = (w, st, lp, lp_ptrs, own_ptrs, rows)
    return _SETUPS[cfg]


def buffers(st, lp):
    return [st.p32, st.m, st.v, st.steps, st.arena, st.flag] + lp


def snapshot(st, lp):
    return [t.clone() for t in buffers(st, lp)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [1, "1-nd64", 2])
@pytest.mark.parametrize("path", ["unfused", "fused"])
def test_captured_step_replays_like_eager_steps(cfg, path):
    w, st, lp, lp_ptrs, own_ptrs, rows = setup_workload(cfg)
    flat = rows.view(-1)
    stride = rows.shape[1]
    r = w.rank

    def rows_of(b):
        bk = st.buckets[b]
        return flat[bk.block_offset + r * bk.row_stride:], stride

    hp = (w.lr, w.betas[0], w.betas[1], w.eps, w.grad_scale)

    def step():
        st.flag.zero_()
        if path == "unfused":
            st.pack(own_ptrs, out=rows[r])
            st.reduce(rows_of)
            st.adam(*hp)
        else:
            st.pack(own_ptrs, out=rows[r], check=True)
            st.reduce_adam(rows_of, *hp)
        st.unpack(lp_ptrs)

    start = snapshot(st, lp)
    eager = []
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        eager.append(snapshot(st, lp))
    assert not torch.equal(eager[0][0], start[0])  # the step moves p32
    # back to the starting state, then capture one step (capture runs nothing)
    for t, s0 in zip(buffers(st, lp), start):
        t.copy_(s0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # torch's capture stream is the current stream inside
        step()
    torch.cuda.synchronize()
    for t, s0 in zip(buffers(st, lp), start):
        assert torch.equal(t, s0)  # capturing executed nothing
    for i in range(3):
        torch.cuda.empty_cache()
        g.replay()
        torch.cuda.synchronize()
        _ = (st.p32 * 2).sum().item()  # eager work between replays
        for j, (a, b) in enumerate(zip(buffers(st, lp), eager[i])):
            assert torch.equal(a, b), (cfg, path, i, j)
        say(f"{w.name} {path}: replay {i} matches eager step {i}")
    del g, start, eager


@pytest.fixture(autouse=True, scope="module")
def _release():
    yield
    _SETUPS.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["one-stream", "prefetch", "fused", "fused-batch2"])
@pytest.mark.parametrize("nd,rank", [(8, 3), (64, 17)])
def test_captured_zero3_step_replays_like_eager_steps(nd, rank, mode):
    prefetch = mode == "prefetch"
    """A whole ZeRO-3 step (forward gathers, backward gathers with each layer's pack + reduce,
    Adam) of a 5-layer model, captured once and replayed; with prefetch the capture spans the
    caller's stream and the gather stream."""
    import numpy as np

    from gpu_harness import random_bits, to_dev16

    d, vocab = 48, 500
    numels, groups = [vocab * d], [0]
    for layer in (1, 2, 3):
        for x in (d * 4 * d, 4 * d, 4 * d * d, d, d, d):
            numels.append(x)
            groups.append(layer)
    numels += [d, d]
    groups += [4, 4]
    say(f"zero3 graph nd={nd} rank={rank}")
    st = Z.ShardStep(numels, nd, rank, 0, Z.ZERO_BF16, groups=groups)
    rng = np.random.default_rng(nd * 7 + rank)
    st.arena.copy_(to_dev16(random_bits(rng, st.arena.numel()) & np.uint16(0xBBFF)))
    st.p32.copy_(torch.from_numpy((rng.standard_normal(st.p32.numel()) * 0.02).astype(np.float32)))
    live = np.ones(len(numels), np.uint8)
    live[[3, 4]] = 0
    st.live.copy_(torch.from_numpy(live))
    gptrs = Z.ptr_table([to_dev16(random_bits(rng, x) & np.uint16(0xBBFF)) if l else None
                         for x, l in zip(numels, live)])
    rows = [to_dev16(random_bits(rng, nd * int(bk.row_stride)) & np.uint16(0xBBFF)) for bk in st.buckets]
    z3 = Z.Zero3Schedule(st, prefetch=prefetch, fused=mode.startswith("fused"), batch=2 if "batch" in mode else 1)
    out = torch.zeros_like(st.packed)

    def rows_of(lid):
        return rows[lid], int(st.buckets[lid].row_stride)

    def step():
        st.flag.zero_()
        z3.forward()
        z3.backward(lambda lid: gptrs, rows_of, out=out)
        st.adam(1e-3, 0.9, 0.999, 1e-8, 1.0 / nd)

    bufs = [st.p32, st.m, st.v, st.steps, st.arena, st.flag, st.g32, out, z3.scratch]
    start = [t.clone() for t in bufs]
    eager = []
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        eager.append([t.clone() for t in bufs])
    # one layer per launch, or batches [0, 1], [2, 3], [4]: either way the last layer (batch)
    # is not gathered twice
    assert z3.order == [0, 1, 2, 3, 4, 3, 2, 1, 0] * 3
    for t, s0 in zip(bufs, start):
        t.copy_(s0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for t, s0 in zip(bufs, start):
        assert torch.equal(t, s0)
    for i in range(3):
        torch.cuda.empty_cache()
        g.replay()
        torch.cuda.synchronize()
        _ = (st.p32 * 2).sum().item()
        for j, (a, b) in enumerate(zip(bufs, eager[i])):
            assert torch.equal(a, b), (nd, rank, mode, i, j)
    say(f"zero3 graph nd={nd} {mode}: 3 replays match 3 eager steps")
