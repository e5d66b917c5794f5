"""The hot calls inside a HIP graph: they allocate nothing, never synchronise and clear nothing
with a memset (the flag is cleared by a fill kernel), so one whole step — pack, reduce with
the fused check, Adam, unpack, or the fused path — can be captured and replayed.  Each replay,
with eager work and synchronisations between replays, must leave exactly the state the same
number of eager steps leaves."""
import numpy as np
import pytest
import torch

import workloads as W
import zero_sharded_mixed_amd as Z
from gpu_harness import DEV, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skip(reason="graph capture is switched off: a benchmark run that replayed a captured "
                                      "step of the GPT-2 1.5B-shaped list ended in a GPU memory fault whose cause "
                                      "has not been found; these MlpModel-sized replays passed, but share the "
                                      "mechanism")]


def mlp_setup():
    w = W.workload(1)
    st = Z.ShardStep(w.numels, w.nd, w.rank, w.bucket_bytes, w.dtype)
    masters = [m.to(DEV) for m in W.masters(w, "cpu")]
    st.init_master(Z.ptr_table(masters), 0)
    lp = [m.to(torch.bfloat16) for m in masters]
    lp_ptrs = Z.ptr_table(lp)
    st.pack(lp_ptrs, out=st.arena)
    live = W.live_mask(w, 0)
    st.live.copy_(torch.from_numpy(live))
    rows = torch.zeros((w.nd, int(st.summary.arena_numel)), dtype=torch.int16, device=DEV)
    own = None
    for k in range(w.nd):
        g = [t.to(DEV) if l else None for t, l in zip(W.grads(w, 0, k, "cpu"), live)]
        st.pack(Z.ptr_table(g), out=rows[k])
        if k == w.rank:
            own = g
    return w, st, lp, lp_ptrs, Z.ptr_table(own), rows, own


def state_of(st, lp):
    return [t.clone() for t in (st.p32, st.m, st.v, st.steps, st.arena, st.flag)] + [t.clone() for t in lp]


@pytest.mark.parametrize("path", ["unfused", "fused"])
def test_captured_step_replays_like_eager_steps(path):
    w, st, lp, lp_ptrs, own_ptrs, rows, own = mlp_setup()
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

    start = state_of(st, lp)
    eager = []
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        eager.append(state_of(st, lp))
    # back to the starting state, then capture one step (capture runs nothing)
    for t, s0 in zip([st.p32, st.m, st.v, st.steps, st.arena, st.flag] + lp, start):
        t.copy_(s0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # torch's capture stream is the current stream inside
        step()
    torch.cuda.synchronize()
    for t, s0 in zip([st.p32, st.m, st.v, st.steps, st.arena, st.flag] + lp, start):
        assert torch.equal(t, s0)  # capturing executed nothing
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        _ = (st.p32 * 2).sum().item()  # eager work between replays
        got = state_of(st, lp)
        for a, b in zip(got, eager[i]):
            assert torch.equal(a, b), (path, i)
        say(f"{path}: replay {i} matches eager step {i}")
