"""zero_adam_step_noalloc (the Adam step whose staging lives in the library's static device
array) against zero_adam_step, through the C ABI: the same kernels, so p32, m, v, the step
counts and the all-gather arena must agree bit for bit.  Two calls in a row, the second on a
smaller plan (the array then still holds the first call's values), each over two steps (one
with a dead parameter set, one with the overflow flag set); plans beyond the array's maximum
are refused before anything is launched."""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_amd as Z
from zero_sharded_mixed_amd import _binding as B
from gpu_harness import DEV, ragged_numels, say

pytestmark = pytest.mark.gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _pair(numels, nd, rank, dtype, seed):
    """Two identical ShardSteps with random state; returns them and the generator."""
    A = Z.ShardStep(numels, nd, rank, 1 << 14, dtype)
    Bs = Z.ShardStep(numels, nd, rank, 1 << 14, dtype)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    S = int(A.summary.shard_numel)
    p32 = torch.randn(S, generator=gen, device=DEV) * 0.02
    arena = torch.randint(-32768, 32767, (int(A.summary.arena_numel),), generator=gen, dtype=torch.int16,
                          device=DEV)
    for X in (A, Bs):
        X.p32.copy_(p32)
        X.arena.copy_(arena)
    return A, Bs, gen


def _same(A, Bs, what):
    for name in ("p32", "m", "v"):
        a, b = getattr(A, name), getattr(Bs, name)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{what}: {name}"
    assert torch.equal(A.steps, Bs.steps), f"{what}: steps"
    assert torch.equal(A.arena, Bs.arena), f"{what}: arena"


def _steps(numels, nd, rank, dtype, seed, what):
    A, Bs, gen = _pair(numels, nd, rank, dtype, seed)
    n = len(numels)
    S = int(A.summary.shard_numel)
    rng = np.random.default_rng(seed)
    allocated = torch.cuda.memory_allocated()
    for step, flag in ((0, 0), (1, 0), (2, 1)):
        g32 = torch.randn(S, generator=gen, device=DEV) * 3.0
        live = torch.from_numpy((rng.random(n) < 0.8).astype(np.uint8)).to(DEV)
        for X in (A, Bs):
            X.g32.copy_(g32)
            X.live.copy_(live)
            X.flag.fill_(flag)
        gs = 1.0 / nd
        A.adam(grad_scale=gs, **HP)
        before = torch.cuda.memory_allocated()
        Z.zero_adam_step_noalloc(Bs.plan, Bs.g32, Bs.p32, Bs.m, Bs.v, Bs.live, Bs.steps, grad_scale=gs,
                                 flag=Bs.flag, arena=Bs.arena, **HP)
        assert torch.cuda.memory_allocated() == before  # nothing allocated through torch either
        torch.cuda.synchronize()
        _same(A, Bs, f"{what} step {step}")
    assert int(A.steps.sum().item()) > 0
    say(f"[noalloc] {what}: n={n} nd={nd} shard={S} ok (allocated before {allocated})")


def test_noalloc_matches_adam_step_twice_second_smaller():
    rng = np.random.default_rng(71)
    big = ragged_numels(rng, 3000, 8, 1 << 14)
    small = ragged_numels(rng, 40, 3, 2000)
    _steps(big, 8, 5, Z.ZERO_BF16, 1, "first call, 3000 parameters")
    _steps(small, 3, 1, Z.ZERO_FP16, 2, "second call, 40 parameters")


def test_noalloc_refuses_plans_beyond_its_maximum():
    n = B.ADAM_NOALLOC_MAX_PARAMS + 1
    st = Z.ShardStep([1] * n, 2, 0, 0, Z.ZERO_BF16)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_adam_step_noalloc(st.plan, st.g32, st.p32, st.m, st.v, st.live, st.steps, grad_scale=1.0,
                                 flag=None, arena=st.arena, **HP)
    assert e.value.status == Z.ZERO_ERANGE
    torch.cuda.synchronize()
    assert int(st.steps.sum().item()) == 0  # nothing ran
