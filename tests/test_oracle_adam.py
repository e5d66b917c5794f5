"""Pins of the oracle's mixed-precision Adam step (the shard optimizer step of the ColossalAI
"low level zero" issue, Design / Optim; state as in the ZeRO paper summary's model-states
section) against torch.optim.Adam in float64 (a library routine for textbook Adam),
closed forms (first step, constant gradient, zero gradient), the layer-drop and skip rules."""
import numpy as np
import pytest
import torch

import oracle
from oracle import B_BASE, B_STRIDE, BF16, FP16, P_OFFSET, P_SHARD

HP = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=1.0)


def close(got, ref, rel=1e-6, abs_=1e-7):
    return np.all(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)) <= abs_ + rel * np.abs(ref))


def run_oracle_steps(p0, grads, hp=HP, live_seq=None):
    n = p0.size
    pl = oracle.plan([n], 1, 0, 0)
    p32 = np.zeros(pl.shard_len, np.float32)
    p32[:n] = p0
    m = np.zeros_like(p32)
    v = np.zeros_like(p32)
    steps = np.zeros(1, np.int32)
    arena = np.zeros(pl.shard_len, np.uint16)
    for t, g in enumerate(grads):
        g32 = np.zeros_like(p32)
        g32[:n] = g
        live = np.array([1 if live_seq is None else live_seq[t]], np.uint8)
        oracle.adam(pl, g32, p32, m, v, live, steps, hp, 0, arena, BF16)
    return p32[:n], m[:n], v[:n], int(steps[0]), arena[:n]


def test_matches_torch_adam_float64():
    rng = np.random.default_rng(0)
    p0 = (rng.standard_normal(400) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal(400) * 10.0 ** rng.uniform(-4, 0)).astype(np.float32) for _ in range(6)]
    p, m, v, t, _ = run_oracle_steps(p0, grads)
    w = torch.nn.Parameter(torch.from_numpy(p0.astype(np.float64)))
    opt = torch.optim.Adam([w], lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps)
    for g in grads:
        w.grad = torch.from_numpy(g.astype(np.float64))
        opt.step()
    st = opt.state[w]
    assert t == 6
    assert close(p, w.detach().numpy())
    assert close(m, st["exp_avg"].numpy()) and close(v, st["exp_avg_sq"].numpy(), rel=2e-6, abs_=0)


def test_first_step_closed_form():
    """From m = v = 0: m_hat = g and v_hat = g^2, so p1 = p0 - lr * g / (|g| + eps)."""
    rng = np.random.default_rng(1)
    p0 = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    g = (rng.standard_normal(1000) * 1e-3).astype(np.float32)
    p, m, v, _, _ = run_oracle_steps(p0, [g])
    g64 = g.astype(np.float64)
    assert close(p, p0 - HP.lr * g64 / (np.abs(g64) + HP.eps), rel=2e-7, abs_=0)
    assert close(m, (1 - HP.beta1) * g64, rel=2e-7, abs_=0)
    assert close(v, (1 - HP.beta2) * g64 ** 2, rel=2e-7, abs_=0)


def test_constant_gradient_closed_form():
    """With a constant gradient the bias-corrected moments stay g and g^2 exactly, so every
    step moves p by lr * g / (|g| + eps); after T steps p = p0 - T * lr * g / (|g| + eps)."""
    rng = np.random.default_rng(2)
    p0 = (rng.standard_normal(500) * 0.02).astype(np.float32)
    g = (rng.standard_normal(500) * 1e-2).astype(np.float32)
    T = 12
    p, _, _, t, _ = run_oracle_steps(p0, [g] * T)
    g64 = g.astype(np.float64)
    expect = p0 - T * HP.lr * g64 / (np.abs(g64) + HP.eps)
    assert t == T
    assert np.all(np.abs(p - expect) <= T * 2.0 ** -24 * (np.abs(p0) + T * HP.lr) + 1e-9)


def test_zero_gradient_leaves_parameter():
    p0 = np.linspace(-0.05, 0.05, 64, dtype=np.float32)
    p, m, v, t, _ = run_oracle_steps(p0, [np.zeros(64, np.float32)] * 3)
    assert np.array_equal(p, p0) and np.all(m == 0) and np.all(v == 0) and t == 3


def test_grad_scale_is_a_plain_multiplier():
    rng = np.random.default_rng(3)
    p0 = (rng.standard_normal(200) * 0.02).astype(np.float32)
    g = (rng.standard_normal(200) * 1e-3).astype(np.float32)
    a = run_oracle_steps(p0, [g * np.float32(2.0 ** -10)] * 2)
    b = run_oracle_steps(p0, [g] * 2, hp=oracle.AdamHP(grad_scale=2.0 ** -10))
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


def test_dead_parameters_skipped_steps_and_padding():
    """Layer drop (issue, Design / Optim): a parameter without a gradient keeps its p32, m,
    v, step count and published 16-bit value.  A set overflow flag skips the whole step.
    Padding slots see a zero gradient, so their p32 stays +0."""
    rng = np.random.default_rng(4)
    nd, r = 8, 3
    numels = [30, 64, 13, 5]
    pl = oracle.plan(numels, nd, r, 0)
    S = pl.shard_len
    p32 = np.zeros(S, np.float32)
    masters = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in numels]
    oracle.shard_init(pl, masters, p32)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    steps = np.zeros(4, np.int32)
    arena = np.full(nd * S, 0x1234, np.uint16)
    live = np.array([1, 0, 1, 1], np.uint8)
    g32 = (rng.standard_normal(S) * 1e-3).astype(np.float32)
    for i in range(4):  # zero gradient at padding positions, as a packer sends
        off, s, n = pl.params[i, P_OFFSET], pl.params[i, P_SHARD], numels[i]
        real = max(0, min(s, n - r * s))
        g32[off + real:off + s] = 0
    before = [a.copy() for a in (p32, m, v, steps, arena)]
    oracle.adam(pl, g32, p32, m, v, live, steps, HP, 1, arena, BF16)  # flag set: nothing changes
    for x, y in zip(before, (p32, m, v, steps, arena)):
        assert np.array_equal(x, y)
    oracle.adam(pl, g32, p32, m, v, live, steps, HP, 0, arena, BF16)
    assert list(steps) == [1, 0, 1, 1]
    L, base = pl.buckets[0, B_STRIDE], pl.buckets[0, B_BASE]
    row = arena.reshape(nd, L)[r]
    for i in range(4):
        off, s, n = pl.params[i, P_OFFSET], pl.params[i, P_SHARD], numels[i]
        sl = slice(off, off + s)
        if live[i]:
            assert not np.array_equal(p32[sl], before[0][sl]) or s == 0
            assert np.array_equal(row[sl], oracle.from_f32(p32[sl], BF16))
            real = max(0, min(s, n - r * s))
            assert np.all(p32[off + real:off + s] == 0)
        else:
            for x, y in zip(before[:3], (p32, m, v)):
                assert np.array_equal(x[sl], y[sl])
            assert np.all(row[sl] == 0x1234)
    others = np.delete(arena.reshape(nd, L), r, axis=0)
    assert np.all(others == 0x1234)  # only row r is written


@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_published_param_is_rne_of_master(dtype):
    rng = np.random.default_rng(5)
    p0 = (rng.standard_normal(300) * 0.02).astype(np.float32)
    g = (rng.standard_normal(300) * 1e-3).astype(np.float32)
    pl = oracle.plan([300], 1, 0, 0)
    p32 = np.zeros(pl.shard_len, np.float32)
    p32[:300] = p0
    z = np.zeros_like(p32)
    g32 = z.copy()
    g32[:300] = g
    arena = np.zeros(pl.shard_len, np.uint16)
    oracle.adam(pl, g32, p32, z.copy(), z.copy(), np.ones(1, np.uint8), np.zeros(1, np.int32), HP, 0, arena, dtype)
    t = torch.from_numpy(p32[:300]).to(torch.bfloat16 if dtype == BF16 else torch.float16)
    assert np.array_equal(arena[:300], t.view(torch.int16).numpy().view(np.uint16))
