"""The device loss scaler, through the C ABI: the update kernel against the oracle's rule step
by step (every field bit for bit), and the Adam step reading the scale on the device (unfused
and fused paths, against the oracle and against each other) over steps with overflows."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_amd as Z
from gpu_harness import (DEV, assert_close_f32, check_arena, ragged_numels, random_bits, say, to_dev16, to_np16,
                         to_np32)

pytestmark = pytest.mark.gpu
FP16 = Z.ZERO_FP16


def device_scaler(cfg):
    t = torch.zeros(Z.LOSS_SCALER_BYTES // 4, dtype=torch.int32, device=DEV)
    Z.zero_loss_scaler_init(cfg, t)
    return t


def fields(s):
    return tuple(getattr(s, f) for f, _ in s._fields_)


@pytest.mark.parametrize("cfg", [
    (2.0 ** 16, 0, 3, 2.0, 0.5, 1.0, 2.0 ** 24, 0),
    (2.0 ** 24, 0, 1, 2.0, 0.5, 2.0 ** 20, 2.0 ** 24, 0),       # growth clamped at max
    (4.0, 0, 2, 2.0, 0.5, 1.0, 2.0 ** 24, 0),                   # back-off clamped at min
    (3.0, 1, 2, float(np.float32(1.1)), float(np.float32(0.7)), 0.01, 1e6, 5),  # rounding products
])
def test_update_matches_oracle(cfg):
    rng = np.random.default_rng(int(cfg[2]) * 17 + int(cfg[0]) % 97)
    d = device_scaler(Z.zero_loss_scaler(*cfg))
    o = oracle.Scaler(*cfg)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert fields(Z.read_loss_scaler(d)) == o.as_tuple()
    for step in range(300):
        f = int(rng.random() < 0.15)
        flag.fill_(f)
        Z.zero_loss_scaler_update(flag, d)
        oracle.loss_scaler_update(o, f)
        got = fields(Z.read_loss_scaler(d))
        assert got == o.as_tuple(), (step, got, o.as_tuple())
    assert int(flag.item()) == f  # the update reads the flag and leaves it


def test_adam_with_device_scale_both_paths():
    """Five steps at Nd = 8 with fp16 rows; the scale starts at 2^16, grows every 2 clean steps
    and backs off on the overflow steps (flag preset, as after the all-reduce of the ranks'
    flags).  grad_scale = 1/Nd; the oracle divides by its own scale."""
    nd, rank, cap = 8, 3, 2 * 60000
    rng = np.random.default_rng(44)
    numels = ragged_numels(rng, 70, nd, 40000)
    say(f"scaled adam n={len(numels)}")
    cfg = (2.0 ** 16, 0, 2, 2.0, 0.5, 1.0, 2.0 ** 24, 0)
    A = Z.ShardStep(numels, nd, rank, cap, FP16)
    F = Z.ShardStep(numels, nd, rank, cap, FP16)
    pl = oracle.plan(numels, nd, rank, cap)
    S = pl.shard_len
    p32 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    steps = np.zeros(len(numels), np.int32)
    arena = random_bits(rng, nd * S) & np.uint16(0xBBFF)
    for X in (A, F):
        X.p32.copy_(torch.from_numpy(p32))
        X.arena.copy_(to_dev16(arena))
        X.enable_loss_scaler(cfg[0], growth_interval=cfg[2], growth_factor=cfg[3], backoff_factor=cfg[4],
                             min_scale=cfg[5], max_scale=cfg[6])
    o_s = oracle.Scaler(*cfg)
    ever = np.zeros(S, dtype=bool)
    lr, b1, b2, eps, gs = 1e-3, 0.9, 0.999, 1e-8, 1.0 / nd
    for step, overflow in enumerate((0, 0, 1, 0, 1, 0, 0)):
        live = (rng.random(len(numels)) > 0.2).astype(np.uint8)
        # rows: fp16 of N(0, 1e-3) * current loss scale, as a scaled backward would give
        rows, rdev = [], []
        for b in range(pl.n_buckets):
            L = int(pl.buckets[b, oracle.B_STRIDE])
            vals = (rng.standard_normal((nd, L)) * 1e-3 * o_s.scale).astype(np.float16)
            rows.append(vals.view(np.uint16).copy())
            rdev.append(to_dev16(rows[-1].reshape(-1)))
        for X in (A, F):
            X.live.copy_(torch.from_numpy(live))
            X.flag.fill_(overflow)
        rows_of = lambda b: (rdev[b], int(pl.buckets[b, oracle.B_STRIDE]))
        A.reduce(rows_of)
        A.adam(lr, b1, b2, eps, gs)
        F.reduce_adam(rows_of, lr, b1, b2, eps, gs)
        g32 = np.zeros(S, np.float32)
        for b in range(pl.n_buckets):
            oracle.reduce_bucket(pl, b, rows[b], FP16, live, g32)
        assert oracle.overflow(pl, g32, live) == 0
        hp = oracle.AdamHP(lr=lr, beta1=b1, beta2=b2, eps=eps, grad_scale=gs / o_s.scale)
        oracle.adam(pl, g32, p32, m, v, live, steps, hp, overflow, arena, FP16)
        for X in (A, F):
            X.update_loss_scale()
        oracle.loss_scaler_update(o_s, overflow)
        torch.cuda.synchronize()
        for X in (A, F):
            assert fields(Z.read_loss_scaler(X.scaler)) == o_s.as_tuple(), step
        for ta, tf in ((A.p32, F.p32), (A.m, F.m), (A.v, F.v)):
            assert torch.equal(ta.view(torch.int32), tf.view(torch.int32)), step
        assert torch.equal(A.arena, F.arena) and torch.equal(A.steps, F.steps)
        assert np.array_equal(to_np32(A.steps), steps)
        assert_close_f32(to_np32(A.p32), p32, f"p32 step {step}")
        assert_close_f32(to_np32(A.m), m, f"m step {step}")
        assert_close_f32(to_np32(A.v), v, f"v step {step}", abs_=0.0, rel=2e-6)
        if not overflow:
            for i in np.flatnonzero(live):
                ever[pl.params[i, oracle.P_OFFSET]:pl.params[i, oracle.P_OFFSET] + pl.params[i, oracle.P_SHARD]] = True
        check_arena(pl, to_np16(A.arena), arena, to_np32(A.p32), p32, ever, FP16, f"arena {step}")
    assert o_s.scale == 2.0 ** 16 and o_s.overflows == 2  # grew at step 1, halved at 2 and 4, grew at 6


def test_misaligned_scaler_rejected():
    st = Z.ShardStep([1000], 2, 0, 0, FP16)
    buf = torch.zeros(16, dtype=torch.int32, device=DEV)
    bad = buf.view(torch.int8)[2:2 + Z.LOSS_SCALER_BYTES]
    with pytest.raises(Z.ZeroError):
        Z.zero_adam_step(st.plan, st.g32, st.p32, st.m, st.v, st.live, st.steps, 1e-3, 0.9, 0.999, 1e-8, 0.5,
                         st.flag, st.arena, loss_scaler=bad)
    with pytest.raises(Z.ZeroError):
        Z.zero_loss_scaler_update(st.flag, bad)
    torch.cuda.synchronize()
    assert int(st.steps.sum().item()) == 0
