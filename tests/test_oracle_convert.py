"""Pins of the oracle's 16-bit conversions against library conversions: numpy's binary16
and torch's bfloat16 (both round to nearest, ties to even)."""
import numpy as np
import torch

import oracle
from oracle import BF16, FP16


def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
    return a == b


def test_f16_to_f32_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    assert np.all(_same(oracle.to_f32(bits, FP16), ref))


def test_bf16_to_f32_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.all(_same(oracle.to_f32(bits, BF16), ref))


def _probe_values():
    rng = np.random.default_rng(0)
    rand_bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # values next to 16-bit ties and boundaries, in both types
    h = np.arange(1 << 16, dtype=np.uint16)
    f16 = h.view(np.float16).astype(np.float32)
    b16 = (h.astype(np.uint32) << 16).view(np.float32)
    around = []
    for base in (f16[np.isfinite(f16)], b16[np.isfinite(b16)]):
        bb = base.view(np.uint32).astype(np.int64)
        for d in (-1, 0, 1, 0x1000 - 1, 0x1000, 0x1000 + 1, 0x8000 - 1, 0x8000, 0x8000 + 1):
            around.append(np.clip(bb + d, 0, 0xFFFFFFFF).astype(np.uint32))
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -24,
                        3.4e38, np.inf, -np.inf, np.nan], dtype=np.float32).view(np.uint32)
    return np.concatenate([rand_bits, *around, special]).view(np.float32)


def test_f32_to_f16_matches_numpy():
    x = _probe_values()
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.from_f32(x, FP16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan].view(np.float16)))


def test_f32_to_bf16_matches_torch():
    x = _probe_values()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.from_f32(x, BF16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.to_f32(got[nan], BF16)))
