"""The bandwidth probes (include/zero_probe.h) move the bytes they claim to move: the copy
reproduces its source, the write leaves its pattern, and the Adam-stream probe computes
p + g, m + g, v + g and the top 16 bits of the new p at every column of the lane-strided
layout.  (They are measurement kernels beside the method; these checks make sure a ceiling
is the time of real work.)"""
import numpy as np
import pytest
import torch

from gpu_harness import DEV, say

pytestmark = pytest.mark.gpu


def test_copy_write_read_probes():
    from zero_sharded_mixed_amd import probe

    say("probes: copy / write / read")
    n = (3 << 20) + 4096  # int32 words: 12 MiB + 16 KiB, a partial last block
    src = torch.arange(n, dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    probe.copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    probe.write(dst)
    torch.cuda.synchronize()
    w = dst.view(-1, 4).cpu().numpy().astype(np.uint32)
    c = np.arange(w.shape[0], dtype=np.uint32)
    assert np.array_equal(w[:, 0], c) and np.array_equal(w[:, 1], c ^ np.uint32(0x55555555))
    assert np.array_equal(w[:, 2], c ^ np.uint32(0xAAAAAAAA)) and np.array_equal(w[:, 3], ~c)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    probe.read(src, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)  # written only for an improbable XOR
    with pytest.raises(RuntimeError):  # a size that is not a multiple of 16 bytes
        probe.read(src[:3], sink)


def test_adam_streams_probe():
    from zero_sharded_mixed_amd import probe

    say("probes: adam streams")
    n = 2048 * 37
    gen = torch.Generator(device=DEV).manual_seed(5)
    g, p, m, v = (torch.randn(n, generator=gen, device=DEV) for _ in range(4))
    p0, m0, v0 = p.clone(), m.clone(), v.clone()
    lp = torch.zeros(n, dtype=torch.int16, device=DEV)
    probe.adam_streams(g, p, m, v, lp)
    torch.cuda.synchronize()
    assert torch.equal(p, p0 + g) and torch.equal(m, m0 + g) and torch.equal(v, v0 + g)
    top = (p.view(torch.int32) >> 16).to(torch.int16)
    assert torch.equal(lp, top)
    with pytest.raises(ValueError):
        probe.adam_streams(g[:2048 * 3 + 8], p, m, v, lp)
