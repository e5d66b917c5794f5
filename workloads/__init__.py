"""Seeded synthetic workloads for the shard pipeline: parameter lists and random values.

This module serves both the GPU path's callers (tests, bench, smoke) and the oracle's
callers, and holds none of the method's arithmetic: it only names parameter shapes and
draws random numbers.  Padding, sharding, packing, reduction and the optimizer live in the
GPU library and, independently, in the oracle.

Shapes follow the models the pages name: the MlpModel of the ColossalAI issue "[zero]
improving compatibility of low level zero" (Design, Optim: a Linear(256,256) that forward
never calls), GPT-2 1.5B (the upskillscore ZeRO summary, model-states section), a
Llama-7B-shaped list (the briefia.fr 7B memory example), a 7.5B list in the style of the
ZeRO paper's Nd = 64 example (ZeRO-DP stages section) with odd-sized biases so that padding
occurs, and a ragged stress list.  No dataset, tokenizer or trained weight is involved.

Seeds: every random tensor is drawn from a generator seeded with
    1_000_003 * config + 10_007 * step + 101 * virtual_rank + slot
(slot 0 = fp32 master, 1 = gradients, 2 = drop mask, 3 = inf/NaN injection, 4 = remote
rows), consumed in parameter-list order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BF16 = 1
FP16 = 2

SLOT_MASTER, SLOT_GRAD, SLOT_DROP, SLOT_INJECT, SLOT_ROWS = 0, 1, 2, 3, 4


def seed_of(config: int, step: int, vrank: int, slot: int) -> int:
    return 1_000_003 * config + 10_007 * step + 101 * vrank + slot


# ----------------------------------------------------------------- parameter lists ----

def mlp_model():
    """MlpModel: linear1 = Linear(128, 256), drop_linear = Linear(256, 256) (never called in
    forward), linear2 = Linear(256, 512); weights are [out, in]."""
    return [("linear1.weight", (256, 128)), ("linear1.bias", (256,)),
            ("drop_linear.weight", (256, 256)), ("drop_linear.bias", (256,)),
            ("linear2.weight", (512, 256)), ("linear2.bias", (512,))]


def gpt2_1p5b():
    """GPT-2 1.5B: 48 layers, d = 1600, vocab 50257, 1024 positions, tied head."""
    d, L = 1600, 48
    out = [("wte", (50257, d)), ("wpe", (1024, d))]
    for l in range(L):
        h = f"h.{l}."
        out += [(h + "ln_1.weight", (d,)), (h + "ln_1.bias", (d,)),
                (h + "attn.c_attn.weight", (d, 3 * d)), (h + "attn.c_attn.bias", (3 * d,)),
                (h + "attn.c_proj.weight", (d, d)), (h + "attn.c_proj.bias", (d,)),
                (h + "ln_2.weight", (d,)), (h + "ln_2.bias", (d,)),
                (h + "mlp.c_fc.weight", (d, 4 * d)), (h + "mlp.c_fc.bias", (4 * d,)),
                (h + "mlp.c_proj.weight", (4 * d, d)), (h + "mlp.c_proj.bias", (d,))]
    out += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    return out


def llama_7b():
    """Llama-7B: 32 layers, d = 4096, ffn 11008, vocab 32000, RMSNorm vectors, untied head."""
    d, f, L = 4096, 11008, 32
    out = [("embed_tokens", (32000, d))]
    for l in range(L):
        h = f"layers.{l}."
        out += [(h + "q_proj", (d, d)), (h + "k_proj", (d, d)), (h + "v_proj", (d, d)), (h + "o_proj", (d, d)),
                (h + "gate_proj", (f, d)), (h + "up_proj", (f, d)), (h + "down_proj", (d, f)),
                (h + "input_layernorm", (d,)), (h + "post_attention_layernorm", (d,))]
    out += [("norm", (d,)), ("lm_head", (32000, d))]
    return out


def paper_7p5b():
    """7.5B list in the style of the ZeRO paper's example: 72 layers, d = 2880, untied head;
    the qkv, out, fc and proj biases have one extra element each so padding occurs."""
    d, L = 2880, 72
    out = [("wte", (50257, d)), ("wpe", (1024, d))]
    for l in range(L):
        h = f"h.{l}."
        out += [(h + "ln_1.weight", (d,)), (h + "ln_1.bias", (d,)),
                (h + "qkv.weight", (d, 3 * d)), (h + "qkv.bias", (3 * d + 1,)),
                (h + "out.weight", (d, d)), (h + "out.bias", (d + 1,)),
                (h + "ln_2.weight", (d,)), (h + "ln_2.bias", (d,)),
                (h + "fc.weight", (d, 4 * d)), (h + "fc.bias", (4 * d + 1,)),
                (h + "proj.weight", (4 * d, d)), (h + "proj.bias", (d + 1,))]
    out += [("ln_f.weight", (d,)), ("ln_f.bias", (d,)), ("lm_head", (50257, d))]
    return out


def ragged(n: int = 10_000, max_numel: int = 4 * 2 ** 20, seed: int = 0):
    """n flat parameters, numel = round(exp(U(0, ln max_numel))), seeded."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, math.log(max_numel), size=n)
    numels = np.rint(np.exp(u)).astype(np.int64)
    return [(f"p{i}", (int(x),)) for i, x in enumerate(numels)]


# ----------------------------------------------------------------- configurations -----

@dataclass
class Workload:
    config: int
    name: str
    params: list               # [(name, shape)]
    nd: int
    rank: int
    bucket_bytes: int          # 0 = one bucket
    dtype: int                 # BF16 / FP16
    steps: int
    grad_std: float
    master_std: float = 0.02
    loss_scale: float = 1.0
    zero_frac: float = 0.0     # fraction of exact +0 gradient elements
    drop_frac: float = 0.0     # fraction of parameters without a gradient, redrawn per step
    always_dead: tuple = ()    # parameter indices never live
    inject_frac: float = 0.0   # fraction of inf/NaN injected on odd steps
    emulation: str = "full"    # "full": every virtual rank's whole gradient list; "rows": only row r
    lr: float = 1e-3
    betas: tuple = (0.9, 0.999)
    eps: float = 1e-8
    extra: dict = field(default_factory=dict)

    @property
    def numels(self) -> np.ndarray:
        return np.array([int(np.prod(s)) for _, s in self.params], dtype=np.int64)

    @property
    def n(self) -> int:
        return len(self.params)

    @property
    def grad_scale(self) -> float:
        """1 / (Nd * loss_scale): mean over ranks of the unscaled gradients."""
        return 1.0 / (self.nd * self.loss_scale)


def workload(config: int) -> Workload:
    if config == 1:
        return Workload(1, "MlpModel", mlp_model(), nd=8, rank=3, bucket_bytes=0, dtype=BF16, steps=3,
                        grad_std=1e-2, always_dead=(2, 3), emulation="full")
    if config == 2:
        return Workload(2, "GPT-2 1.5B", gpt2_1p5b(), nd=8, rank=0, bucket_bytes=1_000_000_000, dtype=BF16,
                        steps=1, grad_std=1e-3, emulation="full")
    if config == 3:
        return Workload(3, "Llama-7B", llama_7b(), nd=8, rank=5, bucket_bytes=1_000_000_000, dtype=BF16, steps=10,
                        grad_std=1e-3, zero_frac=0.01, emulation="rows")
    if config == 4:
        return Workload(4, "7.5B paper-style", paper_7p5b(), nd=64, rank=63, bucket_bytes=1_000_000_000,
                        dtype=FP16, steps=3, grad_std=1e-3, loss_scale=2.0 ** 16, emulation="rows")
    if config == 5:
        return Workload(5, "ragged 10k", ragged(), nd=1024, rank=517, bucket_bytes=1_000_000_000, dtype=FP16,
                        steps=5, grad_std=1e-2, drop_frac=0.3, inject_frac=1e-6, emulation="rows")
    raise ValueError(f"no workload {config}")


def layer_groups(w: Workload) -> list:
    """One id per parameter naming its ZeRO-3 unit (the llm-engineer "ZeRO-3" card gathers and
    frees parameters one layer at a time): the parameters before the first transformer block
    (embeddings), each block ("h.<l>." / "layers.<l>."), and the parameters after the last block
    (final norm, untied head).  Lists without blocks: one unit per module (the name up to its
    last dot)."""
    names = [n for n, _ in w.params]
    blocks = any(n.startswith(("h.", "layers.")) for n in names)
    keys, seen = [], False
    for n in names:
        if n.startswith(("h.", "layers.")):
            keys.append(".".join(n.split(".")[:2]))
            seen = True
        elif blocks:
            keys.append("after" if seen else "before")
        else:
            keys.append(n.rsplit(".", 1)[0])
    ids = []
    for j, k in enumerate(keys):  # runs of equal keys, numbered in list order
        ids.append(0 if j == 0 else ids[-1] + (k != keys[j - 1]))
    return ids


# ----------------------------------------------------------------- random values ------
# Every list of per-parameter tensors is drawn as ONE flat buffer (a few large draws, not one
# per parameter: a 10,000-parameter list would otherwise issue tens of thousands of tiny
# launches) and returned as views into it.  Each view starts 256 bytes after a multiple of 256
# bytes, like separate allocations would, so buffers keep the alignment the kernels' wide
# paths need.

ALIGN_BYTES = 256
DRAW_CHUNK = 1 << 27  # elements per draw call


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _torch_dtype(dtype: int):
    return torch.bfloat16 if dtype == BF16 else torch.float16


def flat_layout(numels, elem_bytes: int):
    """Start of every parameter in one flat buffer (each start a multiple of ALIGN_BYTES) and
    the buffer's length, in elements."""
    align = ALIGN_BYTES // elem_bytes
    starts, pos = [], 0
    for x in numels:
        starts.append(pos)
        pos += (int(x) + align - 1) // align * align
    return starts, max(pos, align)


def _draw_normal(total: int, std: float, out_dtype, gen: torch.Generator, device) -> torch.Tensor:
    """total values N(0, 1) * std, drawn in order in DRAW_CHUNK pieces, converted to out_dtype
    by torch's own conversion."""
    out = torch.empty(total, dtype=out_dtype, device=device)
    for a in range(0, total, DRAW_CHUNK):
        b = min(total, a + DRAW_CHUNK)
        x = torch.randn(b - a, generator=gen, device=device, dtype=torch.float32)
        out[a:b] = x.mul_(std) if out_dtype == torch.float32 else (x * std).to(out_dtype)
    return out


def _views(flat: torch.Tensor, numels, starts) -> list:
    return [flat[s:s + int(x)] for s, x in zip(starts, numels)]


def normal_fp32(numel: int, std: float, gen: torch.Generator, device) -> torch.Tensor:
    return _draw_normal(int(numel), std, torch.float32, gen, device)


def normal_16(numel: int, std: float, scale: float, dtype: int, gen: torch.Generator, device) -> torch.Tensor:
    """N(0, std) * scale rounded to the 16-bit type by torch's own conversion."""
    return _draw_normal(int(numel), std * scale, _torch_dtype(dtype), gen, device)


def masters(w: Workload, device) -> list:
    """Full fp32 master parameters N(0, master_std): one view per parameter into one buffer."""
    g = _gen(seed_of(w.config, 0, 0, SLOT_MASTER), device)
    starts, total = flat_layout(w.numels, 4)
    return _views(normal_fp32(total, w.master_std, g, device), w.numels, starts)


def to_16bit(views: list, dtype: int) -> list:
    """A list of views into one flat buffer (as masters() returns), converted to the 16-bit
    type by one torch conversion of that buffer; the new views sit at the same element
    offsets (so each still starts on a 16-byte boundary)."""
    base = views[0]._base if views[0]._base is not None else views[0]
    assert all(v._base is base or v is base for v in views), "views of one flat buffer expected"
    flat = base.to(_torch_dtype(dtype))
    return [flat[v.storage_offset():v.storage_offset() + v.numel()] for v in views]


def grads(w: Workload, step: int, vrank: int, device) -> list:
    """One virtual rank's full gradient list (16-bit; one view per parameter into one buffer),
    with exact zeros at a fraction zero_frac of the elements if asked."""
    g = _gen(seed_of(w.config, step, vrank, SLOT_GRAD), device)
    starts, total = flat_layout(w.numels, 2)
    flat = normal_16(total, w.grad_std, w.loss_scale, w.dtype, g, device)
    if w.zero_frac > 0:
        for a in range(0, total, DRAW_CHUNK):
            b = min(total, a + DRAW_CHUNK)
            z = torch.rand(b - a, generator=g, device=device) < w.zero_frac
            flat[a:b].masked_fill_(z, 0.0)
    return _views(flat, w.numels, starts)


def live_mask(w: Workload, step: int) -> np.ndarray:
    """uint8 [n]: 1 where the parameter has a gradient this step (same for every rank)."""
    live = np.ones(w.n, dtype=np.uint8)
    for i in w.always_dead:
        live[i] = 0
    if w.drop_frac > 0:
        rng = np.random.default_rng(seed_of(w.config, step, 0, SLOT_DROP))
        live[rng.random(w.n) < w.drop_frac] = 0
    return live


def remote_rows(w: Workload, step: int, bucket: int, length: int, device) -> torch.Tensor:
    """Random 16-bit values standing for every virtual rank's packed row r of one bucket
    ([Nd, length]; row k = virtual rank k's), drawn at once (row-only emulation; the caller
    puts this rank's own row in place and zeroes the positions a real packer leaves zero)."""
    g = _gen(seed_of(w.config, step, 0, SLOT_ROWS) + 7 * bucket, device)
    return normal_16(w.nd * int(length), w.grad_std, w.loss_scale, w.dtype, g, device).view(w.nd, int(length))


def injections(w: Workload, step: int, count_space: int, device="cpu"):
    """Positions (into a space of count_space candidates) and 16-bit values of the inf/NaN
    injected on odd steps: max(1, round(inject_frac * count_space)) draws from {+inf, -inf, NaN}."""
    if w.inject_frac <= 0 or step % 2 == 0 or count_space == 0:
        return np.zeros(0, dtype=np.int64), torch.zeros(0, dtype=_torch_dtype(w.dtype))
    rng = np.random.default_rng(seed_of(w.config, step, 0, SLOT_INJECT))
    k = max(1, int(round(w.inject_frac * count_space)))
    pos = rng.choice(count_space, size=k, replace=False).astype(np.int64)
    kinds = rng.integers(0, 3, size=k)
    vals = torch.tensor([math.inf, -math.inf, math.nan], dtype=torch.float32)[torch.from_numpy(kinds)]
    return pos, vals.to(_torch_dtype(w.dtype))
