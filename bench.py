#!/usr/bin/env python3
"""Shard-step throughput of the ZeRO-1/2 per-rank pipeline on one MI355X.

One step = every hot-path stage for one rank over one batch of synthetic gradients: pack this
rank's gradient buckets rank-major, reduce the Nd virtual ranks' rows into the fp32 shard
(overflow flag fused), the fused mixed-precision Adam step writing the 16-bit all-gather row,
and the unpack of the gathered buckets into the per-parameter flats.  Inputs are resident in
HBM before timing starts; the boundary takes device buffers, so no PCIe transfer is involved.

The reported line is the largest list: the 7.5B paper-style list (72 layers, d = 2880,
odd-sized biases forcing padding) at Nd = 64 virtual ranks, rank 63, fp16 gradients with a
2^16 loss scale, 500M-element buckets.  The other lists (GPT-2 1.5B at Nd = 8 with the ZeRO-3
leg, Llama-7B at Nd = 8, the ragged 10,000-parameter list at Nd = 1024) run in child processes
of this one and are carried as sub-objects under `workloads`.

Prints one JSON line.  value = algorithmic HBM bytes of the step / step time (GB/s).  The line
also carries the per-stage times and roofline fractions (`kernels`), the dominant stage's
`roofline` (with the HBM bytes per launch that rocprofv3 counters measured on the current
kernel sources, or null), the fused path (`fused`: checked pack, reduce + Adam in one kernel
per bucket), the step replayed as a HIP graph (`graph`), the achievable bandwidth of the
kernels' access patterns on this device (`ceilings`, hand-written probes timed in this run),
and the CPU oracle timed on the host (`cpu_baseline`: all cores and one thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import zero_sharded_mixed_amd as Z  # noqa: E402  (fails at first call if the HIP library is missing)

HBM_PEAK_GBS = 8000.0
METRIC = "shard step GB/s & elem/s (pack+reduce+Adam) vs HBM peak, 1 MI355X"
HEADLINE = 4
OTHERS = (2, 3, 5)
ZERO3_BATCH = 2   # consecutive layers per launch in the ZeRO-3 leg
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
WORKLOAD_IDS = {1: "mlp-nd8-r3", 2: "gpt2-1.5b-nd8-r0", 3: "llama-7b-nd8-r5", 4: "paper-7.5b-nd64-r63",
                5: "ragged-10k-nd1024-r517"}
WORKLOAD_TEXT = {
    1: "MlpModel (Linear(128,256), Linear(256,256) never called, Linear(256,512)); Nd=8, rank 3, one bucket; "
       "bf16 grads N(0,1e-2); fp32 master / m / v (about 1 MB: launch-bound)",
    2: "GPT-2 1.5B-shaped parameter list (48 layers, d=1600, vocab 50257, 1024 positions); Nd=8 virtual ranks, "
       "rank 0, 500M-element buckets; bf16 grads N(0,1e-3) and params, fp32 master N(0,0.02) / m / v; Adam lr 1e-3, "
       "betas (0.9, 0.999), eps 1e-8",
    3: "Llama-7B-shaped parameter list (32 layers, d=4096, ffn 11008, vocab 32000, untied head); Nd=8, rank 5, "
       "500M-element buckets; bf16 grads N(0,1e-3) with 1% exact zeros; fp32 master / m / v",
    4: "7.5B paper-style parameter list (72 layers, d=2880, vocab 50257, untied head, odd-sized biases forcing "
       "padding; 869 params, Psi 7.46e9); Nd=64 virtual ranks, rank 63, 500M-element buckets; fp16 grads "
       "N(0,1e-3) x 2^16 loss scale; fp32 master N(0,0.02) / m / v; Adam lr 1e-3, betas (0.9, 0.999), eps 1e-8",
    5: "ragged list of 10,000 parameters, numel log-uniform in [1, 4M]; Nd=1024, rank 517, 500M-element buckets; "
       "30% without gradient; fp16 grads N(0,1e-2); fp32 master / m / v",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(numels, shard_sizes, live, nd):
    """Bytes each stage must move, per the method (not what the kernels happen to move):
    pack 2 B read per gradient element + 2 B written per padded element; reduce Nd 16-bit
    reads + one fp32 write per shard element; Adam 16 B read (g, p, m, v) + 14 B written
    (p, m, v, 16-bit param) per shard element; unpack 2 B read + 2 B written per element.
    The fused reduce + Adam: Nd 16-bit reads + 12 B read (p, m, v) + 14 B written per shard element."""
    numel_live = int(sum(int(n) for n, l in zip(numels, live) if l))
    padded_live = int(sum(int(s) * nd for s, l in zip(shard_sizes, live) if l))
    shard_live = int(sum(int(s) for s, l in zip(shard_sizes, live) if l))
    numel_all = int(sum(int(n) for n in numels))
    return {
        "pack": 2 * numel_live + 2 * padded_live,
        "reduce": (2 * nd + 4) * shard_live,
        "adam": 30 * shard_live,
        "reduce_adam": (2 * nd + 26) * shard_live,
        "unpack": 4 * numel_all,
        "shard_live": shard_live,
        "numel_live": numel_live,
        "numel_all": numel_all,
    }


def stage_elements(ab):
    """Elements each stage processes per step: pack the live gradients' elements; reduce,
    Adam and the fused reduce + Adam the live shard elements; unpack every parameter element."""
    return {"pack": ab["numel_live"], "reduce": ab["shard_live"], "adam": ab["shard_live"],
            "reduce_adam": ab["shard_live"], "unpack": ab["numel_all"]}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "zero_sharded_mixed_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = t.get(workload, {}).get(kernel)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


# --------------------------------------------------------------------------- GPU side --

class Ctx:
    """One rank's buffers and inputs for a workload, resident on the device."""

    def __init__(self, st, own_ptrs, own_out, rows_of, lp, lp_ptrs, live):
        self.st, self.own_ptrs, self.own_out, self.rows_of = st, own_ptrs, own_out, rows_of
        self.lp, self.lp_ptrs, self.live = lp, lp_ptrs, live


def _model(w, device):
    """Plan, fp32 master shard, the 16-bit model (one flat buffer, per-parameter views) and the
    all-gather arena holding it (every rank holds the full model before the step)."""
    import workloads as W

    st = Z.ShardStep(w.numels, w.nd, w.rank, w.bucket_bytes, w.dtype, device=device)
    s = st.summary
    log(f"[bench] plan: n={s.n_params} nd={s.nd} rank={s.rank} buckets={s.n_buckets} shard={s.shard_numel} "
        f"psi={s.padded_total}")
    masters = W.masters(w, device)
    st.init_master(Z.ptr_table(masters), 0)
    lp = W.to_16bit(masters, w.dtype)
    del masters
    lp_ptrs = Z.ptr_table(lp)
    st.pack(lp_ptrs, out=st.arena)
    return st, lp, lp_ptrs


def setup_full(w, device):
    """Full emulation: every virtual rank's whole gradient list is generated and packed; rank
    r's is re-packed inside each timed step."""
    import workloads as W

    t0 = time.time()
    st, lp, lp_ptrs = _model(w, device)
    live = W.live_mask(w, 0)
    st.live.copy_(torch.from_numpy(live))
    packed_all = torch.empty((w.nd, int(st.summary.arena_numel)), dtype=torch.int16, device=device)
    own_ptrs = None
    for k in range(w.nd):
        g = W.grads(w, 0, k, device)
        ptrs = Z.ptr_table([t if l else None for t, l in zip(g, live)])
        st.pack(ptrs, out=packed_all[k])
        if k == w.rank:
            own_ptrs = ptrs
        del g, ptrs
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB ({time.time() - t0:.1f}s)")
    flat = packed_all.view(-1)
    stride = int(st.summary.arena_numel)

    def rows_of(b):
        bk = st.buckets[b]
        return flat[bk.block_offset + w.rank * bk.row_stride:], stride

    ctx = Ctx(st, own_ptrs, packed_all[w.rank], rows_of, lp, lp_ptrs, live)
    ctx.packed_all = packed_all
    return ctx


def setup_rows(w, device):
    """Row-only emulation (lists whose Nd full gradient copies would not fit): the other
    virtual ranks' rows r are generated directly, one block per bucket, with the positions a
    packer leaves zero (padding, dead parameters, the row gap) set to +0.  Row r is this rank's
    own packed row, copied once: the gradients are the same in every timed step, so the reduce
    reads exactly what the step's pack writes."""
    import workloads as W

    t0 = time.time()
    st, lp, lp_ptrs = _model(w, device)
    live = W.live_mask(w, 0)
    st.live.copy_(torch.from_numpy(live))
    g = W.grads(w, 0, w.rank, device)
    own_ptrs = Z.ptr_table([t if l else None for t, l in zip(g, live)])
    del g
    st.pack(own_ptrs)
    info = [Z.zero_plan_param_info(st.plan, i) for i in range(st.n)]
    recv = []
    for b, bk in enumerate(st.buckets):
        L = int(bk.row_stride)
        keep = np.zeros(L, dtype=bool)
        for i in range(int(bk.first_param), int(bk.first_param + bk.n_params)):
            p = info[i]
            if live[i]:
                real = max(0, min(p.shard_size, p.numel - w.rank * p.shard_size))
                keep[p.bucket_col:p.bucket_col + real] = True
        zero = torch.from_numpy(~keep).to(device)
        blk = W.remote_rows(w, 0, b, L, device).view(torch.int16)
        blk.masked_fill_(zero.unsqueeze(0), 0)
        blk[w.rank].copy_(st.own_row(st.packed, b))
        recv.append(blk)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB ({time.time() - t0:.1f}s)")

    def rows_of(b):
        return recv[b].view(-1), int(st.buckets[b].row_stride)

    return Ctx(st, own_ptrs, st.packed, rows_of, lp, lp_ptrs, live)


def setup(w, device):
    torch.cuda.set_device(device)
    return setup_full(w, device) if w.emulation == "full" else setup_rows(w, device)


PHASES = {"unfused": ("pack", "reduce", "adam", "unpack"), "fused": ("pack", "reduce_adam", "unpack")}


def run_gpu(w, ctx, path, steps, warmup):
    """Time `steps` steps of one path, with HIP events on the kernels' stream around every
    stage.  unfused: pack -> reduce with the fused overflow check -> Adam -> unpack; fused:
    pack with the input check -> per-parameter step sizes + per-bucket reduce + Adam in one
    kernel -> unpack."""
    st = ctx.st
    b1, b2 = w.betas
    phases = PHASES[path]

    def one_step(ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record()

        mark(0)
        st.flag.zero_()
        st.pack(ctx.own_ptrs, out=ctx.own_out, check=(path == "fused"))
        mark(1)
        if path == "unfused":
            st.reduce(ctx.rows_of, fused_check=True)
            mark(2)
            st.adam(w.lr, b1, b2, w.eps, w.grad_scale)
        else:
            st.reduce_adam(ctx.rows_of, w.lr, b1, b2, w.eps, w.grad_scale)
        mark(len(phases) - 1)
        st.unpack(ctx.lp_ptrs)
        mark(len(phases))

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_phase = {p: 0.0 for p in phases}
    for ev in events:
        for j, p in enumerate(phases):
            per_phase[p] += ev[j].elapsed_time(ev[j + 1])
    per_phase = {p: v / steps for p, v in per_phase.items()}  # ms per step
    # launches of each stage's streaming kernel (the Adam phases also hold the small
    # per-parameter prepare kernel, a few microseconds; the pack phase a 4-byte fill)
    nb = len(st.buckets)
    launches = {"pack": nb, "reduce": nb, "adam": 1, "reduce_adam": nb, "unpack": nb}
    flag = int(st.flag.item())
    return wall / steps * 1e3, per_phase, {p: launches[p] for p in phases}, flag


def run_graph(w, ctx, steps, warmup):
    """The unfused step captured once into a HIP graph (torch.cuda.graph) and replayed: the hot
    calls allocate nothing, never synchronise and clear the flag with a fill kernel, not a
    memset, so the whole step is one graph launch.  Every buffer the captured kernels touch,
    through pointer tables included, stays referenced for the life of the graph."""
    st = ctx.st
    b1, b2 = w.betas

    def step():
        st.flag.zero_()
        st.pack(ctx.own_ptrs, out=ctx.own_out)
        st.reduce(ctx.rows_of, fused_check=True)
        st.adam(w.lr, b1, b2, w.eps, w.grad_scale)
        st.unpack(ctx.lp_ptrs)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    del g
    return ms


def run_zero3(w, ctx, steps, warmup, device, graph=True, prefetch=False, batch=ZERO3_BATCH, sweep=()):
    """ZeRO-3's step on the same list with one bucket per layer (workloads.layer_groups): the
    forward pass gathers every layer's parameters (unpack into a scratch buffer), the backward
    pass gathers all but the last layer again and reduce-scatters each layer's gradients (pack
    + reduce) right after it, then Adam writes this rank's 16-bit shard.  Full emulation: every
    virtual rank's gradients are packed for the per-layer buckets beforehand; this rank's are
    re-packed inside each timed step, into the rows the reduce reads.  All on one stream, each
    launch (zero_z3_step) handles `batch` consecutive layers: the forward gathers them, a
    backward launch packs them, gathers the batch before and reduces the batch after; `batch_1`
    times the same with one layer per launch, `separate_launches` with a launch per piece
    (`speedup` = their time / the main schedule's); `sweep` lists other batches to time; with
    prefetch=True also with the gathers on a second stream into two scratch buffers.  With graph=True each step is also
    captured into a HIP graph and replayed."""
    import workloads as W

    st2, live = ctx.st, ctx.live
    t0 = time.time()
    z = Z.ShardStep(w.numels, w.nd, w.rank, 0, w.dtype, device=device, groups=W.layer_groups(w))
    z.live.copy_(st2.live)
    z.init_master(ctx.lp_ptrs, w.dtype)  # p32 = row r of the 16-bit model (converted exactly)
    z.pack(ctx.lp_ptrs, out=z.arena)     # every rank holds its row of every layer
    an = int(z.summary.arena_numel)
    packed_all = torch.empty((w.nd, an), dtype=torch.int16, device=device)
    for k in range(w.nd):
        if k == w.rank:
            z.pack(ctx.own_ptrs, out=packed_all[k])
            continue
        g = Z.ptr_table([t if l else None for t, l in zip(W.grads(w, 0, k, device), live)])
        z.pack(g, out=packed_all[k])
        del g
    flat = packed_all.view(-1)

    def rows_of(b):
        bk = z.buckets[b]
        return flat[bk.block_offset + w.rank * bk.row_stride:], an

    shard_sizes = [Z.zero_plan_param_info(z.plan, i).shard_size for i in range(z.n)]
    ab = algorithmic_bytes(w.numels, shard_sizes, live, w.nd)
    numel_all = int(sum(int(x) for x in w.numels))
    b1, b2 = w.betas
    phases = ("forward", "backward", "adam")

    def measure(z3):
        def one_step(ev=None):
            def mark(j):
                if ev is not None:
                    ev[j].record()

            mark(0)
            z.flag.zero_()
            z3.order.clear()
            z3.forward()
            mark(1)
            z3.backward(lambda lid: ctx.own_ptrs, rows_of, out=packed_all[w.rank])
            mark(2)
            z.adam(w.lr, b1, b2, w.eps, w.grad_scale)
            mark(3)

        for _ in range(warmup):
            one_step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
        t1 = time.perf_counter()
        for i in range(steps):
            one_step(events[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t1) / steps * 1e3
        per = {p: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / steps for j, p in enumerate(phases)}
        numel_last = int(sum(int(w.numels[i]) for i in z3.layers[-1]))
        nbytes = {"forward": 4 * numel_all, "backward": 4 * (numel_all - numel_last) + ab["pack"] + ab["reduce"],
                  "adam": ab["adam"]}
        total = sum(nbytes.values())
        res = {"ms_per_step": round(wall, 4), "GBs": round(total / (wall * 1e-3) / 1e9, 1), "step_bytes": total,
               "elem_per_s": round(ab["shard_live"] / (wall * 1e-3), 1), "layers": len(z.buckets),
               "gathers_per_step": len(z3.order), "scratch_elems": int(z3.scratch.numel()),
               "overflow_flag": int(z.flag.item()),
               "phases": {p: {"ms": round(per[p], 4), "bytes": nbytes[p],
                              "GBs": round(nbytes[p] / (per[p] * 1e-3) / 1e9, 1)} for p in phases}}
        if graph:
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_step()
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            gms = (time.perf_counter() - t1) / steps * 1e3
            res["graph"] = {"ms_per_step": round(gms, 4), "GBs": round(total / (gms * 1e-3) / 1e9, 1),
                            "speedup": round(wall / gms, 3)}
            del g
        return res

    z3 = Z.Zero3Schedule(z, fused=True, batch=batch)
    torch.cuda.synchronize()
    log(f"[bench] zero3: {len(z.buckets)} layer buckets, scratch {z3.scratch.numel()} elements "
        f"({time.time() - t0:.1f}s)")
    out = measure(z3)
    out["schedule"] = (f"one stream; {batch} consecutive layers per launch; forward: gather; backward: reduce "
                       "the batch after, pack this batch, gather the batch before")
    out["batch"] = batch
    del z3
    if batch != 1:  # the same with one layer per launch
        z3 = Z.Zero3Schedule(z, fused=True)
        one = measure(z3)
        one["speedup"] = round(one["ms_per_step"] / out["ms_per_step"], 3)
        out["batch_1"] = one
        del z3
    z3 = Z.Zero3Schedule(z)  # one launch per gather, pack and reduce
    sep = measure(z3)
    sep["speedup"] = round(sep["ms_per_step"] / out["ms_per_step"], 3)
    out["separate_launches"] = sep
    del z3
    if sweep:
        out["batch_sweep"] = {}
        for k in sweep:
            z3 = Z.Zero3Schedule(z, fused=True, batch=k)
            r = measure(z3)
            out["batch_sweep"][str(k)] = {"ms_per_step": r["ms_per_step"], "GBs": r["GBs"],
                                                 "forward_ms": r["phases"]["forward"]["ms"],
                                                 "backward_ms": r["phases"]["backward"]["ms"], "scratch_elems": r["scratch_elems"]}
            del z3
    if prefetch:  # the gathers on a second stream into two scratch buffers
        z3 = Z.Zero3Schedule(z, prefetch=True)
        pf = measure(z3)
        pf["speedup"] = round(pf["ms_per_step"] / out["ms_per_step"], 3)
        out["prefetch"] = pf
        del z3
    del packed_all, z
    torch.cuda.empty_cache()
    return out


def copy_reference(device, nbytes=2 << 30, reps=10):
    """GB/s (read + write) of torch's device-to-device copy of a 2 GiB buffer, for context."""
    a = torch.empty(nbytes // 2, dtype=torch.int16, device=device)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def ceilings(device, adam_cols: int, pack_bytes: int, reps: int = 10):
    """What plain streams reach on this device, timed here with the hand-written probes of
    include/zero_probe.h (same launch shape as the pipeline kernels, trivial arithmetic):
    read-only, write-only and copy over a pack-sized buffer, and Adam's 4-read / 4-write
    stream mix over an Adam-sized shard (30 B per column).  GB/s of bytes moved; the kernels'
    fractions of these are reported next to them by the caller."""
    from zero_sharded_mixed_amd import probe

    def timed(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        return {"GBs": round(nbytes / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4), "bytes": nbytes,
                "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    nb = (pack_bytes // 2) // 16 * 16
    src = torch.empty(nb // 4, dtype=torch.int32, device=device)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=device)
    probe.write(src)
    out = {"read": timed(lambda: probe.read(src, sink), nb),
           "write": timed(lambda: probe.write(dst), nb),
           "copy": timed(lambda: probe.copy(src, dst), 2 * nb)}
    del src, dst
    n = max(adam_cols // 2048, 1) * 2048  # the probe takes whole 2048-column spans
    f32 = dict(dtype=torch.float32, device=device)
    g, p, m, v = (torch.zeros(n, **f32) for _ in range(4))
    lp = torch.zeros(n, dtype=torch.int16, device=device)
    out["adam_streams"] = timed(lambda: probe.adam_streams(g, p, m, v, lp), 30 * n)
    del g, p, m, v, lp
    torch.cuda.empty_cache()
    return out


def measure_workload(w, args, device, headline: bool):
    """Everything the line reports for one workload: both paths' per-stage times and
    fractions, the dominant stage's roofline, and the optional graph and ZeRO-3 legs."""
    import workloads as W

    wid = WORKLOAD_IDS[w.config]
    ctx = setup(w, device)
    st = ctx.st
    shard_sizes = [Z.zero_plan_param_info(st.plan, i).shard_size for i in range(st.n)]
    ab = algorithmic_bytes(w.numels, shard_sizes, ctx.live, w.nd)
    ne = stage_elements(ab)
    runs = {}
    for path in ("unfused", "fused"):
        ms_p, per_phase, launches, flag = run_gpu(w, ctx, path, args.steps, args.warmup)
        kernels = {}
        for p in PHASES[path]:
            gbs = ab[p] / (per_phase[p] * 1e-3) / 1e9
            kernels[p] = {"ms": round(per_phase[p], 4), "launches": launches[p], "bytes": ab[p],
                          "GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "elements": ne[p], "elem_per_s": round(ne[p] / (per_phase[p] * 1e-3), 1)}
        runs[path] = dict(ms=ms_p, kernels=kernels, launches=launches, flag=flag,
                          bytes=sum(ab[p] for p in PHASES[path]))
    ms, kernels, launches, flag = (runs["unfused"][k] for k in ("ms", "kernels", "launches", "flag"))
    step_bytes = runs["unfused"]["bytes"]

    def roofline(kern, name):
        d = kern[name]
        per_launch = d["bytes"] // d["launches"]
        avg_ms = d["ms"] / d["launches"]
        ach = per_launch / (avg_ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": name, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, wid),
                "bytes_per_launch": per_launch, "avg_launch_ms": round(avg_ms, 4)}

    fz = runs["fused"]
    fused = {"ms_per_step": round(fz["ms"], 4), "speedup": round(ms / fz["ms"], 3),
             "GBs": round(fz["bytes"] / (fz["ms"] * 1e-3) / 1e9, 1), "step_bytes": fz["bytes"],
             "elem_per_s": round(ab["shard_live"] / (fz["ms"] * 1e-3), 1), "overflow_flag": fz["flag"],
             "kernels": fz["kernels"], "roofline": roofline(fz["kernels"], "reduce_adam")}
    dom = max(kernels, key=lambda p: kernels[p]["ms"])
    res = {
        "workload": WORKLOAD_TEXT[w.config], "workload_id": wid, "nd": w.nd, "rank": w.rank, "n_params": w.n,
        "psi": int(sum(s * w.nd for s in shard_sizes)), "shard_elems": ab["shard_live"],
        "n_buckets": launches["pack"],
        "storage": ("bf16" if w.dtype == W.BF16 else "fp16") + " grads/params, fp32 state",
        "emulation": w.emulation,
        "ms_per_step": round(ms, 4), "GBs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "elem_per_s": round(ab["shard_live"] / (ms * 1e-3), 1),
        "grad_elem_per_s": round(ab["numel_live"] / (ms * 1e-3), 1),
        "step_bytes": step_bytes, "overflow_flag": flag, "kernels": kernels, "fused": fused,
        "roofline": roofline(kernels, dom),
    }
    if not args.no_graph:
        gms = run_graph(w, ctx, args.steps, args.warmup)
        res["graph"] = {"ms_per_step": round(gms, 4), "eager_ms_per_step": round(ms, 4),
                        "speedup": round(ms / gms, 3)}
    if w.emulation == "full" and not args.no_zero3 and not headline:
        res["zero3"] = run_zero3(w, ctx, args.steps, args.warmup, device, graph=not args.no_graph,
                                 prefetch=args.zero3_prefetch, batch=args.zero3_batch,
                                 sweep=[int(x) for x in args.zero3_sweep.split(",") if x])
    del ctx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def run_children(configs, args):
    """Each other workload in a child process of its own (its memory is returned when it
    exits); returns {workload_id: sub-object} (an `error` entry if a child failed)."""
    out = {}
    for c in configs:
        cmd = [sys.executable, os.path.abspath(__file__), "--child", "--config", str(c), "--steps",
               str(min(args.steps, args.other_steps)), "--warmup", str(args.warmup)]
        for flag in ("no_graph", "no_zero3", "zero3_prefetch"):
            if getattr(args, flag):
                cmd.append("--" + flag.replace("_", "-"))
        cmd += ["--zero3-batch", str(args.zero3_batch)]
        if args.zero3_sweep:
            cmd += ["--zero3-sweep", args.zero3_sweep]
        log(f"[bench] workload {WORKLOAD_IDS[c]} (child process) ...")
        t0 = time.time()
        try:
            r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=args.child_timeout)
            lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
            out[WORKLOAD_IDS[c]] = json.loads(lines[-1]) if r.returncode == 0 and lines else \
                {"error": f"exit status {r.returncode}"}
        except subprocess.TimeoutExpired:
            out[WORKLOAD_IDS[c]] = {"error": f"timed out after {args.child_timeout} s"}
        log(f"[bench] workload {WORKLOAD_IDS[c]} done ({time.time() - t0:.1f}s)")
    return out


# --------------------------------------------------------------------------- CPU side --

def host_cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unavailable)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_sample(w, max_elems: int, device):
    """A bounded sample of the workload for the oracle: the longest prefix of the parameter list
    with at most max_elems elements (at least one parameter), with values drawn from the
    workload's distributions (on `device`, then copied to the host)."""
    import oracle
    import workloads as W

    numels = w.numels
    keep = 1
    while keep < len(numels) and numels[:keep + 1].sum() <= max_elems:
        keep += 1
    sub = numels[:keep]
    pl = oracle.plan(sub, w.nd, w.rank, w.bucket_bytes)
    gen = torch.Generator(device=device)
    gen.manual_seed(W.seed_of(w.config, 0, 0, W.SLOT_GRAD))
    tdt = torch.bfloat16 if w.dtype == W.BF16 else torch.float16

    def bits16(n):
        x = torch.randn(n, generator=gen, device=device) * (w.grad_std * w.loss_scale)
        return x.to(tdt).view(torch.int16).cpu().numpy().view(np.uint16)

    S = pl.shard_len
    return {
        "pl": pl, "sub": sub, "keep": keep,
        "grads": [bits16(int(x)) for x in sub],
        "rows": [bits16(w.nd * int(pl.buckets[b, oracle.B_STRIDE])).reshape(w.nd, -1) for b in range(pl.n_buckets)],
        "p32": (torch.randn(S, generator=gen, device=device) * w.master_std).cpu().numpy(),
    }


def oracle_step(w, smp):
    """One full step of the oracle over the sample (pack, reduce, overflow, Adam, unpack);
    returns (seconds, outputs)."""
    import oracle

    pl = smp["pl"]
    S = pl.shard_len
    p32 = smp["p32"].copy()
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    g32 = np.zeros(S, np.float32)
    steps = np.zeros(pl.n, np.int32)
    arena = np.zeros(w.nd * S, np.uint16)
    live = np.ones(pl.n, np.uint8)
    outs = [np.empty(int(x), np.uint16) for x in smp["sub"]]
    packed = [np.zeros((w.nd, int(pl.buckets[b, oracle.B_STRIDE])), np.uint16) for b in range(pl.n_buckets)]
    hp = oracle.AdamHP(lr=w.lr, beta1=w.betas[0], beta2=w.betas[1], eps=w.eps, grad_scale=w.grad_scale)
    t0 = time.perf_counter()
    for b in range(pl.n_buckets):
        oracle.pack_bucket(pl, b, smp["grads"], out=packed[b])
    for b in range(pl.n_buckets):
        oracle.reduce_bucket(pl, b, smp["rows"][b], w.dtype, live, g32)
    flag = oracle.overflow(pl, g32, live)
    oracle.adam(pl, g32, p32, m, v, live, steps, hp, flag, arena, w.dtype)
    for b in range(pl.n_buckets):
        base = w.nd * int(pl.buckets[b, oracle.B_BASE])
        L = int(pl.buckets[b, oracle.B_STRIDE])
        oracle.unpack_bucket(pl, b, arena[base:base + w.nd * L].reshape(w.nd, L), outs)
    secs = time.perf_counter() - t0
    return secs, {"packed": packed, "g32": g32, "p32": p32, "m": m, "v": v, "arena": arena, "outs": outs,
                  "flag": flag}


def cpu_baseline(w, max_elems: int, device="cuda"):
    """The oracle as it stands, on the host cores of this machine, over a bounded sample of the
    same workload: once with one thread and once with every CPU this process may run on
    (sched_getaffinity; the oracle splits each parameter's element loops into disjoint column
    ranges, so the outputs are identical, which is checked here)."""
    import oracle

    smp = cpu_sample(w, max_elems, device)
    pl = smp["pl"]
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(1)
    t1, ref = oracle_step(w, smp)
    oracle.set_threads(cores)
    tn, got = oracle_step(w, smp)
    oracle.set_threads(1)
    same = all(np.array_equal(a.view(np.uint8), b.view(np.uint8)) for k in ("g32", "p32", "m", "v", "arena")
               for a, b in [(ref[k], got[k])])
    same = same and all(np.array_equal(a, b) for a, b in zip(ref["packed"], got["packed"]))
    same = same and all(np.array_equal(a, b) for a, b in zip(ref["outs"], got["outs"])) and ref["flag"] == got["flag"]
    ab = algorithmic_bytes(smp["sub"], pl.params[:, oracle.P_SHARD], np.ones(pl.n, np.uint8), w.nd)
    total = ab["pack"] + ab["reduce"] + ab["adam"] + ab["unpack"]
    names = [n for n, _ in w.params[:smp["keep"]]]
    sample = (f"first {smp['keep']} of {w.n} parameters ({names[0]} .. {names[-1]}), {int(smp['sub'].sum())} "
              f"elements, shard {ab['shard_live']} columns, one full step (pack, {w.nd}-way reduce, overflow, Adam, "
              f"unpack) of the plain C oracle")
    return {"value": round(total / tn / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": sample, "seconds": round(tn, 3), "elem_per_s": round(ab["shard_live"] / tn, 1),
            "identical_to_single_thread": bool(same),
            "single_thread": {"value": round(total / t1 / 1e9, 3), "cores": 1, "seconds": round(t1, 3),
                              "elem_per_s": round(ab["shard_live"] / t1, 1)},
            "cpu_model": host_cpu_model(), "host_cpus": cores, "step_bytes": total}


# ------------------------------------------------------------------- profile summaries --

KERNEL_KEYS = (("probe_adam_streams_kernel", "probe_adam_streams"), ("probe_copy_kernel", "probe_copy"),
               ("probe_read_kernel", "probe_read"), ("probe_write_kernel", "probe_write"),
               ("z3_kernel", "z3"), ("adam_prepare_kernel", "adam_prepare"), ("reduce_adam_kernel", "reduce_adam"),
               ("unpack_kernel", "unpack"), ("pack_kernel", "pack"), ("reduce_kernel", "reduce"),
               ("adam_kernel", "adam"), ("overflow_kernel", "overflow"), ("shard_init_kernel", "shard_init"))
SHORT_NAMES = tuple(s for _, s in KERNEL_KEYS) + ("pack_check",) + tuple(
    f"z3{g} (up to {k} bucket{'s' if k != 1 else ''} per kind)" for k in (1, 2, 4) for g in ("", " gathers only"))


def _short(name: str) -> str:
    for key, short in KERNEL_KEYS:
        if key in name:
            if short == "pack" and ("true>" in name or "Lb1E" in name):
                return "pack_check"  # the pack with the input check (fused path)
            if short == "z3":  # the ZeRO-3 launch, by buckets per kind (K) and kinds compiled in
                k = (name.split("Z3Parts<")[1].split(">")[0] if "Z3Parts<" in name else
                     name.split("Z3PartsILi")[1].split("E")[0] if "Z3PartsILi" in name else "?")
                targs = name.split("z3_kernel<")[1].split(">")[0].replace(" ", "").split(",") if "z3_kernel<" in name \
                    else []
                kind = " gathers only" if targs[-1:] == ["4"] else ""
                return f"z3{kind} (up to {k} bucket{'s' if k != '1' else ''} per kind)"
            return short
    return name[:60]


def summarize_profiles(root: str, workload: str, command: str, pid: str = "") -> str:
    """Reduce rocprofv3 CSV output (root/trace: --kernel-trace --stats; root/FETCH_SIZE and
    root/WRITE_SIZE: one --pmc pass each) to a short text summary, and record the HBM bytes
    per launch of every pipeline kernel in profiles/traffic.json.  The counters are scaled by
    what they read for a 2 GiB device copy (2 GiB fetched, 2 GiB written).  pid: use only the
    files of that process (the benchmark's own, not its children's).  Without root/FETCH_SIZE
    the summary holds the kernel times only and traffic.json is left alone."""
    import csv
    import glob

    def rows(pattern):
        files = sorted(glob.glob(os.path.join(root, pattern), recursive=True))
        if pid:
            files = [f for f in files if os.path.basename(f).startswith(f"{pid}_")]
        if not files:
            raise FileNotFoundError(pattern)
        with open(files[0]) as fh:
            return list(csv.DictReader(fh))

    lines = [f"# rocprofv3 summary — {workload}", "", "Commands (repo root as working directory):", "",
             "```", command, "```", "", "## Kernel time (--kernel-trace --stats)", "",
             "| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---|---|---|---|---|---|"]
    stats = rows("trace/**/*kernel_stats.csv")
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = _short(r["Name"])
        if name not in SHORT_NAMES and float(r["Percentage"]) < 1.0:
            continue
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    extra = extra_counters(root, pid)
    if not glob.glob(os.path.join(root, "FETCH_SIZE")):  # a kernel trace alone: no traffic section
        return "\n".join(lines + extra) + "\n"
    traffic = {}
    counters = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        per = {}
        for r in rows(f"{cname}/**/*counter_collection.csv"):
            if r.get("Counter_Name", cname) != cname:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        counters[cname] = per
    # calibration: the largest "copy" dispatches (a 2 GiB device copy)
    copies = [(max(v), k) for k, v in counters["FETCH_SIZE"].items() if "copy" in k.lower()]
    cal_kernel = max(copies)[1]
    known_kib = 2.0 * 1024 * 1024
    fetch_cal = max(counters["FETCH_SIZE"][cal_kernel])
    write_cal = max(counters["WRITE_SIZE"].get(cal_kernel, [known_kib]))
    f_fac, w_fac = known_kib / fetch_cal, known_kib / write_cal
    lines += ["", "## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)", "",
              f"Calibration: a 2 GiB device copy reads FETCH_SIZE {fetch_cal:.0f} KiB and WRITE_SIZE "
              f"{write_cal:.0f} KiB against 2097152 KiB each: factors {f_fac:.4f} (fetch), {w_fac:.4f} (write).", "",
              "| kernel | dispatches | avg FETCH KiB | avg WRITE KiB | scaled bytes / dispatch |",
              "|---|---|---|---|---|"]
    src_hash = kernel_source_hash()
    for kname, vals in counters["FETCH_SIZE"].items():
        short = _short(kname)
        if short not in SHORT_NAMES:
            continue
        wv = counters["WRITE_SIZE"].get(kname, [0.0])
        fk, wk = sum(vals) / len(vals), sum(wv) / len(wv)
        b = fk * 1024 * f_fac + wk * 1024 * w_fac
        prev = traffic.get(short)
        if prev:  # several instantiations (dtypes) of one kernel: keep the busiest
            if prev["bytes_per_launch"] >= b:
                continue
        traffic[short] = {"bytes_per_launch": int(b), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                          "dispatches": len(vals), "source_hash": src_hash}
        lines.append(f"| {short} | {len(vals)} | {fk:.0f} | {wk:.0f} | {b:.3e} |")
    lines += extra
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    try:
        with open(TRAFFIC_FILE) as fh:
            allt = json.load(fh)
    except (OSError, ValueError):
        allt = {}
    allt[workload] = traffic
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allt, fh, indent=1, sort_keys=True)
    return "\n".join(lines) + "\n"


def extra_counters(root: str, pid: str = "") -> list:
    """Lines of a table per further --pmc pass under root (every directory other than trace/,
    FETCH_SIZE/ and WRITE_SIZE/): the average per dispatch of each counter, per kernel."""
    import csv
    import glob

    out = []
    for d in sorted(os.listdir(root)) if os.path.isdir(root) else []:
        if d in ("trace", "FETCH_SIZE", "WRITE_SIZE") or not os.path.isdir(os.path.join(root, d)):
            continue
        files = sorted(glob.glob(os.path.join(root, d, "**", "*counter_collection.csv"), recursive=True))
        if pid:
            files = [f for f in files if os.path.basename(f).startswith(f"{pid}_")]
        if not files:
            continue
        per = {}
        with open(files[0]) as fh:
            for r in csv.DictReader(fh):
                short = _short(r["Kernel_Name"])
                if short not in SHORT_NAMES:
                    continue
                per.setdefault(short, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        names = sorted({c for v in per.values() for c in v})
        if not names:
            continue
        out += ["", f"## Counters, pass `{d}` (--pmc; average per dispatch)", "",
                "| kernel | dispatches | " + " | ".join(names) + " |", "|---" * (len(names) + 2) + "|"]
        for k in sorted(per):
            vals = per[k]
            nd = max(len(v) for v in vals.values())
            out.append(f"| {k} | {nd} | " + " | ".join(
                f"{sum(vals[c]) / len(vals[c]):.4g}" if c in vals else "" for c in names) + " |")
    return out


# -------------------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE, choices=(1, 2, 3, 4, 5),
                    help="workload of the reported line: 4 = 7.5B paper-style list at Nd=64 (default); 1 MlpModel "
                         "(launch-bound), 2 GPT-2 1.5B, 3 Llama-7B, 5 ragged at Nd=1024")
    ap.add_argument("--others", default=",".join(str(c) for c in OTHERS),
                    help="comma-separated workloads run in child processes and carried under `workloads` "
                         "('none' for none)")
    ap.add_argument("--other-steps", type=int, default=20, help="timed steps of each other workload (at most --steps)")
    ap.add_argument("--child-timeout", type=int, default=300)
    ap.add_argument("--child", action="store_true", help="internal: measure --config and print its sub-object")
    ap.add_argument("--cpu-sample-elems", type=int, default=1_500_000_000,
                    help="oracle sample: the longest prefix of the parameter list with at most this many elements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--no-zero3", action="store_true", help="skip the ZeRO-3 (one bucket per layer) leg")
    ap.add_argument("--zero3-prefetch", action="store_true",
                    help="also time ZeRO-3 with the gathers on a second stream (slower without model compute)")
    ap.add_argument("--zero3-batch", type=int, default=ZERO3_BATCH,
                    help="consecutive layers per launch in the ZeRO-3 leg (1 = one layer per launch)")
    ap.add_argument("--zero3-sweep", default="", help="comma-separated other batches to time")
    ap.add_argument("--no-graph", action="store_true", help="skip the leg that replays the step as a HIP graph")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="reduce rocprofv3 CSVs under DIR (trace/, FETCH_SIZE/, WRITE_SIZE/) to a text summary "
                         "on stdout and profiles/traffic.json, then exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summary")
    ap.add_argument("--profile-pid", default="", help="process whose rocprofv3 files are summarized")
    args = ap.parse_args()
    if args.summarize_profiles:
        print(summarize_profiles(args.summarize_profiles, WORKLOAD_IDS[args.config], args.profile_command,
                                 args.profile_pid), end="")
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU reduce-scatter/all-gather path is not implemented)", file=sys.stderr)
        sys.exit(2)
    import workloads as W

    w = W.workload(args.config)
    device = torch.device("cuda:0")
    if args.child:
        print(json.dumps(measure_workload(w, args, device, headline=False)), flush=True)
        return
    res = measure_workload(w, args, device, headline=True)
    kernels = res["kernels"]
    out = {
        "metric": METRIC,
        "value": res["GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {k: res[k] for k in ("workload", "workload_id", "nd", "rank", "n_params", "psi", "shard_elems",
                                       "n_buckets", "storage", "emulation")},
        "frac": res["frac"],
        "elem_per_s": res["elem_per_s"],
        "grad_elem_per_s": res["grad_elem_per_s"],
        "step_bytes": res["step_bytes"],
        "overflow_flag": res["overflow_flag"],
        "kernels": kernels,
        "fused": res["fused"],
        "graph": res.get("graph"),
        "roofline": res["roofline"],
        "ceilings": None,
        "copy_reference_GBs": copy_reference(device),
        "cpu_baseline": None,
        "workloads": {},
        "pid": os.getpid(),
    }
    if not args.no_ceilings:
        shard = res["shard_elems"]
        c = ceilings(device, adam_cols=shard, pack_bytes=kernels["pack"]["bytes"] // kernels["pack"]["launches"])
        for stage, pat in (("adam", "adam_streams"), ("pack", "copy"), ("unpack", "copy"), ("reduce", "read")):
            c[pat].setdefault("kernels_vs_pattern", {})[stage] = round(kernels[stage]["GBs"] / c[pat]["GBs"], 4)
        out["ceilings"] = c
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (cpu_baseline) ...")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_elems)
        log(f"[bench] oracle: {out['cpu_baseline']['single_thread']['seconds']} s on one thread, "
            f"{out['cpu_baseline']['seconds']} s on {out['cpu_baseline']['cores']}")
    others = [] if args.others in ("", "none") else [int(c) for c in args.others.split(",")]
    others = [c for c in others if c != args.config]
    torch.cuda.empty_cache()
    if others:
        out["workloads"] = run_children(others, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
