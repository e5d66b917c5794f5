#!/usr/bin/env python3
"""Shard-step throughput of the ZeRO-1/2 per-rank pipeline on one MI355X.

One step = every hot-path stage for one rank over one batch of synthetic gradients:
pack this rank's gradient buckets rank-major, reduce the Nd virtual ranks' rows into the fp32
shard (overflow flag fused), the fused mixed-precision Adam step writing the 16-bit all-gather
row, and the unpack of the gathered buckets into the per-parameter flats.  The default
workload is a GPT-2 1.5B-shaped parameter list at Nd = 8 virtual ranks, rank 0, 500M-element
buckets, bf16 gradients and parameters, fp32 master / momentum / variance, with the other
virtual ranks' gradients packed beforehand (their rows are what a reduce-scatter would
deliver).  Inputs are resident in HBM before timing starts.

Prints one JSON line (rank 0).  value = algorithmic HBM bytes of the step / step time.  The
line also carries per-stage times and roofline fractions, the fused path (`fused`: checked
pack, reduce + Adam in one kernel per bucket), the step replayed as a HIP graph (`graph`),
ZeRO-3's step with one bucket per layer (`zero3`, one stream and `prefetch`), torch's device
copy as a reference, and the CPU oracle's throughput (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import zero_sharded_mixed_amd as Z  # noqa: E402  (fails at first call if the HIP library is missing)

HBM_PEAK_GBS = 8000.0
METRIC = "shard step GB/s & elem/s (pack+reduce+Adam) vs HBM peak, 1 MI355X"
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
    4: "7.5B paper-style list (72 layers, d=2880, odd-sized biases forcing padding); Nd=64, rank 63; fp16 grads "
       "N(0,1e-3) x 2^16 loss scale; fp32 master / m / v",
    5: "ragged list of 10,000 parameters, numel log-uniform in [1, 4M]; Nd=1024, rank 517; 30% without gradient; "
       "fp16 grads N(0,1e-2); fp32 master / m / v",
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

def setup_gpu(w, device):
    import workloads as W

    torch.cuda.set_device(device)
    t0 = time.time()
    st = Z.ShardStep(w.numels, w.nd, w.rank, w.bucket_bytes, w.dtype, device=device)
    s = st.summary
    log(f"[bench] plan: n={s.n_params} nd={s.nd} rank={s.rank} buckets={s.n_buckets} shard={s.shard_numel} "
        f"psi={s.padded_total} ({time.time() - t0:.1f}s)")
    masters = W.masters(w, device)
    st.init_master(Z.ptr_table(masters), 0)
    lp = [m.to(torch.bfloat16 if w.dtype == W.BF16 else torch.float16) for m in masters]
    del masters
    lp_ptrs = Z.ptr_table(lp)
    st.pack(lp_ptrs, out=st.arena)  # every rank holds the full model: the gathered rows start equal
    live = W.live_mask(w, 0)
    st.live.copy_(torch.from_numpy(live))
    # every virtual rank's packed gradients; rank r's are re-packed inside each timed step
    packed_all = torch.empty((w.nd, int(s.arena_numel)), dtype=torch.int16, device=device)
    own = None
    for k in range(w.nd):
        g = W.grads(w, 0, k, device)
        gl = [t if l else None for t, l in zip(g, live)]
        ptrs = Z.ptr_table(gl)
        st.pack(ptrs, out=packed_all[k])
        if k == w.rank:
            own = (gl, ptrs)
        else:
            del gl, g
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB ({time.time() - t0:.1f}s)")
    flat = packed_all.view(-1)
    stride = int(s.arena_numel)

    def rows_of(b):
        bk = st.buckets[b]
        return flat[bk.block_offset + w.rank * bk.row_stride:], stride

    return st, own, packed_all, rows_of, lp, lp_ptrs, live


def setup_gpu_rows(w, device):
    """Row-only emulation (lists whose Nd full gradient copies would not fit): the other
    virtual ranks' rows r are generated directly per bucket, with the positions a packer leaves
    zero (padding, dead parameters, the row gap) set to +0.  Row r is this rank's own packed
    row, copied once: the gradients are the same in every timed step, so the reduce reads
    exactly what the step's pack writes."""
    import workloads as W

    torch.cuda.set_device(device)
    t0 = time.time()
    st = Z.ShardStep(w.numels, w.nd, w.rank, w.bucket_bytes, w.dtype, device=device)
    s = st.summary
    log(f"[bench] plan: n={s.n_params} nd={s.nd} rank={s.rank} buckets={s.n_buckets} shard={s.shard_numel} "
        f"psi={s.padded_total} ({time.time() - t0:.1f}s)")
    masters = W.masters(w, device)
    st.init_master(Z.ptr_table(masters), 0)
    lp = [m.to(torch.bfloat16 if w.dtype == W.BF16 else torch.float16) for m in masters]
    del masters
    lp_ptrs = Z.ptr_table(lp)
    st.pack(lp_ptrs, out=st.arena)
    live = W.live_mask(w, 0)
    st.live.copy_(torch.from_numpy(live))
    g = W.grads(w, 0, w.rank, device)
    gl = [t if l else None for t, l in zip(g, live)]
    own_ptrs = Z.ptr_table(gl)
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
        blk = torch.empty((w.nd, L), dtype=torch.int16, device=device)
        for k in range(w.nd):
            if k == w.rank:
                blk[k].copy_(st.own_row(st.packed, b))
            else:
                blk[k].copy_(W.remote_row(w, 0, k, b, L, device).view(torch.int16))
                blk[k].masked_fill_(zero, 0)
        recv.append(blk)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB ({time.time() - t0:.1f}s)")

    def rows_of(b):
        return recv[b].view(-1), int(st.buckets[b].row_stride)

    return st, (gl, own_ptrs), st.packed, rows_of, lp, lp_ptrs, live


def setup(w, device):
    if w.emulation == "full":
        st, own, packed_all, rows_of, lp, lp_ptrs, live = setup_gpu(w, device)
        own_out = packed_all[w.rank]
    else:
        st, own, own_out, rows_of, lp, lp_ptrs, live = setup_gpu_rows(w, device)
    return st, own[1], own_out, rows_of, lp, lp_ptrs, live


PHASES = {"unfused": ("pack", "reduce", "adam", "unpack"), "fused": ("pack", "reduce_adam", "unpack")}


def run_gpu(w, ctx, path, steps, warmup):
    """Time `steps` steps of one path.  unfused: pack -> reduce with the fused overflow check
    -> Adam -> unpack; fused: pack with the input check -> per-parameter step sizes + per-bucket
    reduce + Adam in one kernel -> unpack."""
    st, own_ptrs, own_out, rows_of, lp, lp_ptrs, live = ctx
    b1, b2 = w.betas
    phases = PHASES[path]

    def one_step(ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record()

        mark(0)
        st.flag.zero_()
        st.pack(own_ptrs, out=own_out, check=(path == "fused"))
        mark(1)
        if path == "unfused":
            st.reduce(rows_of, fused_check=True)
            mark(2)
            st.adam(w.lr, b1, b2, w.eps, w.grad_scale)
        else:
            st.reduce_adam(rows_of, w.lr, b1, b2, w.eps, w.grad_scale)
        mark(len(phases) - 1)
        st.unpack(lp_ptrs)
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
    st, own_ptrs, own_out, rows_of, lp, lp_ptrs, live = ctx
    b1, b2 = w.betas

    def step():
        st.flag.zero_()
        st.pack(own_ptrs, out=own_out)
        st.reduce(rows_of, fused_check=True)
        st.adam(w.lr, b1, b2, w.eps, w.grad_scale)
        st.unpack(lp_ptrs)

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


def run_zero3(w, ctx, steps, warmup, device, graph=True):
    """ZeRO-3's step on the same list with one bucket per layer (workloads.layer_groups): the
    forward pass gathers every layer's parameters (unpack into a scratch buffer), the backward
    pass gathers all but the last layer again and reduce-scatters each layer's gradients (pack
    + reduce) right after it, then Adam writes this rank's 16-bit shard.  Full emulation: every
    virtual rank's gradients are packed for the per-layer buckets beforehand; this rank's are
    re-packed inside each timed step, into the rows the reduce reads.  Timed twice: all on one
    stream, and with prefetch (the gathers on a second stream into two scratch buffers, the
    next layer's gather overlapping the current layer's pack and reduce).  With graph=True each
    step (about 200 launches) is also captured once into a HIP graph and the replays timed."""
    import workloads as W

    st2, own_ptrs, _, _, lp, lp_ptrs, live = ctx
    t0 = time.time()
    z = Z.ShardStep(w.numels, w.nd, w.rank, 0, w.dtype, device=device, groups=W.layer_groups(w))
    z.live.copy_(st2.live)
    z.init_master(lp_ptrs, w.dtype)  # p32 = row r of the 16-bit model (converted exactly)
    z.pack(lp_ptrs, out=z.arena)     # every rank holds its row of every layer
    an = int(z.summary.arena_numel)
    packed_all = torch.empty((w.nd, an), dtype=torch.int16, device=device)
    for k in range(w.nd):
        if k == w.rank:
            z.pack(own_ptrs, out=packed_all[k])
            continue
        g = [t if l else None for t, l in zip(W.grads(w, 0, k, device), live)]
        z.pack(Z.ptr_table(g), out=packed_all[k])
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
            z3.backward(lambda lid: own_ptrs, rows_of, out=packed_all[w.rank])
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

    z3 = Z.Zero3Schedule(z)
    torch.cuda.synchronize()
    log(f"[bench] zero3: {len(z.buckets)} layer buckets, scratch {z3.scratch.numel()} elements "
        f"({time.time() - t0:.1f}s)")
    out = measure(z3)
    del z3
    # the same step with the gathers on a second stream into two scratch buffers
    z3 = Z.Zero3Schedule(z, prefetch=True)
    pf = measure(z3)
    pf["speedup"] = round(out["ms_per_step"] / pf["ms_per_step"], 3)
    out["prefetch"] = pf
    del packed_all, z3, z
    torch.cuda.empty_cache()
    return out


def copy_reference(device, nbytes=2 << 30, reps=10):
    """GB/s (read + write) of torch's device-to-device copy of a 2 GiB buffer: what a plain
    streaming kernel reaches on this device, for context next to the 8 TB/s peak."""
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


def cpu_baseline(w, max_elems: int):
    """The oracle, single-threaded, on a prefix of the same parameter list (the whole step:
    pack, reduce, overflow, Adam, unpack), inputs drawn from the same distributions."""
    import oracle
    import workloads as W

    numels = w.numels
    keep = 1
    while keep < len(numels) and numels[:keep + 1].sum() <= max_elems:
        keep += 1
    sub = numels[:keep]
    pl = oracle.plan(sub, w.nd, w.rank, w.bucket_bytes)
    # values drawn on the device (fast) from the workload's distributions, copied to the host
    gen = torch.Generator(device="cuda")
    gen.manual_seed(W.seed_of(w.config, 0, 0, W.SLOT_GRAD))
    tdt = torch.bfloat16 if w.dtype == W.BF16 else torch.float16

    def bits16(n, std):
        x = torch.randn(n, generator=gen, device="cuda") * std
        return x.to(tdt).view(torch.int16).cpu().numpy().view(np.uint16)

    grads = [bits16(int(x), w.grad_std) for x in sub]
    S = pl.shard_len
    rows = [bits16(w.nd * int(pl.buckets[b, oracle.B_STRIDE]), w.grad_std).reshape(w.nd, -1)
            for b in range(pl.n_buckets)]
    p32 = (torch.randn(S, generator=gen, device="cuda") * w.master_std).cpu().numpy()
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    g32 = np.zeros(S, np.float32)
    steps = np.zeros(pl.n, np.int32)
    arena = np.zeros(w.nd * S, np.uint16)
    live = np.ones(pl.n, np.uint8)
    outs = [np.empty(int(x), np.uint16) for x in sub]
    hp = oracle.AdamHP(lr=w.lr, beta1=w.betas[0], beta2=w.betas[1], eps=w.eps, grad_scale=w.grad_scale)
    t0 = time.perf_counter()
    for b in range(pl.n_buckets):
        oracle.pack_bucket(pl, b, grads)
    for b in range(pl.n_buckets):
        oracle.reduce_bucket(pl, b, rows[b], w.dtype, live, g32)
    flag = oracle.overflow(pl, g32, live)
    oracle.adam(pl, g32, p32, m, v, live, steps, hp, flag, arena, w.dtype)
    for b in range(pl.n_buckets):
        base = w.nd * int(pl.buckets[b, oracle.B_BASE])
        L = int(pl.buckets[b, oracle.B_STRIDE])
        oracle.unpack_bucket(pl, b, arena[base:base + w.nd * L].reshape(w.nd, L), outs)
    secs = time.perf_counter() - t0
    ab = algorithmic_bytes(sub, pl.params[:, oracle.P_SHARD], live, w.nd)
    total = ab["pack"] + ab["reduce"] + ab["adam"] + ab["unpack"]
    names = [n for n, _ in w.params[:keep]]
    return {"value": round(total / secs / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "cpu_model": host_cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "seconds": round(secs, 2), "elem_per_s": round(ab["shard_live"] / secs, 1),
            "sample": f"first {keep} of {len(numels)} parameters ({names[0]} .. {names[-1]}), "
                      f"{int(sub.sum())} elements, one full step (pack, reduce, overflow, Adam, unpack), "
                      f"single thread, plain C oracle"}


# ------------------------------------------------------------------- profile summaries --

KERNEL_KEYS = (("adam_prepare_kernel", "adam_prepare"), ("reduce_adam_kernel", "reduce_adam"),
               ("unpack_kernel", "unpack"), ("pack_kernel", "pack"), ("reduce_kernel", "reduce"),
               ("adam_kernel", "adam"), ("overflow_kernel", "overflow"), ("shard_init_kernel", "shard_init"))
SHORT_NAMES = tuple(s for _, s in KERNEL_KEYS) + ("pack_check",)


def _short(name: str) -> str:
    for key, short in KERNEL_KEYS:
        if key in name:
            if short == "pack" and ("true>" in name or "Lb1E" in name):
                return "pack_check"  # the pack with the input check (fused path)
            return short
    return name[:60]


def summarize_profiles(root: str, workload: str, command: str) -> str:
    """Reduce rocprofv3 CSV output (root/trace: --kernel-trace --stats; root/FETCH_SIZE and
    root/WRITE_SIZE: one --pmc pass each) to a short text summary, and record the HBM bytes
    per launch of every pipeline kernel in profiles/traffic.json.  The counters are scaled by
    what they read for torch's 2 GiB device copy (2 GiB fetched, 2 GiB written).  Without
    root/FETCH_SIZE the summary holds the kernel times only and traffic.json is left alone."""
    import csv
    import glob

    def rows(pattern):
        files = glob.glob(os.path.join(root, pattern), recursive=True)
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
    if not glob.glob(os.path.join(root, "FETCH_SIZE")):  # a kernel trace alone: no traffic section
        return "\n".join(lines) + "\n"
    traffic = {}
    counters = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        per = {}
        for r in rows(f"{cname}/**/*counter_collection.csv"):
            if r.get("Counter_Name", cname) != cname:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        counters[cname] = per
    # calibration: the largest "copy" dispatches (torch's 2 GiB device copy)
    copies = [(max(v), k) for k, v in counters["FETCH_SIZE"].items() if "copy" in k.lower()]
    cal_kernel = max(copies)[1]
    known_kib = 2.0 * 1024 * 1024
    fetch_cal = max(counters["FETCH_SIZE"][cal_kernel])
    write_cal = max(counters["WRITE_SIZE"].get(cal_kernel, [known_kib]))
    f_fac, w_fac = known_kib / fetch_cal, known_kib / write_cal
    lines += ["", "## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)", "",
              f"Calibration: torch's 2 GiB device copy reads FETCH_SIZE {fetch_cal:.0f} KiB and WRITE_SIZE "
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


# -------------------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=(1, 2, 3, 4, 5),
                    help="workload: 2 = GPT-2 1.5B-shaped list (the default and the reported line); 1 MlpModel "
                         "(launch-bound), 3 Llama-7B, 4 7.5B paper-style at Nd=64, 5 ragged at Nd=1024 (informational)")
    ap.add_argument("--cpu-sample-elems", type=int, default=1_600_000_000,
                    help="oracle sample: the longest prefix of the parameter list with at most this many elements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-zero3", action="store_true", help="skip the ZeRO-3 (one bucket per layer) leg")
    ap.add_argument("--no-graph", action="store_true", help="skip the leg that replays the step as a HIP graph")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="reduce rocprofv3 CSVs under DIR (trace/, FETCH_SIZE/, WRITE_SIZE/) to a text summary "
                         "on stdout and profiles/traffic.json, then exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summary")
    args = ap.parse_args()
    if args.summarize_profiles:
        print(summarize_profiles(args.summarize_profiles, WORKLOAD_IDS[args.config], args.profile_command), end="")
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU reduce-scatter/all-gather path is not implemented)", file=sys.stderr)
        sys.exit(2)
    import workloads as W

    w = W.workload(args.config)
    device = torch.device("cuda:0")
    ctx = setup(w, device)
    st = ctx[0]
    shard_sizes = [Z.zero_plan_param_info(st.plan, i).shard_size for i in range(st.n)]
    live = W.live_mask(w, 0)
    ab = algorithmic_bytes(w.numels, shard_sizes, live, w.nd)
    ne = stage_elements(ab)
    runs = {}
    for path in ("unfused", "fused"):
        ms_p, per_phase, launches, flag = run_gpu(w, ctx, path, args.steps, args.warmup)
        kernels = {}
        for p in PHASES[path]:
            kernels[p] = {"ms": round(per_phase[p], 4), "launches": launches[p], "bytes": ab[p],
                          "GBs": round(ab[p] / (per_phase[p] * 1e-3) / 1e9, 1),
                          "frac": round(ab[p] / (per_phase[p] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "elements": ne[p], "elem_per_s": round(ne[p] / (per_phase[p] * 1e-3), 1)}
        runs[path] = dict(ms=ms_p, kernels=kernels, launches=launches, flag=flag,
                          bytes=sum(ab[p] for p in PHASES[path]))
    ms, kernels, launches, flag = (runs["unfused"][k] for k in ("ms", "kernels", "launches", "flag"))
    step_bytes = runs["unfused"]["bytes"]
    fz = runs["fused"]
    fused = {"ms_per_step": round(fz["ms"], 4), "speedup": round(ms / fz["ms"], 3),
             "GBs": round(fz["bytes"] / (fz["ms"] * 1e-3) / 1e9, 1), "step_bytes": fz["bytes"],
             "elem_per_s": round(ab["shard_live"] / (fz["ms"] * 1e-3), 1), "overflow_flag": fz["flag"],
             "kernels": fz["kernels"]}
    graph = None
    if not args.no_graph:
        graph_ms = run_graph(w, ctx, args.steps, args.warmup)
        graph = {"ms_per_step": round(graph_ms, 4), "eager_ms_per_step": round(ms, 4),
                 "speedup": round(ms / graph_ms, 3)}
    zero3 = None
    if w.emulation == "full" and not args.no_zero3:
        zero3 = run_zero3(w, ctx, args.steps, args.warmup, device, graph=not args.no_graph)
    fk = fz["kernels"]["reduce_adam"]
    fused["roofline"] = {"bound": "hbm", "kernel": "reduce_adam", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "achieved": fk["GBs"], "frac": fk["frac"],
                         "traffic": measured_traffic("reduce_adam", WORKLOAD_IDS[args.config]),
                         "bytes_per_launch": fk["bytes"] // fk["launches"],
                         "avg_launch_ms": round(fk["ms"] / fk["launches"], 4)}
    dom = max(kernels, key=lambda p: kernels[p]["ms"])
    workload = WORKLOAD_IDS[args.config]
    traffic = measured_traffic(dom, workload)
    d = kernels[dom]
    out = {
        "metric": METRIC,
        "value": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config],
                   "workload_id": workload, "nd": w.nd, "rank": w.rank, "n_params": w.n,
                   "psi": int(sum(s * w.nd for s in shard_sizes)), "shard_elems": ab["shard_live"],
                   "n_buckets": launches["pack"],
                   "storage": ("bf16" if w.dtype == W.BF16 else "fp16") + " grads/params, fp32 state",
                   "emulation": w.emulation},
        "elem_per_s": round(ab["shard_live"] / (ms * 1e-3), 1),
        "grad_elem_per_s": round(ab["numel_live"] / (ms * 1e-3), 1),
        "step_bytes": step_bytes,
        "overflow_flag": flag,
        "kernels": kernels,
        "fused": fused,
        "zero3": zero3,
        "graph": graph,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(d["bytes"] / launches[dom] /
                                                                      (d["ms"] / launches[dom] * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d["frac"],
                     "traffic": traffic, "bytes_per_launch": d["bytes"] // launches[dom],
                     "avg_launch_ms": round(d["ms"] / launches[dom], 4)},
        "copy_reference_GBs": copy_reference(device),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.config == 2:
        log("[bench] timing the oracle on the host (cpu_baseline) ...")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_elems)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
