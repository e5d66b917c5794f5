"""One rank's shard step, driven through the C ABI: pack -> reduce (+ overflow flag) -> Adam ->
unpack (or pack with the input check -> fused reduce + Adam -> unpack), the order of the ZeRO-1
sequence on the briefia.fr page ("ZeRO-1 : Partitionnement des états de l'optimiseur": gradients
synchronised, own partition stepped, parameters all-gathered) with the ZeRO-2 reduce-scatter of
the ColossalAI "low level zero" issue (BWD).

This class only allocates the rank's device buffers (sizes read from the plan) and issues the
entry points in order on one stream; every element of work runs in the HIP kernels.
Zero3Schedule issues ZeRO-3's per-layer gathers and reduce-scatters over a plan with one bucket
per layer."""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import torch

from . import _binding as B


class ShardStep:
    def __init__(self, numels: Sequence[int], nd: int, rank: int, bucket_bytes: int, dtype: int, device="cuda",
                 groups: Optional[Sequence[int]] = None):
        """groups: one id per parameter (a bucket never spans a change of id), e.g. the layer
        index, giving ZeRO-3's one bucket per layer with bucket_bytes = 0."""
        self.device = torch.device(device)
        self.plan = (B.zero_plan_create(numels, nd, rank, bucket_bytes, dtype) if groups is None else
                     B.zero_plan_create_grouped(numels, groups, nd, rank, bucket_bytes, dtype))
        self.summary = B.zero_plan_get_summary(self.plan)
        s = self.summary
        self.nd, self.rank, self.dtype = nd, rank, dtype
        self.n = int(s.n_params)
        self.buckets = [B.zero_plan_bucket_info(self.plan, b) for b in range(int(s.n_buckets))]
        S = int(s.shard_numel)
        f32 = dict(dtype=torch.float32, device=self.device)
        self.p32 = torch.zeros(S, **f32)
        self.m = torch.zeros(S, **f32)
        self.v = torch.zeros(S, **f32)
        self.g32 = torch.zeros(S, **f32)
        self.steps = torch.zeros(self.n, dtype=torch.int32, device=self.device)
        self.live = torch.ones(self.n, dtype=torch.uint8, device=self.device)
        self.flag = torch.zeros(1, dtype=torch.int32, device=self.device)
        # this rank's packed gradient buckets and the all-gather arena share one layout:
        # bucket b's [Nd][L_b] block starts at block_offset
        self.packed = torch.zeros(int(s.arena_numel), dtype=torch.int16, device=self.device)
        self.arena = torch.zeros(int(s.arena_numel), dtype=torch.int16, device=self.device)
        self.scaler: Optional[torch.Tensor] = None  # device zero_loss_scaler, once enabled

    def enable_loss_scaler(self, scale: float, growth_interval: int = 2000, growth_factor: float = 2.0,
                           backoff_factor: float = 0.5, min_scale: float = 1.0, max_scale: float = 2.0 ** 24,
                           stream=None) -> None:
        """Dynamic loss scaling on the device; adam()/reduce_adam() then divide the gradient
        multiplier by the current scale, and update_loss_scale() applies the rule after a step."""
        self.scaler = torch.zeros(B.LOSS_SCALER_BYTES // 4, dtype=torch.int32, device=self.device)
        cfg = B.zero_loss_scaler(scale, 0, growth_interval, growth_factor, backoff_factor, min_scale, max_scale, 0)
        B.zero_loss_scaler_init(cfg, self.scaler, stream)

    def update_loss_scale(self, stream=None) -> None:
        B.zero_loss_scaler_update(self.flag, self.scaler, stream)

    # -- views ---------------------------------------------------------------------------
    def block(self, buf: torch.Tensor, b: int) -> torch.Tensor:
        """Bucket b's [Nd][L_b] block of an arena-layout buffer (ValueError if buf is shorter
        than the arena)."""
        bk = self.buckets[b]
        end = bk.block_offset + self.nd * bk.row_stride
        if buf.numel() < end:
            raise ValueError(f"buffer of {buf.numel()} elements is shorter than bucket {b}'s block end {end}")
        return buf[bk.block_offset:end]

    def own_row(self, buf: torch.Tensor, b: int, k: Optional[int] = None) -> torch.Tensor:
        bk = self.buckets[b]
        k = self.rank if k is None else k
        start = bk.block_offset + k * bk.row_stride
        if not 0 <= k < self.nd or buf.numel() < start + bk.row_stride:
            raise ValueError(f"row {k} of bucket {b} does not fit a buffer of {buf.numel()} elements")
        return buf[start:start + bk.row_stride]

    # -- the steps -----------------------------------------------------------------------
    def init_master(self, src_ptrs: torch.Tensor, src_dtype: int = 0, stream=None) -> None:
        B.zero_shard_init(self.plan, src_ptrs, src_dtype, self.p32, stream)

    def pack(self, grad_ptrs: torch.Tensor, out: Optional[torch.Tensor] = None, check: bool = False,
             stream=None) -> None:
        """check=True: also OR this rank's input verdict into self.flag (the fused path's check)."""
        out = self.packed if out is None else out
        for b in range(len(self.buckets)):
            if check:
                B.zero_pack_bucket_check(self.plan, b, grad_ptrs, self.block(out, b), self.flag, stream)
            else:
                B.zero_pack_bucket(self.plan, b, grad_ptrs, self.block(out, b), stream)

    def reduce(self, rows_of: Callable[[int], tuple], fused_check: bool = True, stream=None) -> None:
        """rows_of(b) -> (tensor starting at row 0 of bucket b, row stride in elements)."""
        for b in range(len(self.buckets)):
            rows, stride = rows_of(b)
            B.zero_reduce_shard(self.plan, b, rows, stride, self.live, self.g32,
                                self.flag if fused_check else None, stream)

    def overflow_check(self, stream=None) -> None:
        B.zero_overflow_check(self.plan, self.g32, self.live, self.flag, stream)

    def adam(self, lr: float, beta1: float, beta2: float, eps: float, grad_scale: float, use_flag: bool = True,
             stream=None) -> None:
        B.zero_adam_step(self.plan, self.g32, self.p32, self.m, self.v, self.live, self.steps, lr, beta1, beta2,
                         eps, grad_scale, self.flag if use_flag else None, self.arena, stream, loss_scaler=self.scaler)

    def reduce_adam(self, rows_of: Callable[[int], tuple], lr: float, beta1: float, beta2: float, eps: float,
                    grad_scale: float, use_flag: bool = True, stream=None) -> None:
        """The fused path after pack(check=True): step sizes once, then per bucket the sum of its
        rows goes straight into the Adam update (self.g32 is not written)."""
        flag = self.flag if use_flag else None
        B.zero_adam_prepare(self.plan, self.live, self.steps, lr, beta1, beta2, eps, grad_scale, flag, stream,
                            loss_scaler=self.scaler)
        for b in range(len(self.buckets)):
            rows, stride = rows_of(b)
            B.zero_reduce_adam_bucket(self.plan, b, rows, stride, self.live, self.p32, self.m, self.v, flag,
                                      self.arena, stream)

    def unpack(self, param_ptrs: torch.Tensor, src: Optional[torch.Tensor] = None, stream=None) -> None:
        src = self.arena if src is None else src
        for b in range(len(self.buckets)):
            B.zero_unpack(self.plan, b, self.block(src, b), param_ptrs, stream)

    def close(self) -> None:
        self.plan.close()


class Zero3Schedule:
    """ZeRO-3's per-layer parameter traffic over a ShardStep whose plan has one bucket per
    layer (groups = layer index, bucket_bytes = 0), following the llm-engineer "ZeRO-3" card:
    before a layer runs, its parameters are all-gathered into a scratch buffer, used and freed;
    the forward pass gathers layers 0, 1, ..., L-1, the backward pass keeps the last layer and
    gathers L-2, ..., 0 again (the 0 -> 1 -> 2 -> 1 -> 0 order for three layers); each layer's
    gradients are reduce-scattered (pack + reduce) as soon as its backward has run.

    The gather of layer l is zero_unpack of bucket l from the all-gather block (the Nd ranks'
    rows of that layer).  Without prefetch its destination is one scratch buffer sized for the
    largest layer, so at most one layer's full parameters exist at a time, and everything runs
    in order on the caller's stream.  With batch=k the layers go k at a time, in k scratch slots
    (k layers' full parameters at a time).

    With prefetch=True the gathers run on a second stream into two scratch buffers (layer l in
    buffer l % 2), so the gather of the next layer overlaps the use of the current one and, in
    the backward pass, its pack and reduce.  Events order the two streams: a gather waits until
    the caller's stream has finished using the buffer's previous layer, a layer's use waits
    for its gather, and each pass starts by waiting for the caller's stream (Adam's writes to
    the all-gather block included) and ends with the caller's stream waiting for the gathers,
    so a pass can also be captured into a graph.  At most two layers' parameters exist at a
    time.  `use` callbacks run with the caller's stream current."""

    def __init__(self, st: ShardStep, prefetch: bool = False, fused: bool = False, batch: int = 1):
        """fused=True (one stream only): each backward step is one zero_z3_step launch -- the
        reduce of layer l + 1, the pack of layer l and the gather of layer l - 1 share a launch --
        instead of three launches per layer.  batch=k (fused only): every launch handles k
        consecutive layers -- the forward pass gathers layers [l, l + k) together, a backward
        step packs [l, l + k), gathers [l - k, l) and reduces [l + k, l + 2k) -- so that k layers
        share one launch tail; the scratch then holds k layers (layer l at slot l mod k)."""
        if prefetch and fused:
            raise ValueError("the fused backward runs on one stream (prefetch=False)")
        if not 1 <= batch <= B.Z3_MAX_BUCKETS:
            raise ValueError(f"batch must be in 1..{B.Z3_MAX_BUCKETS}")
        if batch > 1 and not fused:
            raise ValueError("batches of layers need the fused schedule (fused=True)")
        self.st = st
        self.prefetch = prefetch
        self.fused = fused
        self.batch = batch
        nb = len(st.buckets)
        infos = [B.zero_plan_param_info(st.plan, i) for i in range(st.n)]
        self.layers = [list(range(int(bk.first_param), int(bk.first_param + bk.n_params))) for bk in st.buckets]
        self.numel = [[int(infos[i].numel) for i in params] for params in self.layers]
        biggest = max((sum(x) for x in self.numel), default=0)
        # each parameter 16-byte aligned inside the scratch (the unpack's wide path)
        per = [sum((x + 7) // 8 * 8 for x in xs) for xs in self.numel]
        need = max(per + [biggest, 8])
        nbuf = 2 if prefetch else batch
        self.buffer_numel = need
        self.scratch = torch.zeros(nbuf * need, dtype=torch.int16, device=st.device)
        self.views, self.tables = [], []
        for lid in range(nb):
            views, pos = [], (lid % nbuf) * need
            for x in self.numel[lid]:
                views.append(self.scratch[pos:pos + x])
                pos += (x + 7) // 8 * 8
            full = [None] * st.n
            for i, v in zip(self.layers[lid], views):
                full[i] = v
            self.views.append(views)
            self.tables.append(B.ptr_table(full, device=st.device))
        # batches of layers [lo, hi): one destination table per batch
        self.batches = [(lo, min(lo + batch, nb)) for lo in range(0, nb, batch)]
        self.batch_tables = []
        for lo, hi in self.batches:
            if hi - lo == 1:
                self.batch_tables.append(self.tables[lo])
                continue
            full = [None] * st.n
            for lid in range(lo, hi):
                for i, v in zip(self.layers[lid], self.views[lid]):
                    full[i] = v
            self.batch_tables.append(B.ptr_table(full, device=st.device))
        self.order: list = []  # layers in the order they were gathered
        if prefetch:
            self.side = torch.cuda.Stream(device=st.device)
            self.ready = [torch.cuda.Event() for _ in range(nb)]
            self.free = [torch.cuda.Event(), torch.cuda.Event()]
            self.fork_ev, self.join_ev = torch.cuda.Event(), torch.cuda.Event()

    def gather(self, lid: int, src: Optional[torch.Tensor] = None, stream=None) -> list:
        """All-gather layer lid's parameters (the unpack of its bucket) into its scratch buffer;
        returns one view per parameter, valid until that buffer's next gather."""
        st = self.st
        src = st.arena if src is None else src
        B.zero_unpack(st.plan, lid, st.block(src, lid), self.tables[lid], stream)
        self.order.append(lid)
        return self.views[lid]

    # -- two-stream helpers (prefetch) -------------------------------------------------------

    def _main(self, stream) -> torch.cuda.Stream:
        if stream is None:
            return torch.cuda.current_stream(self.st.device)
        if isinstance(stream, torch.cuda.Stream):
            return stream
        return torch.cuda.ExternalStream(int(stream), device=self.st.device)

    def _fork(self, main) -> None:
        self.fork_ev.record(main)
        self.side.wait_event(self.fork_ev)
        self._recorded = [False, False]  # free[b] recorded in this pass

    def _join(self, main) -> None:
        self.join_ev.record(self.side)
        main.wait_event(self.join_ev)

    def _gather_side(self, lid: int) -> None:
        buf = lid % 2
        if self._recorded[buf]:
            self.side.wait_event(self.free[buf])  # the buffer's previous layer is no longer used
        self.gather(lid, stream=self.side)
        self.ready[lid].record(self.side)

    def _use(self, main, lid: int, use) -> None:
        if use is not None:
            with torch.cuda.stream(main):
                use(lid, self.views[lid])
        self.free[lid % 2].record(main)
        self._recorded[lid % 2] = True

    # -- passes --------------------------------------------------------------------------------

    def forward(self, use: Optional[Callable[[int, list], None]] = None, stream=None) -> None:
        if self.batch > 1:
            st = self.st
            for j, (lo, hi) in enumerate(self.batches):
                B.zero_z3_step(st.plan, gather_b0=lo, gathered=[st.block(st.arena, l) for l in range(lo, hi)],
                               param_ptrs=self.batch_tables[j], stream=stream)
                self.order.extend(range(lo, hi))
                if use is not None:
                    for lid in range(lo, hi):
                        use(lid, self.views[lid])
            return
        if not self.prefetch:
            for lid in range(len(self.layers)):
                params = self.gather(lid, stream=stream)
                if use is not None:
                    use(lid, params)
            return
        main = self._main(stream)
        self._fork(main)
        for lid in range(len(self.layers)):
            self._gather_side(lid)
            main.wait_event(self.ready[lid])
            self._use(main, lid, use)
        self._join(main)

    def backward(self, grads_of: Callable[[int], torch.Tensor], rows_of: Callable[[int], tuple],
                 use: Optional[Callable[[int, list], None]] = None, check: bool = False,
                 out: Optional[torch.Tensor] = None, stream=None) -> None:
        """grads_of(l): pointer table of this rank's gradients (entries of layer l used);
        rows_of(l): (rows of bucket l from the Nd ranks, row stride) for the reduce-scatter;
        out: where the packed gradient blocks go (arena layout; default st.packed)."""
        st = self.st
        out = st.packed if out is None else out
        last = len(self.layers) - 1
        if self.fused:
            self._backward_fused(grads_of, rows_of, use, check, out, stream)
            return
        main = self._main(stream) if self.prefetch else stream
        if self.prefetch:
            self._fork(main)  # the last layer is still in its buffer from the forward pass
        for lid in range(last, -1, -1):
            if not self.prefetch:
                params = self.views[lid] if lid == last else self.gather(lid, stream=stream)
                if use is not None:
                    use(lid, params)
            else:
                if lid != last:
                    main.wait_event(self.ready[lid])
                if lid > 0:
                    self._gather_side(lid - 1)  # the next layer's gather overlaps this layer's work
                self._use(main, lid, use)
            if check:
                B.zero_pack_bucket_check(st.plan, lid, grads_of(lid), st.block(out, lid), st.flag, main)
            else:
                B.zero_pack_bucket(st.plan, lid, grads_of(lid), st.block(out, lid), main)
            rows, stride = rows_of(lid)
            B.zero_reduce_shard(st.plan, lid, rows, stride, st.live, st.g32, st.flag, main)
        if self.prefetch:
            self._join(main)

    def _backward_fused(self, grads_of, rows_of, use, check, out, stream) -> None:
        """Batches of layers J-1 .. 0 (one layer each unless batch > 1); before step j's launch,
        batch j's parameters are in the scratch (the last batch's since the forward pass) and
        `use` runs on its layers, last first; the launch then packs batch j's gradients
        (grads_of(lo) must name those of the whole batch [lo, hi)), gathers batch j - 1 into
        the scratch and reduces batch j + 1 (packed one step earlier).  A last launch reduces
        batch 0."""
        st = self.st
        J = len(self.batches)
        for j in range(J - 1, -2, -1):
            if j >= 0 and use is not None:
                lo, hi = self.batches[j]
                for lid in range(hi - 1, lo - 1, -1):
                    use(lid, self.views[lid])
            kw = {}
            if j + 1 < J:
                lo, hi = self.batches[j + 1]
                rs = [rows_of(b) for b in range(lo, hi)]
                kw.update(reduce_b0=lo, rows=[r for r, _ in rs], row_strides=[x for _, x in rs], live=st.live,
                          g32=st.g32)
            if j >= 0:
                lo, hi = self.batches[j]
                kw.update(pack_b0=lo, grad_ptrs=grads_of(lo), packed=[st.block(out, b) for b in range(lo, hi)],
                          check=check)
            if j >= 1:
                lo, hi = self.batches[j - 1]
                kw.update(gather_b0=lo, gathered=[st.block(st.arena, b) for b in range(lo, hi)],
                          param_ptrs=self.batch_tables[j - 1])
            B.zero_z3_step(st.plan, flag=st.flag, stream=stream, **kw)
            if j >= 1:
                self.order.extend(range(hi - 1, lo - 1, -1))
