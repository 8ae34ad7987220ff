"""A whole Muon optimizer step over many matrices, on one device.

State lives in flat device buffers laid out micro-bucket by micro-bucket
(addresses planned once, views per step: the blog "Muon Optimizer + FSDP",
sections "Memory control" item 2 and "DBuffer").  Per micro-bucket the step
enqueues, on one stream (its lane's, below) and with no host
synchronisation:
    momentum (+ Nesterov) -> batched Newton-Schulz per unit shape -> apply
(the blog's recommended chunked-execution pseudocode, minus the all-to-all
exchanges, which one device does not need).  The momentum pass also leaves
the sums of squares of every 4096-element block of the update, from which the
Newton-Schulz call takes each matrix's Frobenius norm without reading the
update again (groups whose matrices do not lie on whole blocks read it).  The
Newton-Schulz input/output buffer holds one micro-bucket, so device memory
beyond the caller's state is cap-bounded: update buffer <= cap (full-byte
caps), its partials (8 bytes per 4096 elements), plus the context workspace
<= max over micro-buckets of the Newton-Schulz workspace.

Micro-buckets in flight (the blog, section "Memory control" item 3: start
with one bucket in flight, then try two): with inflight = k > 1 the step
keeps k lanes, each with its own update buffer, partials and context
workspace, and runs micro-bucket i on lane i % k: lane 0 on the caller's
stream, the others on side streams of default priority that wait for the
caller's stream at the start of the step and that it waits for at the end.
Micro-buckets touch disjoint parts of the state, and each lane runs its
micro-buckets in order, so the results are bit-identical for every k; what
changes is that one lane's launches can fill the CUs another lane's leave
idle (a launch's last, partial round of tiles, the epilogue bursts of short
contractions).  Device memory beyond the state grows by (k - 1) lanes.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from .api import SQ_BLOCK, Context, Plan, ns_params, sq_blocks


class MuonStep:
    def __init__(self, shapes: Sequence[Tuple[int, int, int]], device=None, lr: float = 0.02,
                 beta: float = 0.95, nesterov: bool = True, compute: str = "bf16",
                 grad_dtype: torch.dtype = torch.bfloat16, cap_bytes: int = 512 << 20,
                 cap_kind: str = "full", ns_steps: int = 5, keep_bf16_weights: bool = False,
                 weight_decay: float = 0.0, scale: float = 1.0, ns_method: str = "quintic",
                 ns_coeffs=None, norms_from_momentum: bool = True, ns_fuse: str = "auto",
                 inflight: int = 1):
        if inflight < 1:
            raise ValueError("inflight must be >= 1")
        self.inflight = inflight
        self.device = torch.device(device if device is not None else "cuda")
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.shapes = [tuple(s) for s in shapes]
        self.lr, self.beta, self.nesterov = lr, beta, nesterov
        self.weight_decay, self.scale = weight_decay, scale
        self.compute = compute
        self.cdtype = torch.bfloat16 if compute == "bf16" else torch.float32
        self.params = ns_params(steps=ns_steps, compute=compute, method=ns_method, coeffs=ns_coeffs,
                                fuse=ns_fuse)
        cus = torch.cuda.get_device_properties(self.device).multi_processor_count
        self.plan = Plan(self.shapes, cap_bytes, cap_kind, compute, compute_units=cus)

        # flat layout: the plan's element offsets (matrices in plan order)
        self.order: List[int] = [i for b in self.plan.buckets for i in b.indices]
        self.offset = [0] * len(self.shapes)
        for b in self.plan.buckets:
            for i, o in zip(b.indices, b.offsets):
                self.offset[i] = o
        self.numel = self.plan.total_elems
        self.max_bucket = max((b.numel for b in self.plan.buckets), default=0)
        self.norms_from_momentum = norms_from_momentum
        self.ctx = Context(self.device, self.plan.max_workspace)
        self._alloc_state(grad_dtype, keep_bf16_weights)

    def _alloc_state(self, grad_dtype: torch.dtype, keep_bf16_weights: bool):
        off, dev = self.numel, self.device
        self.grad = torch.zeros(off, dtype=grad_dtype, device=dev)
        self.momentum = torch.zeros(off, dtype=torch.float32, device=dev)
        self.master = torch.zeros(off, dtype=torch.float32, device=dev)
        self.weight_bf16 = torch.zeros(off, dtype=torch.bfloat16, device=dev) if keep_bf16_weights else None
        # per lane: context (workspace), update buffer, per-4096-element sums
        # of squares of the update from the momentum pass, micro-bucket views
        self.lanes: List[Tuple[Context, torch.Tensor, torch.Tensor, list]] = []
        for k in range(self.inflight):
            ctx = self.ctx if k == 0 else Context(dev, self.plan.max_workspace)
            upd = torch.empty(max(self.max_bucket, 1), dtype=self.cdtype, device=dev)
            sq = torch.empty(max(sq_blocks(self.max_bucket), 1), dtype=torch.float64, device=dev)
            self.lanes.append((ctx, upd, sq, self._bucket_work(upd)))
        _, self.update, self.sq, self._work = self.lanes[0]
        self._side = [torch.cuda.Stream(dev) for _ in range(self.inflight - 1)]
        self._ev_start = torch.cuda.Event()
        self._ev_end = [torch.cuda.Event() for _ in self._side]

    def _bucket_work(self, update: torch.Tensor):
        """Per micro-bucket: its element range and its Newton-Schulz calls,
        each with views of `update` (the micro-bucket laid out from its start)
        and the cached pointer arrays of those views.

        A per-head matrix (head_rows h < rows) is rows / h independent h x cols
        units, each a contiguous block of the row-major matrix, so the calls
        pass units rather than matrices: consecutive shape groups whose units
        have one shape and follow each other in memory become one call (the
        per-head q and k/v projections of a micro-bucket: one launch over all
        their heads instead of one per shape, with one partial round of tiles
        instead of one per call).  The units, and so the results, are the
        same.  The merged call needs no more workspace than the separate ones
        together, which the plan's per-micro-bucket figure already covers."""
        work = []
        pos = 0
        for b in self.plan.buckets:
            lo = b.elem_offset
            hi = lo + b.numel
            calls = []  # [unit rows, cols, unit offsets relative to lo]
            j = 0
            while j < len(b.indices):
                k = j
                while k < len(b.indices) and self.shapes[b.indices[k]] == self.shapes[b.indices[j]]:
                    k += 1
                r, c, h = self.shapes[b.indices[j]]
                ur = h if h else r
                units = [self.offset[i] - lo + q * ur * c for i in b.indices[j:k] for q in range(r // ur)]
                prev = calls[-1] if calls else None
                if prev is not None and (prev[0], prev[1]) == (ur, c) and units[0] == prev[2][-1] + ur * c:
                    prev[2].extend(units)
                else:
                    calls.append([ur, c, units])
                j = k
            groups = []
            for ur, c, units in calls:
                mats = [update[o:o + ur * c].view(ur, c) for o in units]
                # norms from the momentum partials when every unit of the call
                # starts on, and spans, whole 4096-element blocks
                whole = self.norms_from_momentum and (ur * c) % SQ_BLOCK == 0 and all(
                    o % SQ_BLOCK == 0 for o in units)
                groups.append((0, mats, self.ctx.pointer_arrays(mats), whole))
            work.append((lo, hi, groups, any(g[3] for g in groups)))
            pos = hi
        assert pos == self.numel
        return work

    def view(self, buf: torch.Tensor, i: int) -> torch.Tensor:
        """Matrix i of a flat state buffer (grad, momentum, master, weight_bf16)."""
        r, c, _ = self.shapes[i]
        return buf[self.offset[i]:self.offset[i] + r * c].view(r, c)

    def momentum_only(self, stream=None):
        """Momentum update of every matrix, without Newton-Schulz or apply
        (used to pre-fill momentum); the update output is discarded."""
        for lo, hi, _, _ in self._work:
            self.ctx.momentum_update(self.grad[lo:hi], self.momentum[lo:hi], self.update[:hi - lo],
                                     self.beta, self.nesterov, stream)

    def _run_bucket(self, grad, momentum, upd, sq, groups, want_sq, master, wb, stream, flag, ctx=None):
        """momentum -> Newton-Schulz per shape group -> apply, for one
        micro-bucket whose update buffer `upd` is laid out as in _bucket_work."""
        ctx = ctx if ctx is not None else self.ctx
        ctx.momentum_update(grad, momentum, upd, self.beta, self.nesterov, stream,
                            sq_partials=sq if want_sq else None)
        self._run_nsa(upd, sq, groups, master, wb, stream, flag, ctx)

    def _run_nsa(self, upd, sq, groups, master, wb, stream, flag, ctx=None):
        """Newton-Schulz per shape group, in place on `upd`, then the apply."""
        ctx = ctx if ctx is not None else self.ctx
        for h, mats, ptrs, whole in groups:
            ctx.newton_schulz(mats, None, h, self.params, flag, stream, _ptrs=ptrs,
                              sq=(sq, upd) if whole else None)
        ctx.apply(master, upd, self.lr, self.scale, self.weight_decay, wb, stream)

    def capture(self, nonfinite_flag: Optional[torch.Tensor] = None) -> "torch.cuda.CUDAGraph":
        """Record one whole step, every lane's launches included, into a HIP
        graph (stream capture through torch.cuda.CUDAGraph); replay() then
        runs it with no host work per launch.  Recording runs nothing.  The
        graph keeps what the step passed when it was recorded: lr, beta,
        scale and weight decay, and the state buffers' addresses (their
        contents are read at replay).  Per-kernel timing skips recorded
        launches.  Record again after changing a hyperparameter."""
        g = torch.cuda.CUDAGraph()
        cur = torch.cuda.current_stream(self.device)
        side = torch.cuda.Stream(self.device)
        side.wait_stream(cur)
        with torch.cuda.graph(g, stream=side):
            self.step(stream=side, nonfinite_flag=nonfinite_flag)
        cur.wait_stream(side)
        self._graph = g
        return g

    def replay(self):
        """Run the step recorded by capture() on the current stream."""
        if getattr(self, "_graph", None) is None:
            raise RuntimeError("no recorded step: call capture() first")
        self._graph.replay()

    @property
    def contexts(self) -> List[Context]:
        """The lanes' contexts (per-kernel timing is kept per context)."""
        return [lane[0] for lane in self.lanes]

    def step(self, stream=None, nonfinite_flag: Optional[torch.Tensor] = None):
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        if self._side:
            self._ev_start.record(main)
            for sd in self._side:
                sd.wait_event(self._ev_start)
        for i in range(len(self._work)):
            k = i % self.inflight
            ctx, upd, sq, work = self.lanes[k]
            lo, hi, groups, want_sq = work[i]
            st = main if k == 0 else self._side[k - 1]
            wb = self.weight_bf16[lo:hi] if self.weight_bf16 is not None else None
            self._run_bucket(self.grad[lo:hi], self.momentum[lo:hi], upd[:hi - lo], sq, groups, want_sq,
                             self.master[lo:hi], wb, st, nonfinite_flag, ctx)
        for sd, ev in zip(self._side, self._ev_end):
            ev.record(sd)
            main.wait_event(ev)
