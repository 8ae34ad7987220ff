"""The Muon step with its momentum in pinned host memory (host offload).

DeepSpeed PR "[Muon] CPU offload: pin the momentum and overlap the host
writeback": under optimizer offload every step copies each Muon gradient and
momentum to the accelerator, runs Newton-Schulz there, and copies the update
and the momentum back.  The PR's two changes are the momentum in pinned host
memory (section Motivation: pinned copies reach about 43 GB/s host-to-device
and 57 GB/s device-to-host where pageable ones ran near 10 GB/s) and the
writeback of batch i on a side stream while batch i+1 is gathered and
orthogonalised, with at most one batch computed and one in flight (section
Changes; blog "Muon Optimizer + FSDP", section "Memory control", item 3:
start with one bucket in flight, then two).

On one device this becomes a three-stream pipeline over the plan's
micro-buckets.  Host (pinned unless pin=False): the gradient (when
grads_on_host), the fp32 momentum, and, when update_to_host, the
orthogonalised update for a host-side consumer.  Device: the fp32 master
weights (the apply stays on the device), one Newton-Schulz workspace, and
`inflight` slots that each hold one micro-bucket's gradient, momentum,
update and sum-of-squares partials.  Micro-bucket i uses slot i % inflight:

    copy-in stream   waits until the slot's previous micro-bucket no longer
                     needs its gradient and momentum, then copies both in;
    caller's stream  waits for the copy-in (and until the slot's previous
                     update has been copied out), runs the momentum kernel,
                     then Newton-Schulz and the apply, with the resident
                     step's kernels on the resident step's buffer layout, so
                     every result is bit-identical;
    copy-out stream  copies the momentum back as soon as the momentum kernel
                     has written it, and the update once the apply is done.

The momentum leaves its slot while Newton-Schulz still runs, so with two
slots the copy-in never waits for a whole copy-out: both directions stay
busy on the DMA engines while micro-bucket i computes, and the step is
bounded by the larger of the two transfers.  With one slot every stage is
serialised.  Ordering uses device-side waits on events (hipStreamWaitEvent).
The PR waited on the host instead because on its accelerator a
cross-stream wait serialised the two queues; HIP streams do not.  The
step's first copy-in waits for the caller's stream, and at the end the
caller's stream waits for the last copy-out: work enqueued before step() is
ordered before it, and once the caller's stream has been synchronised the
host momentum and update are complete.  Every stream has the default
priority.
"""
from __future__ import annotations

from typing import Dict, List, NamedTuple, Optional, Sequence, Tuple

import torch

from .api import sq_blocks
from .muon_step import MuonStep

# op kinds and the stream each runs on: the copy-in stream, the caller's
# stream (momentum kernel, then Newton-Schulz + apply), the copy-out stream
KINDS = ("h2d", "mom", "nsa", "d2h_mom", "d2h_upd")
STREAM = {"h2d": "h2d", "mom": "main", "nsa": "main", "d2h_mom": "d2h", "d2h_upd": "d2h"}


class Op(NamedTuple):
    kind: str                      # one of KINDS
    bucket: int
    slot: int
    waits: Tuple[Tuple[str, int], ...]  # (kind, bucket) on other streams this op follows


def offload_schedule(n: int, slots: int) -> List[Op]:
    """Issue order of one offloaded step over n micro-buckets and `slots`
    device slots (micro-bucket i in slot i % slots).  Ops run on the stream
    STREAM[kind] in this order; `waits` lists the cross-stream dependencies:
      h2d i      after mom i-slots and d2h_mom i-slots (the slot's gradient
                 and momentum are free again);
      mom i      after h2d i and d2h_upd i-slots (its update buffer is free);
      d2h_mom i  after mom i;  d2h_upd i  after nsa i.
    The copy-in runs slots - 1 micro-buckets ahead of the compute."""
    if slots < 1:
        raise ValueError("slots must be >= 1")
    ops: List[Op] = []

    def h2d(i):
        prev = (("mom", i - slots), ("d2h_mom", i - slots)) if i >= slots else ()
        ops.append(Op("h2d", i, i % slots, prev))

    for i in range(min(slots - 1, n)):
        h2d(i)
    for i in range(n):
        s = i % slots
        if i + slots - 1 < n:
            h2d(i + slots - 1)
        ops.append(Op("mom", i, s, (("h2d", i),) + ((("d2h_upd", i - slots),) if i >= slots else ())))
        ops.append(Op("d2h_mom", i, s, (("mom", i),)))
        ops.append(Op("nsa", i, s, ()))
        ops.append(Op("d2h_upd", i, s, (("nsa", i),)))
    return ops


class _Slot(NamedTuple):
    grad: Optional[torch.Tensor]
    mom: torch.Tensor
    upd: torch.Tensor
    sq: torch.Tensor
    work: list


class MuonOffloadStep(MuonStep):
    """MuonStep with the momentum (and the gradient) in host memory.

    inflight: device slots (1 = serialised, 2 = one micro-bucket computed
    while the next is copied in and the previous copied out).  pin: pinned
    host buffers (page-locked, allocated as such) or pageable ones.
    grads_on_host: the gradient is a host buffer copied in per micro-bucket
    (else a device buffer, as in MuonStep).  update_to_host: copy the
    orthogonalised update back to `update_host` as well.  timing: record
    events around every copy and compute stage (copy_stats())."""

    def __init__(self, shapes: Sequence[Tuple[int, int, int]], device=None, inflight: int = 2,
                 pin: bool = True, grads_on_host: bool = True, update_to_host: bool = True,
                 timing: bool = False, **kw):
        if inflight < 1:
            raise ValueError("inflight must be >= 1")
        self.pin = pin
        self.grads_on_host, self.update_to_host = grads_on_host, update_to_host
        self.timing = timing
        super().__init__(shapes, device, inflight=inflight, **kw)

    def _alloc_state(self, grad_dtype: torch.dtype, keep_bf16_weights: bool):
        n, dev = self.numel, self.device

        def host(dtype):
            return torch.zeros(n, dtype=dtype, pin_memory=self.pin)

        self.grad = host(grad_dtype) if self.grads_on_host else torch.zeros(n, dtype=grad_dtype, device=dev)
        self.momentum = host(torch.float32)
        self.update_host = host(self.cdtype) if self.update_to_host else None
        self.master = torch.zeros(n, dtype=torch.float32, device=dev)
        self.weight_bf16 = torch.zeros(n, dtype=torch.bfloat16, device=dev) if keep_bf16_weights else None
        mb = max(self.max_bucket, 1)
        self.slots: List[_Slot] = []
        for _ in range(self.inflight):
            g = torch.empty(mb, dtype=grad_dtype, device=dev) if self.grads_on_host else None
            upd = torch.empty(mb, dtype=self.cdtype, device=dev)
            self.slots.append(_Slot(g, torch.empty(mb, dtype=torch.float32, device=dev), upd,
                                    torch.empty(max(sq_blocks(mb), 1), dtype=torch.float64, device=dev),
                                    self._bucket_work(upd)))
        self.update, self.sq, self._work = self.slots[0].upd, self.slots[0].sq, self.slots[0].work
        # one context: every Newton-Schulz call runs on the caller's stream
        self.lanes = [(self.ctx, self.update, self.sq, self._work)]
        self.streams = {"h2d": torch.cuda.Stream(dev), "d2h": torch.cuda.Stream(dev)}
        self.schedule = offload_schedule(len(self.plan.buckets), self.inflight)
        # one event per (kind, slot), re-recorded for each micro-bucket that
        # uses the slot: every wait on it is issued before the next record
        self._ev: Dict[str, List[torch.cuda.Event]] = {
            k: [torch.cuda.Event() for _ in range(self.inflight)] for k in KINDS}
        self._ev_start = torch.cuda.Event()
        self._tev: List[Tuple[str, int, torch.cuda.Event, torch.cuda.Event]] = []  # kind, bytes

    def device_bytes(self) -> int:
        """Device memory beyond the master weights: the slots (inflight x one
        micro-bucket's gradient, momentum, update and partials) and the
        Newton-Schulz workspace."""
        per = sum(t.numel() * t.element_size() for t in (self.slots[0].mom, self.slots[0].upd, self.slots[0].sq))
        if self.slots[0].grad is not None:
            per += self.slots[0].grad.numel() * self.slots[0].grad.element_size()
        return self.inflight * per + self.plan.max_workspace

    def momentum_only(self, stream=None):
        """Momentum of every matrix through the same pipeline, without
        Newton-Schulz or apply (used to pre-fill the momentum)."""
        self._run(stream, None, momentum_only=True)

    def step(self, stream=None, nonfinite_flag: Optional[torch.Tensor] = None):
        self._run(stream, nonfinite_flag, momentum_only=False)

    def _timed(self, kind: str, nbytes: int, stream, fn):
        if not self.timing:
            fn()
            return
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        self._tev.append((kind, nbytes, a, b))

    def _run(self, stream, flag, momentum_only: bool):
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        streams = {"main": main, **self.streams}
        self._ev_start.record(main)
        self.streams["h2d"].wait_event(self._ev_start)
        self.streams["d2h"].wait_event(self._ev_start)
        buckets = self.plan.buckets
        for op in self.schedule:
            b = buckets[op.bucket]
            lo, hi = b.elem_offset, b.elem_offset + b.numel
            n = hi - lo
            sl = self.slots[op.slot]
            st = streams[STREAM[op.kind]]
            for kind, j in op.waits:
                st.wait_event(self._ev[kind][j % self.inflight])
            fn, nbytes = None, 0
            if op.kind == "h2d":
                nbytes = n * (4 + (sl.grad.element_size() if sl.grad is not None else 0))

                def fn():
                    if sl.grad is not None:
                        sl.grad[:n].copy_(self.grad[lo:hi], non_blocking=True)
                    sl.mom[:n].copy_(self.momentum[lo:hi], non_blocking=True)
            elif op.kind == "mom":
                grad = sl.grad[:n] if sl.grad is not None else self.grad[lo:hi]
                _, _, groups, want_sq = sl.work[op.bucket]
                sq = sl.sq if want_sq and not momentum_only else None

                def fn():
                    self.ctx.momentum_update(grad, sl.mom[:n], sl.upd[:n], self.beta, self.nesterov, st,
                                             sq_partials=sq)
            elif op.kind == "nsa" and not momentum_only:
                _, _, groups, _ = sl.work[op.bucket]
                wb = self.weight_bf16[lo:hi] if self.weight_bf16 is not None else None

                def fn():
                    self._run_nsa(sl.upd[:n], sl.sq, groups, self.master[lo:hi], wb, st, flag)
            elif op.kind == "d2h_mom":
                nbytes = 4 * n

                def fn():
                    self.momentum[lo:hi].copy_(sl.mom[:n], non_blocking=True)
            elif op.kind == "d2h_upd" and self.update_host is not None and not momentum_only:
                nbytes = n * sl.upd.element_size()

                def fn():
                    self.update_host[lo:hi].copy_(sl.upd[:n], non_blocking=True)
            if fn is not None:
                with torch.cuda.stream(st):
                    self._timed(op.kind, nbytes, st, fn)
            # recorded even for a stage with nothing to do, so that every
            # wait names this micro-bucket's record
            self._ev[op.kind][op.slot].record(st)
        if self.schedule:
            main.wait_event(self._ev["d2h_upd"][self.schedule[-1].slot])

    def copy_stats(self, reset: bool = True) -> dict:
        """Per stage (h2d, compute, d2h): total ms, bytes and timed ops since
        the last reset (synchronises on the recorded events)."""
        stage = {"h2d": "h2d", "mom": "compute", "nsa": "compute", "d2h_mom": "d2h", "d2h_upd": "d2h"}
        out = {k: {"ms": 0.0, "bytes": 0, "ops": 0} for k in ("h2d", "compute", "d2h")}
        for kind, nbytes, a, b in self._tev:
            b.synchronize()
            o = out[stage[kind]]
            o["ms"] += a.elapsed_time(b)
            o["ops"] += 1
            o["bytes"] += nbytes
        if reset:
            self._tev = []
        return out
