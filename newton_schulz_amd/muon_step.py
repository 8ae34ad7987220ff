"""A whole Muon optimizer step over many matrices, on one device.

State lives in flat device buffers laid out micro-bucket by micro-bucket
(addresses planned once, views per step: the blog "Muon Optimizer + FSDP",
sections "Memory control" item 2 and "DBuffer").  Per micro-bucket the step
enqueues, on one stream and with no host synchronisation:
    momentum (+ Nesterov) -> batched Newton-Schulz per shape group -> apply
(the blog's recommended chunked-execution pseudocode, minus the all-to-all
exchanges, which one device does not need).  The momentum pass also leaves
the sums of squares of every 4096-element block of the update, from which the
Newton-Schulz call takes each matrix's Frobenius norm without reading the
update again (groups whose matrices do not lie on whole blocks read it).  The
Newton-Schulz input/output buffer holds one micro-bucket, so device memory
beyond the caller's state is cap-bounded: update buffer <= cap (full-byte
caps), its partials (8 bytes per 4096 elements), plus the context workspace
<= max over micro-buckets of the Newton-Schulz workspace.
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
                 ns_coeffs=None, norms_from_momentum: bool = True, ns_fuse: str = "auto"):
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
        self.update = torch.empty(max(self.max_bucket, 1), dtype=self.cdtype, device=dev)
        # per-4096-element sums of squares of the update, from the momentum pass
        self.sq = torch.empty(max(sq_blocks(self.max_bucket), 1), dtype=torch.float64, device=dev)
        self._work = self._bucket_work(self.update)

    def _bucket_work(self, update: torch.Tensor):
        """Per micro-bucket: its element range and its shape groups, each with
        views of `update` (the micro-bucket laid out from its start) and the
        cached pointer arrays of those views."""
        work = []
        pos = 0
        for b in self.plan.buckets:
            lo = b.elem_offset
            hi = lo + b.numel
            groups = []
            j = 0
            while j < len(b.indices):
                k = j
                while k < len(b.indices) and self.shapes[b.indices[k]] == self.shapes[b.indices[j]]:
                    k += 1
                r, c, h = self.shapes[b.indices[j]]
                rel = [self.offset[i] - lo for i in b.indices[j:k]]
                mats = [update[o:o + r * c].view(r, c) for o in rel]
                # norms from the momentum partials when every unit of the group
                # starts on, and spans, whole 4096-element blocks
                unit = (h if h else r) * c
                whole = self.norms_from_momentum and unit % SQ_BLOCK == 0 and all(
                    o % SQ_BLOCK == 0 for o in rel)
                groups.append((h, mats, self.ctx.pointer_arrays(mats), whole))
                j = k
            work.append((lo, hi, groups, any(g[3] for g in groups)))
            pos = hi
        assert pos == self.numel
        return work

    def _uview(self, off: int, r: int, c: int) -> torch.Tensor:
        return self.update[off:off + r * c].view(r, c)

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

    def _run_bucket(self, grad, momentum, upd, sq, groups, want_sq, master, wb, stream, flag):
        """momentum -> Newton-Schulz per shape group -> apply, for one
        micro-bucket whose update buffer `upd` is laid out as in _bucket_work."""
        self.ctx.momentum_update(grad, momentum, upd, self.beta, self.nesterov, stream,
                                 sq_partials=sq if want_sq else None)
        self._run_nsa(upd, sq, groups, master, wb, stream, flag)

    def _run_nsa(self, upd, sq, groups, master, wb, stream, flag):
        """Newton-Schulz per shape group, in place on `upd`, then the apply."""
        for h, mats, ptrs, whole in groups:
            self.ctx.newton_schulz(mats, None, h, self.params, flag, stream, _ptrs=ptrs,
                                   sq=(sq, upd) if whole else None)
        self.ctx.apply(master, upd, self.lr, self.scale, self.weight_decay, wb, stream)

    def step(self, stream=None, nonfinite_flag: Optional[torch.Tensor] = None):
        for lo, hi, groups, want_sq in self._work:
            wb = self.weight_bf16[lo:hi] if self.weight_bf16 is not None else None
            self._run_bucket(self.grad[lo:hi], self.momentum[lo:hi], self.update[:hi - lo], self.sq,
                             groups, want_sq, self.master[lo:hi], wb, stream, nonfinite_flag)
