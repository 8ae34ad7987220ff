"""Python binding of libmuon: argument marshalling only.

Every step of the optimizer runs in the HIP kernels behind include/muon.h;
PyTorch supplies device memory and the current HIP stream.  When libmuon.so
is missing the calls raise instead of falling back to any other code.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import MUON_BF16, MUON_CAP_FULL_BYTES, MUON_CAP_WORKSPACE, MUON_F32, NsParams, Shape


class MuonError(RuntimeError):
    def __init__(self, status: int, msg: str = ""):
        lib = _lib.load()
        text = lib.muon_status_string(status).decode()
        super().__init__(f"libmuon status {status} ({text}){': ' + msg if msg else ''}")
        self.status = status


_DT = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; libmuon takes float32 or bfloat16")
    return _DT[t.dtype]


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t: torch.Tensor, name: str, device: torch.device):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


NS_FUSE = {"auto": 0, "off": 1, "on": 2}
SQ_BLOCK = 4096  # MUON_SQ_BLOCK
NS_METHODS = {"quintic": 0, "gram": 1}


def minimax_coeffs(steps: int, lo: float = 1e-3, margin: float = 0.05) -> Tuple[list, float]:
    """Per-iteration (a, b, c) rows from libmuon's muon_ns_minimax_coeffs and
    the bound E after the last one (every singular value of X_0 in [lo, 1]
    ends in [1 - E, 1 + E] in exact arithmetic)."""
    lib = _lib.load()
    out = (ctypes.c_float * (3 * steps))()
    bound = ctypes.c_double()
    st = lib.muon_ns_minimax_coeffs(steps, lo, margin, out, ctypes.byref(bound))
    if st != _lib.MUON_OK:
        raise MuonError(st, "muon_ns_minimax_coeffs")
    return [tuple(out[3 * k:3 * k + 3]) for k in range(steps)], bound.value


def ns_params(steps: int = 5, a: float = 3.4445, b: float = -4.7750, c: float = 2.0315,
              eps: float = 1e-7, compute: str = "bf16", method: str = "quintic",
              fuse: str = "auto", coeffs=None, lo: float = 1e-3,
              margin: float = 0.05) -> NsParams:
    """Newton-Schulz parameters.  coeffs: None (the fixed a, b, c), "minimax"
    (libmuon's per-iteration schedule for `lo`, `margin`), or `steps` rows of
    (a, b, c).  The returned structure keeps its coefficient table alive."""
    p = NsParams(steps, a, b, c, eps, MUON_BF16 if compute == "bf16" else MUON_F32,
                 NS_METHODS[method], NS_FUSE[fuse], None)
    if coeffs is not None:
        if isinstance(coeffs, str) and coeffs != "minimax":
            raise ValueError(f"unknown coefficient schedule {coeffs!r}")
        rows = minimax_coeffs(steps, lo, margin)[0] if isinstance(coeffs, str) else coeffs
        flat = [float(v) for r in rows for v in r]
        if len(flat) != 3 * steps:
            raise ValueError("coeffs must hold `steps` rows of (a, b, c)")
        table = (ctypes.c_float * len(flat))(*flat)
        p.coeffs = ctypes.cast(table, ctypes.POINTER(ctypes.c_float))
        p._table = table  # owned by the structure for as long as it lives
    return p


def sq_blocks(numel: int) -> int:
    """Sum-of-squares partials a momentum pass over `numel` elements writes."""
    return (int(numel) + SQ_BLOCK - 1) // SQ_BLOCK


def ns_workspace_bytes(rows: int, cols: int, count: int, head_rows: int = 0,
                       compute: str = "bf16") -> int:
    return int(_lib.load().muon_ns_workspace_bytes(
        Shape(rows, cols, head_rows), count, MUON_BF16 if compute == "bf16" else MUON_F32))


def workspace_bytes(shapes: Sequence[Tuple[int, int, int]], compute: str = "bf16") -> int:
    """muon_workspace_bytes: workspace for Newton-Schulz over mixed shapes, one
    call per shape group, one after another on one context."""
    arr = (Shape * max(len(shapes), 1))(*[Shape(r, c, h) for (r, c, h) in shapes])
    return int(_lib.load().muon_workspace_bytes(arr, len(shapes),
                                                MUON_BF16 if compute == "bf16" else MUON_F32))


def newton_schulz_noalloc(mats: Sequence[torch.Tensor], out: Optional[Sequence[torch.Tensor]] = None,
                          head_rows: int = 0, params: Optional[NsParams] = None,
                          nonfinite_flag: Optional[torch.Tensor] = None, stream=None):
    """muon_newton_schulz_batched_noalloc: the batched Newton-Schulz without a
    context or any allocation (static device scratch of
    MUON_NOALLOC_SCRATCH_BYTES per GPU).  Matrices evenly spaced; out None
    (in place), the inputs, or disjoint from them."""
    lib = _lib.load()
    device = mats[0].device
    if params is None:
        params = ns_params(compute="bf16" if mats[0].dtype == torch.bfloat16 else "f32")
    shape, dt = mats[0].shape, mats[0].dtype
    for i, m in enumerate(mats):
        _check(m, f"mats[{i}]", device)
        if m.dim() != 2 or m.shape != shape or m.dtype != dt:
            raise ValueError("all matrices of one call must be 2D with one shape and dtype")
    arr_t = ctypes.c_void_p * len(mats)
    pin = arr_t(*[m.data_ptr() for m in mats])
    pout = None
    if out is not None:
        for i, o in enumerate(out):
            _check(o, f"out[{i}]", device)
        pout = arr_t(*[o.data_ptr() for o in out])
    flag = ctypes.c_void_p(nonfinite_flag.data_ptr()) if nonfinite_flag is not None else None
    st = lib.muon_newton_schulz_batched_noalloc(
        device.index, _stream(device, stream), pin, len(mats), Shape(shape[0], shape[1], head_rows),
        _dtype(mats[0]), ctypes.byref(params), pout, flag)
    if st != _lib.MUON_OK:
        raise MuonError(st, f"muon_newton_schulz_batched_noalloc: {lib.muon_noalloc_last_error().decode()}")


class Context:
    """A libmuon context: one device and one preallocated workspace slab."""

    def __init__(self, device=None, workspace_bytes: int = 0):
        self.lib = _lib.load()
        self.device = torch.device(device if device is not None else "cuda", )
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        h = ctypes.c_void_p()
        st = self.lib.muon_create(self.device.index, int(workspace_bytes), ctypes.byref(h))
        if st != _lib.MUON_OK:
            raise MuonError(st, "muon_create")
        self.handle = h
        self.workspace_bytes = int(workspace_bytes)

    def close(self):
        if getattr(self, "handle", None):
            self.lib.muon_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _raise(self, st: int, what: str):
        if st != _lib.MUON_OK:
            raise MuonError(st, f"{what}: {self.lib.muon_last_error(self.handle).decode()}")

    # -- the three steps ----------------------------------------------------
    def momentum_update(self, grad: torch.Tensor, momentum: torch.Tensor, update_out: torch.Tensor,
                        beta: float = 0.95, nesterov: bool = True, stream=None,
                        sq_partials: Optional[torch.Tensor] = None):
        """Momentum step; with `sq_partials` (float64, ceil(numel / 4096)
        elements) also the per-block sums of squares of the stored update."""
        for t, n in ((grad, "grad"), (momentum, "momentum"), (update_out, "update_out")):
            _check(t, n, self.device)
        if momentum.dtype != torch.float32:
            raise TypeError("momentum must be float32")
        numel = grad.numel()
        if momentum.numel() != numel or update_out.numel() != numel:
            raise ValueError("grad, momentum and update_out must have the same numel")
        args = (self.handle, _stream(self.device, stream), ctypes.c_void_p(grad.data_ptr()), _dtype(grad),
                ctypes.c_void_p(momentum.data_ptr()), ctypes.c_void_p(update_out.data_ptr()),
                _dtype(update_out), numel, float(beta), 1 if nesterov else 0)
        if sq_partials is None:
            st = self.lib.muon_momentum_update(*args)
        else:
            _check(sq_partials, "sq_partials", self.device)
            if sq_partials.dtype != torch.float64 or sq_partials.numel() < sq_blocks(numel):
                raise ValueError(f"sq_partials must be float64 with at least {sq_blocks(numel)} elements")
            st = self.lib.muon_momentum_update_sq(*args, ctypes.c_void_p(sq_partials.data_ptr()))
        self._raise(st, "muon_momentum_update")

    def newton_schulz(self, mats: Sequence[torch.Tensor], out: Optional[Sequence[torch.Tensor]] = None,
                      head_rows: int = 0, params: Optional[NsParams] = None,
                      nonfinite_flag: Optional[torch.Tensor] = None, stream=None,
                      _ptrs: Optional[Tuple] = None, sq: Optional[Tuple] = None):
        """Orthogonalise a same-shape group of matrices (in place when out is None).

        sq = (partials, base): norms from a momentum pass's sum-of-squares
        partials (float64 tensor) written for the update buffer `base` (a
        tensor, or its device address) that the matrices are views of."""
        if params is None:
            params = ns_params(compute="bf16" if mats[0].dtype == torch.bfloat16 else "f32")
        if sq is not None:
            partials, base = sq
            p = NsParams()
            ctypes.memmove(ctypes.byref(p), ctypes.byref(params), ctypes.sizeof(NsParams))
            p.sq_partials = partials.data_ptr()
            p.sq_base = base if isinstance(base, int) else base.data_ptr()
            p.sq_count = partials.numel()
            params = p
        if _ptrs is None:
            _ptrs = self.pointer_arrays(mats, out)
        rows, cols = mats[0].shape[-2], mats[0].shape[-1]
        flag = ctypes.c_void_p(nonfinite_flag.data_ptr()) if nonfinite_flag is not None else None
        pin, pout, count = _ptrs
        st = self.lib.muon_newton_schulz_batched(
            self.handle, _stream(self.device, stream), pin, count, Shape(rows, cols, head_rows),
            _dtype(mats[0]), ctypes.byref(params), pout, flag)
        self._raise(st, "muon_newton_schulz_batched")

    def pointer_arrays(self, mats: Sequence[torch.Tensor], out: Optional[Sequence[torch.Tensor]] = None):
        """Host pointer arrays for newton_schulz (cacheable while the tensors live)."""
        if isinstance(mats, torch.Tensor) and mats.dim() == 3:
            mats = list(mats.unbind(0))
        if out is not None and isinstance(out, torch.Tensor) and out.dim() == 3:
            out = list(out.unbind(0))
        shape, dt = mats[0].shape, mats[0].dtype
        for i, m in enumerate(mats):
            _check(m, f"mats[{i}]", self.device)
            if m.dim() != 2 or m.shape != shape or m.dtype != dt:
                raise ValueError("all matrices of one call must be 2D with one shape and dtype")
        arr_t = ctypes.c_void_p * len(mats)
        pin = arr_t(*[m.data_ptr() for m in mats])
        pout = None
        if out is not None:
            if len(out) != len(mats):
                raise ValueError("out must have one matrix per input")
            for i, o in enumerate(out):
                _check(o, f"out[{i}]", self.device)
                if o.shape != shape or o.dtype != dt:
                    raise ValueError("out matrices must match the inputs")
            pout = arr_t(*[o.data_ptr() for o in out])
        return pin, pout, len(mats)

    def apply(self, master: torch.Tensor, update: torch.Tensor, lr: float, scale: float = 1.0,
              weight_decay: float = 0.0, weight_bf16: Optional[torch.Tensor] = None, stream=None):
        _check(master, "master", self.device)
        _check(update, "update", self.device)
        if master.dtype != torch.float32:
            raise TypeError("master must be float32")
        numel = master.numel()
        if update.numel() != numel:
            raise ValueError("master and update must have the same numel")
        wb = None
        if weight_bf16 is not None:
            _check(weight_bf16, "weight_bf16", self.device)
            if weight_bf16.dtype != torch.bfloat16 or weight_bf16.numel() != numel:
                raise ValueError("weight_bf16 must be bfloat16 with the master's numel")
            wb = ctypes.c_void_p(weight_bf16.data_ptr())
        st = self.lib.muon_apply(self.handle, _stream(self.device, stream),
                                 ctypes.c_void_p(master.data_ptr()), ctypes.c_void_p(update.data_ptr()),
                                 _dtype(update), wb, numel, float(lr), float(scale), float(weight_decay))
        self._raise(st, "muon_apply")

    # -- timing ---------------------------------------------------------------
    def timing_enable(self, enable: bool = True, capacity: int = 8192):
        self._raise(self.lib.muon_timing_enable(self.handle, 1 if enable else 0, capacity), "timing_enable")

    def timing_select(self, classes=None):
        """Time only the named kernel classes (names of timing_read); None: all."""
        names = list(_lib.KERNEL_CLASSES)
        if classes is None:
            mask = (1 << len(names)) - 1
        else:
            mask = 0
            for c in classes:
                if c not in names:
                    raise ValueError(f"unknown kernel class {c!r}; one of {names}")
                mask |= 1 << names.index(c)
        self._raise(self.lib.muon_timing_select(self.handle, mask), "timing_select")

    def timing_reset(self):
        self._raise(self.lib.muon_timing_reset(self.handle), "timing_reset")

    def timing_read(self) -> dict:
        res = {}
        for k, name in enumerate(_lib.KERNEL_CLASSES):
            ms, n = ctypes.c_double(), ctypes.c_int64()
            self._raise(self.lib.muon_timing_read(self.handle, k, ctypes.byref(ms), ctypes.byref(n)),
                        "timing_read")
            res[name] = (ms.value, n.value)
        return res


@dataclass
class BucketInfo:
    m: int
    n: int
    count: int
    units: int
    numel: int
    full_bytes: int
    workspace_bytes: int
    over_cap: bool
    shape_groups: int
    indices: List[int]
    elem_offset: int = 0
    offsets: List[int] = None


class Plan:
    """Host scheduler result: micro-buckets of whole matrices under a cap."""

    def __init__(self, shapes: Sequence[Tuple[int, int, int]], cap_bytes: int, cap_kind: str = "full",
                 compute: str = "bf16", compute_units: int = 0):
        lib = _lib.load()
        arr = (Shape * len(shapes))(*[Shape(r, c, h) for (r, c, h) in shapes])
        h = ctypes.c_void_p()
        kind = MUON_CAP_FULL_BYTES if cap_kind == "full" else MUON_CAP_WORKSPACE
        st = lib.muon_plan_create(arr, len(shapes), int(cap_bytes), kind,
                                  MUON_BF16 if compute == "bf16" else MUON_F32, int(compute_units),
                                  ctypes.byref(h))
        if st != _lib.MUON_OK:
            raise MuonError(st, "muon_plan_create")
        try:
            self.buckets: List[BucketInfo] = []
            for b in range(lib.muon_plan_num_buckets(h)):
                info = _lib.BucketInfo()
                lib.muon_plan_bucket(h, b, ctypes.byref(info), None, None)
                idx = (ctypes.c_int64 * info.count)()
                off = (ctypes.c_int64 * info.count)()
                lib.muon_plan_bucket(h, b, ctypes.byref(info), idx, off)
                self.buckets.append(BucketInfo(info.m, info.n, info.count, info.units, info.numel,
                                               info.full_bytes, info.workspace_bytes,
                                               bool(info.over_cap), info.shape_groups, list(idx),
                                               info.elem_offset, list(off)))
            self.max_workspace = int(lib.muon_plan_max_workspace(h))
            self.total_elems = int(lib.muon_plan_total_elems(h))
        finally:
            lib.muon_plan_destroy(h)
