"""ctypes declarations of libmuon's C ABI (include/muon.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon.so")

MUON_OK, MUON_EINVAL, MUON_ESHAPE, MUON_EDTYPE, MUON_EWORKSPACE, MUON_EHIP, MUON_ENOMEM = range(7)
MUON_F32, MUON_BF16 = 0, 1
MUON_CAP_FULL_BYTES, MUON_CAP_WORKSPACE = 0, 1
MUON_NOALLOC_SCRATCH_BYTES = 256 << 20
KERNEL_CLASSES = ["momentum", "norm", "gram", "symsq", "update", "apply", "prod", "fused"]

# every symbol include/muon.h declares
EXPORTS = [
    "muon_create", "muon_destroy", "muon_ctx_workspace_bytes", "muon_ns_params_default",
    "muon_ns_minimax_coeffs", "muon_momentum_update_sq",
    "muon_ns_workspace_bytes", "muon_plan_create", "muon_plan_num_buckets", "muon_plan_bucket",
    "muon_plan_max_workspace", "muon_plan_destroy", "muon_momentum_update",
    "muon_newton_schulz_batched", "muon_apply", "muon_status_string", "muon_last_error",
    "muon_timing_enable", "muon_timing_select", "muon_timing_reset", "muon_timing_read",
    "muon_newton_schulz_batched_noalloc", "muon_noalloc_last_error",
    "muon_plan", "muon_plan_total_elems", "muon_workspace_bytes",
]


class NsParams(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int32), ("a", ctypes.c_float), ("b", ctypes.c_float),
                ("c", ctypes.c_float), ("eps", ctypes.c_float), ("compute", ctypes.c_int32),
                ("method", ctypes.c_int32), ("fuse", ctypes.c_int32),
                ("coeffs", ctypes.POINTER(ctypes.c_float)),
                ("sq_partials", ctypes.c_void_p), ("sq_base", ctypes.c_void_p),
                ("sq_count", ctypes.c_int64)]


class Shape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("head_rows", ctypes.c_int64)]


class BucketInfo(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("count", ctypes.c_int64),
                ("units", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("full_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
                ("over_cap", ctypes.c_int32), ("shape_groups", ctypes.c_int32),
                ("elem_offset", ctypes.c_int64)]


_LIB = None


def load() -> ctypes.CDLL:
    """Load the in-tree libmuon.so; raises when it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libmuon.so is missing at {LIB_PATH}; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    P = ctypes.POINTER
    sig = {
        "muon_create": (i32, [ctypes.c_int, sz, P(vp)]),
        "muon_destroy": (i32, [vp]),
        "muon_ctx_workspace_bytes": (sz, [vp]),
        "muon_ns_params_default": (None, [P(NsParams)]),
        "muon_ns_minimax_coeffs": (i32, [i32, ctypes.c_double, ctypes.c_double, P(f32),
                                         P(ctypes.c_double)]),
        "muon_ns_workspace_bytes": (sz, [Shape, i64, i32]),
        "muon_plan_create": (i32, [P(Shape), i64, sz, i32, i32, i32, P(vp)]),
        "muon_plan_num_buckets": (i64, [vp]),
        "muon_plan": (i32, [P(Shape), i64, sz, i32, P(vp)]),
        "muon_plan_bucket": (i32, [vp, i64, P(BucketInfo), P(i64), P(i64)]),
        "muon_plan_total_elems": (i64, [vp]),
        "muon_workspace_bytes": (sz, [P(Shape), i64, i32]),
        "muon_plan_max_workspace": (sz, [vp]),
        "muon_plan_destroy": (None, [vp]),
        "muon_momentum_update": (i32, [vp, vp, vp, i32, vp, vp, i32, i64, f32, i32]),
        "muon_momentum_update_sq": (i32, [vp, vp, vp, i32, vp, vp, i32, i64, f32, i32, vp]),
        "muon_newton_schulz_batched": (i32, [vp, vp, P(vp), i64, Shape, i32, P(NsParams), P(vp), vp]),
        "muon_apply": (i32, [vp, vp, vp, vp, i32, vp, i64, f32, f32, f32]),
        "muon_status_string": (ctypes.c_char_p, [i32]),
        "muon_last_error": (ctypes.c_char_p, [vp]),
        "muon_timing_enable": (i32, [vp, i32, i32]),
        "muon_timing_select": (i32, [vp, ctypes.c_uint32]),
        "muon_timing_reset": (i32, [vp]),
        "muon_timing_read": (i32, [vp, i32, P(ctypes.c_double), P(i64)]),
        "muon_newton_schulz_batched_noalloc": (i32, [ctypes.c_int, vp, P(vp), i64, Shape, i32,
                                                      P(NsParams), P(vp), vp]),
        "muon_noalloc_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
