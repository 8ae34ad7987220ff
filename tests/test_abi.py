"""The C ABI without a GPU: exports, host scheduler, workspace arithmetic,
argument validation.  No compute call is made here."""
import ctypes
import os
import re

import pytest

from newton_schulz_amd import _lib
from newton_schulz_amd.api import Plan, ns_workspace_bytes, workspace_bytes
from newton_schulz_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    # symbols are exported with C linkage
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings():
    lib = _lib.load()
    assert lib.muon_status_string(0) == b"ok"
    assert lib.muon_status_string(4) == b"workspace too small"
    assert lib.muon_status_string(99) == b"unknown status"


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = _lib.load()
    h = ctypes.c_void_p()
    assert lib.muon_create(0, 1 << 20, ctypes.byref(h)) == _lib.MUON_EHIP
    assert not h.value
    assert lib.muon_create(0, 0, None) == _lib.MUON_EINVAL
    assert lib.muon_destroy(None) == _lib.MUON_OK


def test_timing_select_rejects_null_and_unknown_classes():
    lib = _lib.load()
    assert lib.muon_timing_select(None, 1) == _lib.MUON_EINVAL
    assert lib.muon_timing_select(None, 1 << len(_lib.KERNEL_CLASSES)) == _lib.MUON_EINVAL


def test_struct_and_enum_mirrors_match_header():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} muon_ns_params_t;", text).group(1)
    fields = re.findall(r"([a-z_]+)(?:\s*,\s*([a-z_]+))?(?:\s*,\s*([a-z_]+))?\s*;", body)
    names = [n for grp in fields for n in grp if n]
    assert names == [f for f, _ in _lib.NsParams._fields_]
    count = int(re.search(r"MUON_K_COUNT\s*=\s*(\d+)", text).group(1))
    assert len(_lib.KERNEL_CLASSES) == count
    assert int(re.search(r"MUON_NS_GRAM\s*=\s*(\d+)", text).group(1)) == 1
    from newton_schulz_amd.api import NS_FUSE, SQ_BLOCK
    assert int(re.search(r"#define MUON_SQ_BLOCK\s+(\d+)", text).group(1)) == SQ_BLOCK
    for name, v in NS_FUSE.items():
        assert int(re.search(rf"MUON_FUSE_{name.upper()}\s*=\s*(\d+)", text).group(1)) == v


def test_null_context_rejected():
    lib = _lib.load()
    p = _lib.NsParams()
    lib.muon_ns_params_default(ctypes.byref(p))
    assert (p.steps, round(p.a, 4), round(p.b, 4), round(p.c, 4), p.compute) == (5, 3.4445, -4.775, 2.0315, 1)
    assert p.method == 0 and p.fuse == 0 and not p.coeffs
    assert not p.sq_partials and not p.sq_base and p.sq_count == 0
    assert lib.muon_momentum_update(None, None, None, 1, None, None, 1, 10, 0.95, 1) == _lib.MUON_EINVAL
    assert lib.muon_apply(None, None, None, None, 1, None, 10, 0.02, 1.0, 0.0) == _lib.MUON_EINVAL
    assert lib.muon_momentum_update_sq(None, None, None, 1, None, None, 1, 10, 0.95, 1,
                                       None) == _lib.MUON_EINVAL
    assert lib.muon_newton_schulz_batched(None, None, None, 1, _lib.Shape(8, 8, 0), 1, ctypes.byref(p),
                                          None, None) == _lib.MUON_EINVAL


def _aligned(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("rows,cols,h,count,compute", [
    (2560, 4096, 0, 25, "bf16"), (4096, 2560, 0, 3, "bf16"), (128, 2560, 0, 1728, "bf16"),
    (4096, 2560, 128, 2, "bf16"), (96, 96, 0, 1, "f32"), (256, 64, 0, 2, "f32"),
])
def test_workspace_formula(rows, cols, h, count, compute):
    e = 2 if compute == "bf16" else 4
    ur = h if h else rows
    units = count * (rows // ur)
    m, n = min(ur, cols), max(ur, cols)
    ue = ur * cols
    parts = min(max((ue + 32767) // 32768, 1), 512)
    chunk = -(-ue // parts)
    chunk = -(-chunk // 8) * 8
    parts = -(-ue // chunk)
    want = (2 * _aligned(units * m * n * e) + 2 * _aligned(units * m * m * e)
            + 2 * _aligned(units * 4) + _aligned(units * parts * 8))
    lo = 0
    if compute == "bf16":
        # the iterate's residual plane, tile-padded (T = 256 once m >= 256,
        # else 128), and B's diagonal, one float per row
        t = 256 if m >= 256 else 128
        lo = units * (-(-m // t) * t) * (-(-n // t) * t) * 2
        want += _aligned(lo) + _aligned(units * m * 4)
    assert ns_workspace_bytes(rows, cols, count, h, compute) == want
    # the stated bound: (2 + 2 m / n) x full bytes (bf16: 3 + 2 m / n, the
    # residual plane, up to its tile padding), plus small scalars
    full = units * m * n * e
    k = 3 if compute == "bf16" else 2
    pad = (lo - units * m * n * 2) if lo else 0
    assert want <= (k + 2 * m / n) * full + pad + 6 * 256 + units * (12 + 4 * m + parts * 8)


def test_workspace_rejects_bad_shapes():
    assert ns_workspace_bytes(100, 64, 1, 30) == 0      # rows % head_rows
    assert ns_workspace_bytes(0, 64, 1) == 0
    assert ns_workspace_bytes(64, 64, 0) == 0           # count 0: nothing needed


def test_plan_qwen3_4b_buckets():
    w = synth.qwen3_4b(layers=36)
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    plan = Plan(shapes, 512 << 20, "full", "bf16")
    # canonical buckets (2560,4096): q + o; (1024,2560): k + v; (2560,9728): gate, up, down
    keys = [(b.m, b.n) for b in plan.buckets]
    assert keys == [(2560, 4096)] * 3 + [(1024, 2560)] + [(2560, 9728)] * 11
    assert [b.count for b in plan.buckets] == [25, 25, 22, 72] + [10] * 10 + [8]
    # every matrix exactly once; each micro-bucket within the cap
    flat = sorted(i for b in plan.buckets for i in b.indices)
    assert flat == list(range(len(shapes)))
    for b in plan.buckets:
        assert b.full_bytes <= 512 << 20 and not b.over_cap
        assert b.full_bytes == 2 * sum(shapes[i][0] * shapes[i][1] for i in b.indices)
    # inside a bucket, same exact shapes are contiguous (q first, then o)
    first = plan.buckets[0]
    assert [shapes[i][:2] for i in first.indices] == [(4096, 2560)] * 25
    assert [shapes[i][:2] for i in plan.buckets[1].indices] == [(4096, 2560)] * 11 + [(2560, 4096)] * 14
    assert plan.buckets[1].shape_groups == 2 and plan.buckets[2].shape_groups == 1
    # workspace: stated function of the cap, (3 + 2 m/n) x full bytes at most
    # in bf16 (two iterates, the iterate's residual plane, A and B'); these
    # shapes fill whole 256-tiles, so the residual plane has no padding
    for b in plan.buckets:
        scalars = b.units * (8 + 4 * b.m + 512 * 8) + 8 * 256 * b.shape_groups
        assert b.workspace_bytes <= (3 + 2 * b.m / b.n) * b.full_bytes + scalars
    assert plan.max_workspace == max(b.workspace_bytes for b in plan.buckets)


def _round_cost(m, n, units, cus=256):
    # k-elements per tile slot of one bucket's product launches, rounds of
    # ceil(tiles / CUs) (256 x 256 tiles, one per CU)
    t, tn = -(-m // 256), -(-n // 256)
    sym = -(-(units * t * (t + 1) // 2) // cus)
    upd = -(-(units * t * tn) // cus)
    return sym * (n + m) + upd * m


def test_plan_wave_aware_cuts_qwen3_4b():
    w = synth.qwen3_4b(layers=36)
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    plan = Plan(shapes, 512 << 20, "full", "bf16", compute_units=256)
    flat = [i for b in plan.buckets for i in b.indices]
    assert sorted(flat) == list(range(len(shapes)))
    for b in plan.buckets:
        assert b.full_bytes <= 512 << 20 and not b.over_cap
    counts = {}
    for b in plan.buckets:
        counts.setdefault((b.m, b.n), []).append(b.count)
    # (2560, 9728): 10 per micro-bucket (cap-filling) leaves 550 Gram tiles =
    # 2.15 rounds on 256 CUs, so 9 (495 tiles, 2 rounds) is cheaper per matrix
    assert counts[(2560, 9728)] == [9] * 12
    assert _round_cost(2560, 9728, 9) / 9 < _round_cost(2560, 9728, 10) / 10
    assert sum(counts[(2560, 4096)]) == 72 and max(counts[(2560, 4096)]) <= 25
    assert counts[(1024, 2560)] == [72]
    # the cut plan never models slower than the greedy one
    greedy = Plan(shapes, 512 << 20, "full", "bf16")
    cost = lambda p: sum(_round_cost(b.m, b.n, b.units) for b in p.buckets)
    assert cost(plan) < cost(greedy)


def test_plan_workspace_cap_experts():
    w = synth.qwen3_30b_experts(layers=2)
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    plan = Plan(shapes, 1 << 30, "workspace", "bf16")
    assert all(b.workspace_bytes <= 1 << 30 for b in plan.buckets)
    assert all((b.m, b.n) == (768, 2048) for b in plan.buckets)
    assert sum(b.count for b in plan.buckets) == len(shapes)
    # cross-layer merge: one canonical bucket for all expert matrices (gate,
    # up and the transposed down alike), filled greedily up to the cap, so
    # every micro-bucket but the last holds as many experts as the cap allows
    full = [b.count for b in plan.buckets[:-1]]
    assert full and all(c == full[0] for c in full) and plan.buckets[-1].count <= full[0]
    assert len(plan.buckets) == -(-len(shapes) // full[0])


def test_plan_over_cap_matrix_alone():
    plan = Plan([(64, 64, 0), (4096, 4096, 0), (64, 64, 0)], 1 << 20, "full", "bf16")
    big = [b for b in plan.buckets if b.m == 4096]
    assert len(big) == 1 and big[0].over_cap and big[0].count == 1


def test_plan_per_head_units():
    plan = Plan([(4096, 2560, 128), (1024, 2560, 128)], 1 << 40, "full", "bf16")
    assert len(plan.buckets) == 1
    b = plan.buckets[0]
    assert (b.m, b.n, b.units, b.shape_groups) == (128, 2560, 32 + 8, 2)


def _q4b_shapes():
    return [(m.rows, m.cols, m.head_rows) for m in synth.qwen3_4b(layers=36).mats]


def _shape_array(shapes):
    return (_lib.Shape * len(shapes))(*[_lib.Shape(r, c, h) for (r, c, h) in shapes])


def test_plan_offsets_are_the_flat_layout():
    """muon_plan_bucket's offsets: micro-bucket after micro-bucket, members
    packed in execution order, each micro-bucket one contiguous range."""
    shapes = _q4b_shapes() + [(128, 2560, 0)] * 5 + [(768, 2048, 0)] * 3
    for cus in (0, 256):
        plan = Plan(shapes, 512 << 20, "full", "bf16", compute_units=cus)
        pos = 0
        for b in plan.buckets:
            assert b.elem_offset == pos
            assert len(b.offsets) == b.count
            for i, o in zip(b.indices, b.offsets):
                assert o == pos
                pos += shapes[i][0] * shapes[i][1]
            assert pos - b.elem_offset == b.numel
        assert plan.total_elems == pos == sum(r * c for r, c, _ in shapes)


def test_muon_plan_is_plan_create_bf16_greedy():
    """muon_plan (cap and its kind only) through ctypes equals
    muon_plan_create with BF16 compute and compute_units = 0."""
    lib = _lib.load()
    shapes = _q4b_shapes()
    arr = _shape_array(shapes)
    for cap, kind in ((512 << 20, _lib.MUON_CAP_FULL_BYTES), (1 << 30, _lib.MUON_CAP_WORKSPACE)):
        h1, h2 = ctypes.c_void_p(), ctypes.c_void_p()
        assert lib.muon_plan(arr, len(shapes), cap, kind, ctypes.byref(h1)) == _lib.MUON_OK
        assert lib.muon_plan_create(arr, len(shapes), cap, kind, _lib.MUON_BF16, 0,
                                    ctypes.byref(h2)) == _lib.MUON_OK
        try:
            nb = lib.muon_plan_num_buckets(h1)
            assert nb == lib.muon_plan_num_buckets(h2) > 0
            assert lib.muon_plan_total_elems(h1) == lib.muon_plan_total_elems(h2)
            assert lib.muon_plan_max_workspace(h1) == lib.muon_plan_max_workspace(h2)
            for b in range(nb):
                i1, i2 = _lib.BucketInfo(), _lib.BucketInfo()
                assert lib.muon_plan_bucket(h1, b, ctypes.byref(i1), None, None) == _lib.MUON_OK
                lib.muon_plan_bucket(h2, b, ctypes.byref(i2), None, None)
                assert bytes(i1) == bytes(i2)
                x1, x2 = (ctypes.c_int64 * i1.count)(), (ctypes.c_int64 * i1.count)()
                o1, o2 = (ctypes.c_int64 * i1.count)(), (ctypes.c_int64 * i1.count)()
                lib.muon_plan_bucket(h1, b, ctypes.byref(i1), x1, o1)
                lib.muon_plan_bucket(h2, b, ctypes.byref(i2), x2, o2)
                assert list(x1) == list(x2) and list(o1) == list(o2)
            info = _lib.BucketInfo()
            assert lib.muon_plan_bucket(h1, nb, ctypes.byref(info), None, None) == _lib.MUON_EINVAL
            assert lib.muon_plan_bucket(h1, -1, ctypes.byref(info), None, None) == _lib.MUON_EINVAL
            assert lib.muon_plan_bucket(h1, 0, None, None, None) == _lib.MUON_EINVAL
        finally:
            lib.muon_plan_destroy(h1)
            lib.muon_plan_destroy(h2)
    assert lib.muon_plan(arr, len(shapes), 1 << 20, 7, None) == _lib.MUON_EINVAL
    assert lib.muon_plan_total_elems(None) == 0
    lib.muon_plan_destroy(None)


def test_workspace_bytes_mixed_shapes():
    """muon_workspace_bytes: the largest shape group's need (groups by exact
    shape, wherever the members sit in the list)."""
    shapes = [(2560, 4096, 0), (128, 2560, 0), (2560, 4096, 0), (4096, 2560, 128), (2560, 4096, 0)]
    for compute in ("bf16", "f32"):
        want = max(ns_workspace_bytes(2560, 4096, 3, 0, compute),
                   ns_workspace_bytes(128, 2560, 1, 0, compute),
                   ns_workspace_bytes(4096, 2560, 1, 128, compute))
        assert workspace_bytes(shapes, compute) == want
    q = _q4b_shapes()
    groups = {}
    for s in q:
        groups[s] = groups.get(s, 0) + 1
    assert workspace_bytes(q) == max(ns_workspace_bytes(r, c, n, h) for (r, c, h), n in groups.items())
    assert workspace_bytes([]) == 0
    assert workspace_bytes([(100, 64, 30)]) == 0


def test_plan_rejects_bad_input():
    from newton_schulz_amd.api import MuonError
    with pytest.raises(MuonError):
        Plan([(100, 64, 30)], 1 << 20)
    with pytest.raises(MuonError):
        Plan([(0, 64, 0)], 1 << 20)


@pytest.mark.parametrize("steps,lo,margin", [
    (1, 1e-3, 0.02), (6, 1e-3, 0.02), (10, 1e-3, 0.01), (5, 0.1, 0.05), (3, 0.5, 0.01), (8, 1e-4, 0.1),
])
def test_minimax_coeffs_match_oracle(steps, lo, margin):
    """libmuon's host schedule against the oracle's own (independent) one."""
    import numpy as np
    import oracle
    from newton_schulz_amd import minimax_coeffs
    rows, bound = minimax_coeffs(steps, lo, margin)
    ref, E = oracle.minimax_schedule(steps, lo, margin)
    np.testing.assert_allclose(np.array(rows), ref.astype(np.float32), rtol=2e-7, atol=0)
    assert bound == pytest.approx(E, rel=1e-9, abs=1e-15)


def test_minimax_coeffs_rejects_bad_arguments():
    lib = _lib.load()
    out = (ctypes.c_float * 30)()
    ok = lib.muon_ns_minimax_coeffs(10, 1e-3, 0.02, out, None)
    assert ok == _lib.MUON_OK
    # margins outside [0.01, 0.1] are refused (measured to diverge with bf16
    # iterates on low-rank inputs), though the schedule itself is defined
    for steps, lo, margin in [(0, 1e-3, 0.02), (1025, 1e-3, 0.02), (3, 0.0, 0.02), (3, 1.0, 0.02),
                              (3, float("nan"), 0.02), (3, 1e-3, -0.01), (3, 1e-3, 0.0),
                              (3, 1e-3, 0.009), (3, 1e-3, 0.11), (3, 1e-3, 0.2),
                              (3, 1e-3, float("nan"))]:
        assert lib.muon_ns_minimax_coeffs(steps, lo, margin, out, None) == _lib.MUON_EINVAL
    assert lib.muon_ns_minimax_coeffs(3, 1e-3, 0.02, None, None) == _lib.MUON_EINVAL


def test_ns_params_coefficient_table():
    from newton_schulz_amd import minimax_coeffs, ns_params
    p = ns_params(steps=4, coeffs="minimax")
    rows, _ = minimax_coeffs(4)
    assert [p.coeffs[i] for i in range(12)] == [v for r in rows for v in r]
    q = ns_params(steps=2, coeffs=[(1.0, 2.0, 3.0), (4.0, 5.0, 6.0)])
    assert [q.coeffs[i] for i in range(6)] == [1.0, 2.0, 3.0, 4.0, 5.0, 6.0]
    with pytest.raises(ValueError):
        ns_params(steps=3, coeffs=[(1.0, 2.0, 3.0)])
    with pytest.raises(ValueError):
        ns_params(steps=3, coeffs="chebyshev")


def test_plan_orientation_order_and_model():
    """Inside a micro-bucket the members of the first member's orientation come
    first (wide and tall units run as separate launch chains), and the
    wave-aware cuts model each orientation's rounds on its own: the
    Qwen3-4B (2560, 4096) bucket (36 tall q, 36 wide o) gets no micro-bucket
    that mixes the two."""
    shapes = [(2560, 4096, 0), (4096, 2560, 0), (2560, 4096, 0), (4096, 2560, 0)]
    plan = Plan(shapes, 1 << 40, "full", "bf16")
    assert len(plan.buckets) == 1 and plan.buckets[0].indices == [0, 2, 1, 3]
    plan = Plan(_q4b_shapes(), 512 << 20, "full", "bf16", compute_units=256)
    q4 = _q4b_shapes()
    for b in plan.buckets:
        tall = {q4[i][0] > q4[i][1] for i in b.indices}
        assert len(tall) == 1, (b.m, b.n, b.indices)
    sizes = sorted(b.count for b in plan.buckets if (b.m, b.n) == (2560, 4096))
    assert sum(sizes) == 72
