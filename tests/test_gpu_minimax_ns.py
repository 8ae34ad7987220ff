"""Parity of Newton-Schulz with per-iteration coefficients against the oracle.

The HIP path takes its table from libmuon's muon_ns_minimax_coeffs; the
oracle computes its own schedule (oracle.minimax_schedule, independent code)
and runs ns_ref with those rows.  Bars as for the fixed quintic: relative
Frobenius error per unit <= 2e-2 in bf16 compute, <= 1e-4 in fp32; the fused
small-unit kernel is bit-identical to the unfused kernels.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_amd import Context, MuonError, ns_params
from newton_schulz_amd import synth

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Context(DEV, 2 << 30)
    yield c
    c.close()


def host(t):
    return t.detach().float().cpu().numpy()


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def run(ctx, mats, head_rows, p):
    out = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, out, head_rows, p)
    torch.cuda.synchronize()
    return out


def check(ctx, rows, cols, count, dtype, tol, head_rows=0, seed=0, steps=5, lo=1e-3,
          margin=0.05, method="quintic", fuse="auto", rows_table=None, std=1e-3):
    g = gen(7000 + seed)
    mats = [synth.normal((rows, cols), std, g, DEV, dtype) for _ in range(count)]
    ins = [host(m) for m in mats]
    compute = "bf16" if dtype == torch.bfloat16 else "f32"
    if rows_table is None:
        p = ns_params(steps=steps, compute=compute, method=method, fuse=fuse, coeffs="minimax",
                      lo=lo, margin=margin)
        ref_rows, _ = oracle.minimax_schedule(steps, lo, margin)
    else:
        p = ns_params(steps=steps, compute=compute, method=method, fuse=fuse, coeffs=rows_table)
        ref_rows = np.asarray(rows_table, dtype=np.float64)
    out = run(ctx, mats, head_rows, p)
    errs = []
    for x, o in zip(ins, out):
        ref = oracle.ns_ref_heads(x, head_rows, steps=steps, coeffs=ref_rows)
        got = host(o)
        hs = head_rows or rows
        for k in range(rows // hs):
            sl = slice(k * hs, (k + 1) * hs)
            errs.append(oracle.rel_fro(got[sl], ref[sl]))
    say(f"  minimax-ns {method} {rows}x{cols} x{count} {dtype} h={head_rows} steps={steps} "
        f"fuse={fuse}: max rel err {max(errs):.3e}")
    assert max(errs) <= tol, errs
    return mats, out


@pytest.mark.parametrize("rows,cols", [(64, 128), (96, 96), (256, 64), (72, 200)])
def test_minimax_fp32(ctx, rows, cols):
    check(ctx, rows, cols, 3, torch.float32, F32_TOL, seed=rows * cols, std=1.0)


@pytest.mark.parametrize("rows,cols", [(256, 512), (520, 1048), (1048, 520), (768, 2048),
                                       (2048, 768), (256, 256), (384, 640), (202, 618)])
def test_minimax_bf16(ctx, rows, cols):
    check(ctx, rows, cols, 3, torch.bfloat16, BF16_TOL, seed=rows + cols)


@pytest.mark.parametrize("steps", [1, 2, 4, 6, 8])
def test_minimax_step_counts(ctx, steps):
    check(ctx, 768, 2048, 2, torch.bfloat16, BF16_TOL, seed=steps, steps=steps)


def test_minimax_narrow_margin(ctx):
    """A caller-chosen margin reaches the kernels (the schedule differs)."""
    check(ctx, 512, 1024, 2, torch.bfloat16, BF16_TOL, seed=3, steps=6, margin=0.02)


@pytest.mark.parametrize("rows,cols", [(256, 1024), (768, 2048), (2048, 768), (1024, 2560)])
def test_minimax_gram_form(ctx, rows, cols):
    check(ctx, rows, cols, 3, torch.bfloat16, BF16_TOL, seed=rows * 3 + cols, method="gram")


def test_minimax_large_unit(ctx):
    """One 2560 x 4096 unit: the product kernels' 256-tiles, many tiles."""
    check(ctx, 2560, 4096, 1, torch.bfloat16, BF16_TOL, seed=11)


@pytest.mark.parametrize("method", ["quintic", "gram"])
@pytest.mark.parametrize("rows,cols,head_rows", [(128, 2560, 0), (64, 512, 0), (4096, 2560, 128)])
def test_minimax_fused_small_units(ctx, method, rows, cols, head_rows):
    """The fused kernel reads the table row by row; it must equal the unfused
    kernels bit for bit and meet the oracle bar."""
    count = 4 if head_rows else 40
    mats, fused = check(ctx, rows, cols, count, torch.bfloat16, BF16_TOL, head_rows=head_rows,
                        seed=rows + cols + head_rows, method=method, fuse="on")
    p = ns_params(steps=5, method=method, fuse="off", coeffs="minimax")
    plain = run(ctx, mats, head_rows, p)
    for a, b in zip(fused, plain):
        assert torch.equal(a, b)


def test_rows_are_taken_in_order(ctx):
    """A table whose rows differ: rows applied out of order (or one row for
    all) would miss the oracle by far more than the bar."""
    table = [(3.4445, -4.7750, 2.0315), (3.0, -3.2, 1.2), (1.875, -1.25, 0.375),
             (3.4445, -4.7750, 2.0315), (1.875, -1.25, 0.375)]
    for fuse, shape in [("off", (384, 1024)), ("on", (128, 1024))]:
        check(ctx, shape[0], shape[1], 3, torch.bfloat16, BF16_TOL, seed=5, fuse=fuse,
              rows_table=table)
    # sanity of the test itself: the reversed table gives another result
    x = np.random.default_rng(0).standard_normal((64, 256))
    fwd = oracle.ns_ref(x, steps=5, coeffs=table)
    rev = oracle.ns_ref(x, steps=5, coeffs=table[::-1])
    assert oracle.rel_fro(rev, fwd) > 5 * BF16_TOL


def test_table_longer_than_fused_limit_runs_unfused(ctx):
    """More rows than the fused kernel carries: the call still runs (unfused)."""
    steps = 17
    table = [(1.875, -1.25, 0.375)] * steps
    check(ctx, 128, 1024, 3, torch.bfloat16, BF16_TOL, seed=17, steps=steps, fuse="on",
          rows_table=table)


def test_constant_table_equals_fixed_coefficients(ctx):
    """A table repeating (a, b, c) gives the bits of the fixed coefficients."""
    g = gen(99)
    for shape, fuse in [((512, 1024), "auto"), ((128, 1024), "on")]:
        mats = [synth.normal(shape, 1e-3, g, DEV, torch.bfloat16) for _ in range(3)]
        fixed = run(ctx, mats, 0, ns_params(steps=5, fuse=fuse))
        table = run(ctx, mats, 0, ns_params(steps=5, fuse=fuse,
                                            coeffs=[(3.4445, -4.7750, 2.0315)] * 5))
        for a, b in zip(fixed, table):
            assert torch.equal(a, b)


def test_deterministic_and_in_place(ctx):
    g = gen(123)
    mats = [synth.normal((768, 2048), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    p = ns_params(steps=5, coeffs="minimax")
    a = run(ctx, mats, 0, p)
    b = run(ctx, mats, 0, p)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ip = [m.clone() for m in mats]
    ctx.newton_schulz(ip, None, 0, p)
    torch.cuda.synchronize()
    for x, y in zip(a, ip):
        assert torch.equal(x, y)


def test_zero_units_exact(ctx):
    z = torch.zeros((256, 512), dtype=torch.bfloat16, device=DEV)
    out = run(ctx, [z], 0, ns_params(steps=5, coeffs="minimax"))
    assert torch.count_nonzero(out[0]) == 0


def test_nonfinite_coefficient_rejected(ctx):
    m = torch.ones((64, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(MuonError):
        ctx.newton_schulz([m], [torch.empty_like(m)], 0,
                          ns_params(steps=2, coeffs=[(1.0, 0.0, 0.0), (float("nan"), 0.0, 0.0)]))
