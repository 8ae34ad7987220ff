"""Parity of the Gram-form Newton-Schulz (MUON_NS_GRAM) with the CPU oracle.

The Gram form evaluates the same polynomial map as the quintic iteration
(A_{k+1} = P_k A_k P_k, X = P_{steps-1} ... P_0 X_0), so its exact result is
the oracle's ns_ref; the bars are the quintic's: relative Frobenius error per
unit <= 2e-2 in bf16 mode, <= 1e-4 in fp32 mode, zero units exactly zero,
identical inputs give identical bits.
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


def gram_check(ctx, rows, cols, count, dtype, tol, head_rows=0, seed=0, steps=5, std=1e-3):
    g = gen(1000 + seed)
    mats = [synth.normal((rows, cols), std, g, DEV, dtype) for _ in range(count)]
    ins = [host(m) for m in mats]
    out = [torch.empty_like(m) for m in mats]
    p = ns_params(steps=steps, compute="bf16" if dtype == torch.bfloat16 else "f32", method="gram")
    ctx.newton_schulz(mats, out, head_rows, p)
    torch.cuda.synchronize()
    errs = []
    for x, o in zip(ins, out):
        ref = oracle.ns_ref_heads(x, head_rows, steps=steps)
        got = host(o)
        hs = head_rows or rows
        for k in range(rows // hs):
            sl = slice(k * hs, (k + 1) * hs)
            errs.append(oracle.rel_fro(got[sl], ref[sl]))
    say(f"  gram-ns {rows}x{cols} x{count} {dtype} h={head_rows} steps={steps}: max rel err {max(errs):.3e}")
    assert max(errs) <= tol, errs
    return mats, out


@pytest.mark.parametrize("rows,cols", [(64, 128), (128, 128), (256, 64), (96, 96), (72, 200)])
def test_gram_fp32(ctx, rows, cols):
    gram_check(ctx, rows, cols, 3, torch.float32, F32_TOL, seed=rows * cols, std=1.0)


# bf16 runs the Gram form where 2 m <= n
@pytest.mark.parametrize("rows,cols", [(256, 512), (520, 1048), (1048, 520), (128, 2560), (2560, 128),
                                       (768, 2048), (2048, 768), (264, 1040), (1024, 2560), (384, 1000)])
def test_gram_bf16_mfma(ctx, rows, cols):
    gram_check(ctx, rows, cols, 3, torch.bfloat16, BF16_TOL, seed=rows + cols)


@pytest.mark.parametrize("rows,cols", [(202, 618), (618, 202)])
def test_gram_bf16_generic_shapes(ctx, rows, cols):
    gram_check(ctx, rows, cols, 2, torch.bfloat16, BF16_TOL, seed=rows * 3 + cols)


@pytest.mark.parametrize("rows,cols", [(256, 256), (384, 640), (640, 384), (130, 130)])
def test_gram_bf16_near_square_runs_quintic(ctx, rows, cols):
    # 2 m > n: bf16 falls back to the quintic iteration, bit for bit
    g = gen(rows * 7 + cols)
    mats = [synth.normal((rows, cols), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    a = [torch.empty_like(m) for m in mats]
    b = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, a, params=ns_params(method="gram"))
    ctx.newton_schulz(mats, b, params=ns_params())
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 256), (200, 300)])
def test_gram_fp32_square(ctx, rows, cols):
    # fp32 runs the Gram form at any aspect ratio
    gram_check(ctx, rows, cols, 2, torch.float32, F32_TOL, seed=rows + 5 * cols, std=1.0)


@pytest.mark.parametrize("steps", [0, 1, 2, 3, 6])
def test_gram_step_counts(ctx, steps):
    gram_check(ctx, 256, 640, 2, torch.bfloat16, BF16_TOL, seed=steps, steps=steps)
    gram_check(ctx, 96, 160, 2, torch.float32, F32_TOL, seed=steps, steps=steps, std=1.0)


def test_gram_per_head_and_shards(ctx):
    h, heads, cols = 128, 6, 2560
    mats, out = gram_check(ctx, h * heads, cols, 2, torch.bfloat16, BF16_TOL, head_rows=h, seed=11)
    shard = [m[2 * h:5 * h].contiguous() for m in mats]
    sout = [torch.empty_like(s) for s in shard]
    ctx.newton_schulz(shard, sout, h, params=ns_params(method="gram"))
    torch.cuda.synchronize()
    for full, part in zip(out, sout):
        assert torch.equal(full[2 * h:5 * h], part)


def test_gram_deterministic_and_in_place(ctx):
    g = gen(21)
    mats = [synth.normal((768, 2048), 1e-3, g, DEV, torch.bfloat16) for _ in range(3)]
    p = ns_params(method="gram")
    o1 = [torch.empty_like(m) for m in mats]
    o2 = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, o1, params=p)
    ctx.newton_schulz(mats, o2, params=p)
    # in place: the output overlaps the input, so the product goes through the
    # workspace and is copied back
    ip = [m.clone() for m in mats]
    ctx.newton_schulz(ip, None, params=p)
    # irregularly placed, in place (device pointer tables)
    big = torch.zeros(5 * 768 * 2048 + 64, dtype=torch.bfloat16, device=DEV)
    slots = [4, 0, 2]
    tb = [big[s * 768 * 2048 + 8:(s + 1) * 768 * 2048 + 8].view(768, 2048) for s in slots]
    for t, m in zip(tb, mats):
        t.copy_(m)
    ctx.newton_schulz(tb, None, params=p)
    torch.cuda.synchronize()
    for x, y, z, w in zip(o1, o2, ip, tb):
        assert torch.equal(x, y)
        assert torch.equal(x, z)
        assert torch.equal(x, w)


def test_gram_zero_units_exact(ctx):
    g = gen(9)
    mats = [synth.normal((256, 768), 1e-3, g, DEV, torch.bfloat16) for _ in range(3)]
    mats[1].zero_()
    out = [torch.full_like(m, 7.0) for m in mats]
    ctx.newton_schulz(mats, out, params=ns_params(method="gram"))
    torch.cuda.synchronize()
    assert not torch.any(out[1])
    assert oracle.rel_fro(host(out[0]), oracle.ns_ref(host(mats[0]))) <= BF16_TOL
    z = [torch.zeros((40, 72), device=DEV), synth.normal((40, 72), 1.0, g, DEV, torch.float32)]
    zo = [torch.full_like(t, 3.0) for t in z]
    ctx.newton_schulz(z, zo, params=ns_params(compute="f32", method="gram"))
    torch.cuda.synchronize()
    assert not torch.any(zo[0])
    assert oracle.rel_fro(host(zo[1]), oracle.ns_ref(host(z[1]))) <= F32_TOL


def test_gram_rejects_unknown_method(ctx):
    m = [torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)]
    p = ns_params()
    p.method = 7
    with pytest.raises(MuonError) as e:
        ctx.newton_schulz(m, [torch.empty_like(m[0])], params=p)
    assert e.value.status == 1


def test_gram_per_head_workload_sampled():
    # per-head q/k/v of Qwen3-4B (128 x 2560 heads): 6 layers, every head of
    # the first and last matrix of each layer checked
    w = synth.qwen3_4b_heads(layers=6)
    c = Context(DEV, 2 << 30)
    g = gen(w.seed)
    mats = [synth.normal((m.rows, m.cols), w.grad_std, g, DEV, torch.bfloat16) for m in w.mats]
    out = [torch.empty_like(x) for x in mats]
    by_shape = {}
    for i, m in enumerate(w.mats):
        by_shape.setdefault((m.rows, m.cols, m.head_rows), []).append(i)
    p = ns_params(method="gram")
    for (r, cl, h), idx in by_shape.items():
        c.newton_schulz([mats[i] for i in idx], [out[i] for i in idx], h, p)
    torch.cuda.synchronize()
    worst = 0.0
    for i in (0, len(mats) - 1):
        m = w.mats[i]
        ref = oracle.ns_ref_heads(host(mats[i]), m.head_rows)
        got = host(out[i])
        for k in range(m.rows // m.head_rows):
            sl = slice(k * m.head_rows, (k + 1) * m.head_rows)
            worst = max(worst, oracle.rel_fro(got[sl], ref[sl]))
    say(f"  gram-ns per-head sampled: max rel err {worst:.3e}")
    assert worst <= BF16_TOL
    c.close()
