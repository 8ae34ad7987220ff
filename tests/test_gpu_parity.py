"""Parity of the HIP path with the CPU oracle (needs a gfx950 GPU).

Bars: momentum and apply bit-exact (binary32 and their bf16 casts); Newton-
Schulz relative Frobenius error per unit <= 2e-2 in bf16 mode and <= 1e-4 in
fp32 mode; zero units exactly zero; identical inputs give identical bits.
Inputs are seeded synthetic draws (newton_schulz_amd.synth); the oracle gets
exact host copies of the device inputs.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_amd import Context, MuonError, MuonStep, ns_params
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


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bits32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int32).numpy().view(np.uint32)


def gen(seed):
    return torch.Generator(device=DEV).manual_seed(seed)


# ---------------------------------------------------------------------------
# momentum and apply: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gdt,udt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)])
# aligned sizes take the one-shot vector path (4096 elements per workgroup, a
# partial last workgroup and a scalar tail of numel % 8); offsets that break
# 16-byte alignment take the grid-stride scalar path
@pytest.mark.parametrize("numel,offset", [(1, 0), (4099, 0), (1 << 20, 0), (3 * 4096 + 8 * 37 + 5, 0),
                                          (100003, 1), (8 * 1000 + 5, 3)])
@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_bitexact(ctx, gdt, udt, numel, offset, nesterov):
    say(f"momentum {gdt} -> {udt} numel={numel} offset={offset} nesterov={nesterov}")
    g = gen(numel + offset)
    grad = synth.normal((numel + offset,), 1e-3, g, DEV, gdt)[offset:]
    mom = synth.normal((numel + offset,), 1e-3, g, DEV, torch.float32)[offset:]
    upd = torch.empty(numel + offset, dtype=udt, device=DEV)[offset:]
    g_h, m_h = host(grad), host(mom)
    ctx.momentum_update(grad, mom, upd, 0.95, nesterov)
    torch.cuda.synchronize()
    m_ref, u_ref = oracle.momentum_ref(g_h, m_h, 0.95, nesterov)
    assert np.array_equal(bits32(mom), m_ref.view(np.uint32))
    if udt == torch.bfloat16:
        assert np.array_equal(bits16(upd), oracle.bf16_bits(u_ref))
    else:
        assert np.array_equal(bits32(upd), u_ref.view(np.uint32))


@pytest.mark.parametrize("udt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("numel,offset", [(7, 0), (1 << 20, 0), (3 * 4096 + 8 * 37 + 5, 0), (65541, 1)])
@pytest.mark.parametrize("wd,want_bf16", [(0.0, True), (0.1, False), (0.0, False)])
def test_apply_bitexact(ctx, udt, numel, offset, wd, want_bf16):
    say(f"apply {udt} numel={numel} offset={offset} wd={wd} bf16={want_bf16}")
    g = gen(7 * numel + offset)
    W = synth.normal((numel + offset,), 0.02, g, DEV, torch.float32)[offset:]
    u = synth.normal((numel + offset,), 1.0, g, DEV, udt)[offset:]
    wb = torch.empty(numel + offset, dtype=torch.bfloat16, device=DEV)[offset:] if want_bf16 else None
    W_h, u_h = host(W), host(u)
    ctx.apply(W, u, 0.02, 1.5, wd, wb)
    torch.cuda.synchronize()
    res = oracle.apply_ref(W_h, u_h, 0.02, 1.5, wd, bf16_copy=want_bf16)
    W_ref = res[0] if want_bf16 else res
    assert np.array_equal(bits32(W), W_ref.view(np.uint32))
    if want_bf16:
        assert np.array_equal(bits16(wb), res[1])


def test_apply_zero_update_keeps_weights(ctx):
    W = synth.normal((10007,), 0.02, gen(3), DEV, torch.float32)
    before = bits32(W)
    ctx.apply(W, torch.zeros(10007, dtype=torch.bfloat16, device=DEV), 0.02)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(W), before)


# ---------------------------------------------------------------------------
# Newton-Schulz against the oracle
# ---------------------------------------------------------------------------
def ns_check(ctx, rows, cols, count, dtype, tol, head_rows=0, seed=0, steps=5, std=1e-3):
    g = gen(seed)
    mats = [synth.normal((rows, cols), std, g, DEV, dtype) for _ in range(count)]
    ins = [host(m) for m in mats]
    out = [torch.empty_like(m) for m in mats]
    p = ns_params(steps=steps, compute="bf16" if dtype == torch.bfloat16 else "f32")
    ctx.newton_schulz(mats, out, head_rows, p)
    torch.cuda.synchronize()
    errs = []
    for x, o in zip(ins, out):
        ref = oracle.ns_ref_heads(x, head_rows, steps=steps)
        got = host(o)
        if head_rows:
            for k in range(rows // head_rows):
                sl = slice(k * head_rows, (k + 1) * head_rows)
                errs.append(oracle.rel_fro(got[sl], ref[sl]))
        else:
            errs.append(oracle.rel_fro(got, ref))
    say(f"  ns {rows}x{cols} x{count} {dtype} h={head_rows} steps={steps}: max rel err {max(errs):.3e}")
    assert max(errs) <= tol, errs
    return out


@pytest.mark.parametrize("rows,cols", [(64, 128), (128, 128), (256, 64), (96, 96), (72, 200), (300, 40)])
def test_ns_fp32(ctx, rows, cols):
    ns_check(ctx, rows, cols, 3, torch.float32, F32_TOL, seed=rows * cols, std=1.0)


@pytest.mark.parametrize("rows,cols", [(256, 256), (520, 1048), (1048, 520), (264, 264), (128, 2560),
                                       (2560, 128), (768, 2048), (2048, 768), (384, 640)])
def test_ns_bf16_mfma(ctx, rows, cols):
    ns_check(ctx, rows, cols, 3, torch.bfloat16, BF16_TOL, seed=rows + cols)


@pytest.mark.parametrize("rows,cols", [(202, 618), (618, 202), (130, 130)])
def test_ns_bf16_generic_shapes(ctx, rows, cols):
    ns_check(ctx, rows, cols, 2, torch.bfloat16, BF16_TOL, seed=rows * 3 + cols)


# degenerate shapes: one row or column (the normalised unit is its own polar
# factor's direction with singular value 1), a single element, shapes far
# below one tile, and sides that are not multiples of 8 (generic kernels)
@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 64), (64, 1), (1, 7), (3, 5), (5, 3), (8, 8), (1, 4096),
                                       (4096, 1), (2, 2)])
def test_ns_degenerate_shapes(ctx, rows, cols):
    ns_check(ctx, rows, cols, 2, torch.bfloat16, BF16_TOL, seed=rows * 7 + cols)
    ns_check(ctx, rows, cols, 2, torch.float32, F32_TOL, seed=rows * 7 + cols, std=1.0)


# heads of fewer than 16 rows take the fp32 iteration too, per head
@pytest.mark.parametrize("rows,cols,h", [(64, 96, 8), (24, 40, 4), (48, 3, 16)])
def test_ns_small_heads(ctx, rows, cols, h):
    ns_check(ctx, rows, cols, 2, torch.bfloat16, BF16_TOL, head_rows=h, seed=rows + cols + h)


@pytest.mark.parametrize("steps", [0, 1, 2, 6])
def test_ns_step_counts(ctx, steps):
    ns_check(ctx, 256, 512, 2, torch.bfloat16, BF16_TOL, seed=steps, steps=steps)
    ns_check(ctx, 96, 160, 2, torch.float32, F32_TOL, seed=steps, steps=steps, std=1.0)


def test_ns_per_head_and_shards(ctx):
    h, heads, cols = 128, 6, 640
    out = ns_check(ctx, h * heads, cols, 2, torch.bfloat16, BF16_TOL, head_rows=h, seed=11)
    # a row shard of heads gives bitwise the same rows as the whole per-head call
    g = gen(11)
    mats = [synth.normal((h * heads, cols), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    shard = [m[2 * h:5 * h].contiguous() for m in mats]
    sout = [torch.empty_like(s) for s in shard]
    ctx.newton_schulz(shard, sout, h)
    torch.cuda.synchronize()
    for full, part in zip(out, sout):
        assert torch.equal(full[2 * h:5 * h], part)


def test_ns_whole_matrix_differs_from_per_head(ctx):
    g = gen(5)
    m = synth.normal((512, 640), 1e-3, g, DEV, torch.bfloat16)
    a, b = torch.empty_like(m), torch.empty_like(m)
    ctx.newton_schulz([m], [a], 0)
    ctx.newton_schulz([m], [b], 128)
    torch.cuda.synchronize()
    assert oracle.rel_fro(host(a), host(b)) > 0.05


def test_ns_deterministic(ctx):
    g = gen(21)
    mats = [synth.normal((768, 2048), 1e-3, g, DEV, torch.bfloat16) for _ in range(4)]
    o1 = [torch.empty_like(m) for m in mats]
    o2 = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, o1)
    ctx.newton_schulz(mats, o2)
    torch.cuda.synchronize()
    for x, y in zip(o1, o2):
        assert torch.equal(x, y)


def test_ns_zero_units_exact(ctx):
    g = gen(9)
    mats = [synth.normal((256, 768), 1e-3, g, DEV, torch.bfloat16) for _ in range(3)]
    mats[1].zero_()
    out = [torch.full_like(m, 7.0) for m in mats]
    ctx.newton_schulz(mats, out)
    torch.cuda.synchronize()
    assert not torch.any(out[1])
    ref = oracle.ns_ref(host(mats[0]))
    assert oracle.rel_fro(host(out[0]), ref) <= BF16_TOL
    # fp32 and generic path too
    z = [torch.zeros((40, 72), device=DEV), synth.normal((40, 72), 1.0, g, DEV, torch.float32)]
    zo = [torch.full_like(t, 3.0) for t in z]
    ctx.newton_schulz(z, zo, params=ns_params(compute="f32"))
    torch.cuda.synchronize()
    assert not torch.any(zo[0])


@pytest.mark.parametrize("shape", [(768, 2048), (2048, 768), (256, 512)])
def test_ns_zero_units_take_no_slot(ctx, shape):
    """The updates run over a device-built list of the nonzero units: with
    zero units interleaved (and an all-zero call) every nonzero unit equals,
    bit for bit, the same unit in a call without the zero ones, and the zero
    units come out exactly zero."""
    g = gen(12)
    zero = {0, 3, 4, 9, 11}
    mats = [synth.normal(shape, 1e-3, g, DEV, torch.bfloat16) for _ in range(12)]
    for i in zero:
        mats[i].zero_()
    out = [torch.full_like(m, 5.0) for m in mats]
    ctx.newton_schulz(mats, out)
    dense = [m for i, m in enumerate(mats) if i not in zero]
    dout = [torch.empty_like(m) for m in dense]
    ctx.newton_schulz(dense, dout)
    allz = [torch.zeros_like(mats[0]) for _ in range(3)]
    zout = [torch.full_like(m, 5.0) for m in allz]
    ctx.newton_schulz(allz, zout)
    torch.cuda.synchronize()
    k = 0
    for i in range(12):
        if i in zero:
            assert not torch.any(out[i]), i
        else:
            assert torch.equal(out[i], dout[k]), i
            k += 1
    assert all(not torch.any(z) for z in zout)
    ref = oracle.ns_ref(host(mats[1]))
    assert oracle.rel_fro(host(out[1]), ref) <= BF16_TOL


def test_ns_nonfinite_flag(ctx):
    g = gen(4)
    mats = [synth.normal((128, 256), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctx.newton_schulz(mats, [torch.empty_like(m) for m in mats], nonfinite_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    mats[1][3, 5] = float("inf")
    ctx.newton_schulz(mats, [torch.empty_like(m) for m in mats], nonfinite_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1


def test_ns_in_place_and_tables(ctx):
    g = gen(13)
    base = [synth.normal((264, 520), 1e-3, g, DEV, torch.bfloat16) for _ in range(5)]
    ref = [torch.empty_like(b) for b in base]
    ctx.newton_schulz(base, ref)
    # irregularly placed inputs and outputs (device pointer table path)
    big = torch.zeros(7 * 264 * 520 + 64, dtype=torch.bfloat16, device=DEV)
    slots = [6, 0, 3, 1, 5]
    ins = [big[s * 264 * 520 + 8: (s + 1) * 264 * 520 + 8].view(264, 520) for s in slots]
    for i, b in zip(ins, base):
        i.copy_(b)
    ctx.newton_schulz(ins, None)  # in place
    torch.cuda.synchronize()
    for x, y in zip(ins, ref):
        assert torch.equal(x, y)


def test_ns_errors(ctx):
    small = Context(DEV, 1 << 16)
    m = [torch.zeros((512, 512), dtype=torch.bfloat16, device=DEV)]
    with pytest.raises(MuonError) as e:
        small.newton_schulz(m, [torch.empty_like(m[0])])
    assert e.value.status == 4
    with pytest.raises(MuonError) as e:
        ctx.newton_schulz(m, [torch.empty_like(m[0])], head_rows=100)
    assert e.value.status == 2
    with pytest.raises(MuonError) as e:
        ctx.newton_schulz(m, [torch.empty_like(m[0])], params=ns_params(compute="f32"))
    assert e.value.status == 3
    with pytest.raises(MuonError):
        x = torch.zeros(100, device=DEV)
        ctx.momentum_update(x, x, torch.zeros(100, device=DEV))  # grad aliases momentum
    small.close()


def test_empty_calls_are_noops(ctx):
    e = torch.zeros(0, device=DEV)
    ctx.momentum_update(e, e.clone(), e.clone())
    ctx.apply(e, e.clone(), 0.02)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# whole optimizer steps on the workloads
# ---------------------------------------------------------------------------
def build_step(w: synth.Workload, keep_bf16=False):
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    gdt = w.grad_dtype
    ms = MuonStep(shapes, DEV, lr=w.lr, beta=w.beta, nesterov=w.nesterov, compute=w.compute,
                  grad_dtype=gdt, cap_bytes=w.cap_bytes, cap_kind=w.cap_kind, ns_steps=w.ns_steps,
                  keep_bf16_weights=keep_bf16)
    g = gen(w.seed)
    for i, W0 in enumerate(synth.draw_weights(w, g, DEV)):
        ms.view(ms.master, i).copy_(W0)
    return ms, g


def fill_grads(ms, w, g):
    synth.draw_grads(w, g, DEV, out=[ms.view(ms.grad, i) for i in range(len(w.mats))])


def test_tiny_fp32_three_steps(ctx):
    w = synth.tiny()
    ms, g = build_step(w)
    n = len(w.mats)
    W = [host(ms.view(ms.master, i)) for i in range(n)]
    W0 = [x.copy() for x in W]
    M = [np.zeros_like(x) for x in W]
    for step in range(w.steps):
        fill_grads(ms, w, g)
        G = [host(ms.view(ms.grad, i)) for i in range(n)]
        ms.step()
        torch.cuda.synchronize()
        oracle.muon_step_ref(W, G, M, w.lr, w.beta, w.nesterov)
        for i in range(n):
            assert np.array_equal(bits32(ms.view(ms.momentum, i)), M[i].view(np.uint32)), (step, i)
            got = host(ms.view(ms.master, i)).astype(np.float64) - W0[i]
            err = oracle.rel_fro(got, W[i].astype(np.float64) - W0[i])
            say(f"  tiny step {step} matrix {i}: dW rel err {err:.3e}")
            assert err <= F32_TOL


def check_sampled(ms, w, picks, M_before, W_before, G):
    for i in picks:
        m_ref, u_ref = oracle.momentum_ref(G[i], M_before[i], w.beta, w.nesterov)
        assert np.array_equal(bits32(ms.view(ms.momentum, i)), m_ref.view(np.uint32)), i
        O = oracle.ns_ref_heads(oracle.bf16_round(u_ref), w.mats[i].head_rows)
        dW = host(ms.view(ms.master, i)).astype(np.float64) - W_before[i]
        if w.mats[i].zero_grad:
            assert not np.any(dW), i
            continue
        # per Newton-Schulz unit: each head of a per-head matrix on its own
        h = w.mats[i].head_rows or w.mats[i].rows
        errs = [oracle.rel_fro(dW[k:k + h], -np.float32(w.lr) * O[k:k + h])
                for k in range(0, w.mats[i].rows, h)]
        err = max(errs)
        say(f"  {w.mats[i].name} {w.mats[i].rows}x{w.mats[i].cols} ({len(errs)} unit(s)): "
            f"max dW rel err {err:.3e}")
        assert err <= BF16_TOL, (i, err)


def test_qwen3_4b_layer_all_matrices():
    w = synth.qwen3_4b_layer()
    ms, g = build_step(w, keep_bf16=True)
    fill_grads(ms, w, g)
    n = len(w.mats)
    G = [host(ms.view(ms.grad, i)) for i in range(n)]
    M0 = [host(ms.view(ms.momentum, i)) for i in range(n)]
    W0 = [host(ms.view(ms.master, i)).astype(np.float64) for i in range(n)]
    ms.step()
    torch.cuda.synchronize()
    check_sampled(ms, w, range(n), M0, W0, G)
    for i in range(n):
        assert np.array_equal(bits16(ms.view(ms.weight_bf16, i)),
                              oracle.bf16_bits(host(ms.view(ms.master, i))))


def test_qwen3_4b_full_model_sampled():
    w = synth.qwen3_4b()  # 36 layers, 512 MiB micro-buckets, 2 momentum warm-up steps
    ms, g = build_step(w)
    for _ in range(w.warmup_momentum_steps):
        fill_grads(ms, w, g)
        ms.momentum_only()
    fill_grads(ms, w, g)
    # the first and last matrix of every micro-bucket, plus 8 seeded picks;
    # MUON_PARITY_FULL=1: all 252 matrices (some minutes of fp64 on the host)
    rng = np.random.default_rng(2)
    picks = {b.indices[0] for b in ms.plan.buckets} | {b.indices[-1] for b in ms.plan.buckets}
    picks |= {int(x) for x in rng.choice(len(w.mats), 8, replace=False)}
    if os.environ.get("MUON_PARITY_FULL") == "1":
        picks = set(range(len(w.mats)))
    picks = sorted(picks)
    say(f"  qwen3_4b: {len(ms.plan.buckets)} micro-buckets, {len(picks)} matrices checked")
    G = {i: host(ms.view(ms.grad, i)) for i in picks}
    M0 = {i: host(ms.view(ms.momentum, i)) for i in picks}
    W0 = {i: host(ms.view(ms.master, i)).astype(np.float64) for i in picks}
    ms.step()
    torch.cuda.synchronize()
    check_sampled(ms, w, picks, M0, W0, G)


def test_qwen3_4b_per_head_all():
    # every one of the 1728 heads (32 q + 8 k + 8 v per layer, 36 layers)
    w = synth.qwen3_4b_heads(layers=36)
    ms, g = build_step(w)
    assert len(ms.plan.buckets) == 1 and ms.plan.buckets[0].units == 1728
    fill_grads(ms, w, g)
    n = len(w.mats)
    G = [host(ms.view(ms.grad, i)) for i in range(n)]
    W0 = [host(ms.view(ms.master, i)).astype(np.float64) for i in range(n)]
    M0 = [np.zeros_like(x) for x in G]
    ms.step()
    torch.cuda.synchronize()
    assert sum(m.rows // m.head_rows for m in w.mats) == 1728
    check_sampled(ms, w, range(n), M0, W0, G)


def test_moe_experts_two_layers():
    w = synth.qwen3_30b_experts(layers=2)
    ms, g = build_step(w)
    assert all(b.workspace_bytes <= w.cap_bytes for b in ms.plan.buckets)
    fill_grads(ms, w, g)
    n = len(w.mats)
    zero = [i for i in range(n) if w.mats[i].zero_grad]
    rng = np.random.default_rng(4)
    picks = sorted(set(rng.integers(0, n, 10).tolist()) | set(zero[:3]))
    G = {i: host(ms.view(ms.grad, i)) for i in picks}
    M0 = {i: host(ms.view(ms.momentum, i)) for i in picks}
    W0 = {i: host(ms.view(ms.master, i)).astype(np.float64) for i in picks}
    Wz = {i: bits32(ms.view(ms.master, i)) for i in zero}
    ms.step()
    torch.cuda.synchronize()
    check_sampled(ms, w, picks, M0, W0, G)
    for i in zero:  # experts without gradient keep their weights bit for bit
        assert np.array_equal(bits32(ms.view(ms.master, i)), Wz[i])
