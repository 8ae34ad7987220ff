"""The fused whole-iteration Newton-Schulz of small wide units (m <= 128).

It computes the quintic iteration, or its Gram form, with the unfused
kernels' rounding points, MFMA shape and summation order, so its output must
equal theirs bit for bit (fuse "on" against fuse "off" on the same inputs);
against the CPU oracle the bf16 bar holds (relative Frobenius error per unit
<= 2e-2).  Eligibility and the automatic choice are checked through the
per-class launch counts.
"""
import sys

import pytest
import torch

import oracle
from newton_schulz_amd import Context, ns_params
from newton_schulz_amd import synth

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Context(DEV, 1 << 30)
    c.timing_enable(True, 4096)
    yield c
    c.close()


def host(t):
    return t.detach().float().cpu().numpy()


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def launches(ctx, fn):
    ctx.timing_reset()
    fn()
    torch.cuda.synchronize()
    t = ctx.timing_read()
    return t["fused"][1], t["update"][1]


def both(ctx, mats, head_rows=0, steps=5, method="quintic"):
    a = [torch.empty_like(m) for m in mats]
    b = [torch.empty_like(m) for m in mats]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(mats, a, head_rows,
                                                    ns_params(steps=steps, method=method, fuse="on")))
    nu, upd = launches(ctx, lambda: ctx.newton_schulz(mats, b, head_rows,
                                                      ns_params(steps=steps, method=method, fuse="off")))
    assert nf == 1 and nu == 0 and upd == (steps if method == "quintic" else 1), (nf, nu, upd)
    return a, b


def check_oracle(mats, outs, head_rows=0, steps=5, picks=None):
    worst = 0.0
    for i in (picks if picks is not None else range(len(mats))):
        ref = oracle.ns_ref_heads(host(mats[i]), head_rows, steps=steps)
        got = host(outs[i])
        hs = head_rows or got.shape[0]
        for k in range(got.shape[0] // hs):
            sl = slice(k * hs, (k + 1) * hs)
            worst = max(worst, oracle.rel_fro(got[sl], ref[sl]))
    return worst


@pytest.mark.parametrize("rows,cols,count", [(128, 2560, 3), (64, 512, 2), (120, 1000, 2), (128, 136, 3),
                                             (16, 64, 2), (128, 128, 2), (96, 4096, 1), (16, 24, 3)])
def test_fused_equals_unfused_and_oracle(ctx, rows, cols, count):
    g = gen(rows * 31 + cols)
    mats = [synth.normal((rows, cols), 1e-3, g, DEV, torch.bfloat16) for _ in range(count)]
    a, b = both(ctx, mats)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    worst = check_oracle(mats, a)
    say(f"  fused {rows}x{cols} x{count}: bit-identical to unfused; max rel err {worst:.3e}")
    assert worst <= BF16_TOL


@pytest.mark.parametrize("steps", [1, 2, 3, 6])
def test_fused_step_counts(ctx, steps):
    g = gen(100 + steps)
    mats = [synth.normal((128, 640), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    a, b = both(ctx, mats, steps=steps)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert check_oracle(mats, a, steps=steps) <= BF16_TOL


def test_fused_per_head_and_in_place(ctx):
    h, heads, cols = 128, 6, 2560
    g = gen(7)
    mats = [synth.normal((h * heads, cols), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    a, b = both(ctx, mats, head_rows=h)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert check_oracle(mats, a, head_rows=h) <= BF16_TOL
    # in place, unit for unit (output = input)
    ip = [m.clone() for m in mats]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(ip, None, h, ns_params(fuse="on")))
    assert nf == 1
    for x, y in zip(a, ip):
        assert torch.equal(x, y)
    # in place with one step: each block is read before it is overwritten
    ip1 = [m.clone() for m in mats]
    ref1 = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, ref1, h, ns_params(steps=1, fuse="off"))
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(ip1, None, h, ns_params(steps=1, fuse="on")))
    assert nf == 1
    for x, y in zip(ref1, ip1):
        assert torch.equal(x, y)


def test_fused_irregular_placement_and_zero_units(ctx):
    g = gen(11)
    rows, cols = 128, 768
    mats = [synth.normal((rows, cols), 1e-3, g, DEV, torch.bfloat16) for _ in range(4)]
    mats[2].zero_()
    big = torch.zeros(6 * rows * cols + 64, dtype=torch.bfloat16, device=DEV)
    slots = [5, 0, 3, 1]
    ins = [big[s * rows * cols + 8:(s + 1) * rows * cols + 8].view(rows, cols) for s in slots]
    for t, m in zip(ins, mats):
        t.copy_(m)
    out = [torch.full_like(m, 7.0) for m in mats]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(ins, out, 0, ns_params(fuse="on")))
    assert nf == 1
    ref = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, ref, 0, ns_params(fuse="off"))
    torch.cuda.synchronize()
    assert not torch.any(out[2])
    for x, y in zip(out, ref):
        assert torch.equal(x, y)


# units whose smaller side is under 16 run the iteration in fp32 (bf16 A and B'
# alone take some of their Gaussian draws past the bar): never fused, the same
# bits with fusion on or off, and well inside the bar
@pytest.mark.parametrize("rows,cols,count", [(8, 64, 2), (8, 8, 3), (64, 8, 2)])
def test_tiny_units_run_in_fp32(ctx, rows, cols, count):
    g = gen(rows * 13 + cols)
    mats = [synth.normal((rows, cols), 1e-3, g, DEV, torch.bfloat16) for _ in range(count)]
    a = [torch.empty_like(m) for m in mats]
    b = [torch.empty_like(m) for m in mats]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(mats, a, 0, ns_params(fuse="on")))
    launches(ctx, lambda: ctx.newton_schulz(mats, b, 0, ns_params(fuse="off")))
    assert nf == 0
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    worst = check_oracle(mats, a)
    say(f"  {rows}x{cols} x{count}: fp32 iteration, max rel err {worst:.3e}")
    # the fp32 iteration's own error is ~1e-7; the bf16 output adds at most
    # 2^-9 relative per element
    assert worst <= 2.0 ** -8


# the Gram form (bf16: units with 2 m <= n) fuses as well
@pytest.mark.parametrize("rows,cols,count", [(128, 2560, 3), (64, 512, 2), (128, 256, 2), (96, 4096, 1),
                                             (16, 64, 2), (120, 1000, 2)])
def test_fused_gram_form_equals_unfused_and_oracle(ctx, rows, cols, count):
    g = gen(rows * 17 + cols)
    mats = [synth.normal((rows, cols), 1e-3, g, DEV, torch.bfloat16) for _ in range(count)]
    a, b = both(ctx, mats, method="gram")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    worst = check_oracle(mats, a)
    say(f"  fused gram form {rows}x{cols} x{count}: bit-identical to unfused; max rel err {worst:.3e}")
    assert worst <= BF16_TOL


@pytest.mark.parametrize("steps", [1, 2, 3, 6])
def test_fused_gram_form_step_counts_and_in_place(ctx, steps):
    g = gen(200 + steps)
    h = 128
    mats = [synth.normal((3 * h, 1024), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    mats[1][h:2 * h].zero_()  # one zero head
    a, b = both(ctx, mats, head_rows=h, steps=steps, method="gram")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.any(a[1][h:2 * h])
    assert check_oracle(mats, a, head_rows=h, steps=steps) <= BF16_TOL
    ip = [m.clone() for m in mats]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(ip, None, h, ns_params(steps=steps, method="gram",
                                                                            fuse="on")))
    assert nf == 1
    for x, y in zip(a, ip):
        assert torch.equal(x, y)


def test_fused_eligibility(ctx):
    g = gen(13)
    # tall units, m > 128 and fp32 compute are never fused
    tall = [synth.normal((256, 64), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(tall, [torch.empty_like(t) for t in tall], 0,
                                                    ns_params(fuse="on")))
    assert nf == 0
    wide = [synth.normal((256, 512), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(wide, [torch.empty_like(t) for t in wide], 0,
                                                    ns_params(fuse="on")))
    assert nf == 0
    f32 = [synth.normal((64, 128), 1.0, g, DEV, torch.float32) for _ in range(2)]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(f32, [torch.empty_like(t) for t in f32], 0,
                                                    ns_params(compute="f32", fuse="on")))
    assert nf == 0
    # the Gram form on a near-square unit runs the quintic (bf16: 2 m > n), fused
    sq = [synth.normal((128, 200), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    o1 = [torch.empty_like(t) for t in sq]
    o2 = [torch.empty_like(t) for t in sq]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(sq, o1, 0, ns_params(method="gram", fuse="on")))
    assert nf == 1
    ctx.newton_schulz(sq, o2, 0, ns_params(fuse="off"))
    torch.cuda.synchronize()
    for x, y in zip(o1, o2):
        assert torch.equal(x, y)
    # an output that overlaps another unit's input is not fused (and is right)
    buf = synth.normal((3 * 128 * 512,), 1e-3, g, DEV, torch.bfloat16)
    ins = [buf[i * 128 * 512:(i + 1) * 128 * 512].view(128, 512) for i in range(2)]
    ref = [torch.empty_like(t) for t in ins]
    ctx.newton_schulz([t.clone() for t in ins], ref, 0, ns_params(fuse="off"))
    outs = [buf[(i + 1) * 128 * 512:(i + 2) * 128 * 512].view(128, 512) for i in range(2)]
    src = [t for t in ins]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(src, outs, 0, ns_params(fuse="on")))
    assert nf == 0
    for x, y in zip(ref, outs):
        assert torch.equal(x, y)
    # auto: fused for units of at most 3072 columns, and for wider ones once
    # the call has a unit for every compute unit
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    few = [synth.normal((128, 256), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(few, [torch.empty_like(t) for t in few], 0, ns_params()))
    assert nf == 1
    wide_few = [synth.normal((128, 4096), 1e-3, g, DEV, torch.bfloat16) for _ in range(2)]
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(wide_few, [torch.empty_like(t) for t in wide_few], 0,
                                                    ns_params()))
    assert nf == 0
    many = synth.normal((cus, 128, 3200), 1e-3, g, DEV, torch.bfloat16)
    mm = list(many.unbind(0))
    nf, _ = launches(ctx, lambda: ctx.newton_schulz(mm, [torch.empty_like(t) for t in mm], 0, ns_params()))
    assert nf == 1


def test_fused_per_head_workload_sampled():
    # the per-head q/k/v of Qwen3-4B (1728 heads of 128 x 2560) take the fused
    # path by default; sampled against the oracle and against the unfused path
    w = synth.qwen3_4b_heads(layers=36)
    c = Context(DEV, 4 << 30)
    c.timing_enable(True, 64)
    g = gen(w.seed)
    mats = [synth.normal((m.rows, m.cols), w.grad_std, g, DEV, torch.bfloat16) for m in w.mats]
    by_shape = {}
    for i, m in enumerate(w.mats):
        by_shape.setdefault((m.rows, m.cols, m.head_rows), []).append(i)
    out = [torch.empty_like(x) for x in mats]
    c.timing_reset()
    for (r, cl, h), idx in by_shape.items():
        c.newton_schulz([mats[i] for i in idx], [out[i] for i in idx], h, ns_params())
    torch.cuda.synchronize()
    assert c.timing_read()["fused"][1] == len(by_shape)
    picks = [0, 1, 2, len(mats) - 1]
    ref = [torch.empty_like(mats[i]) for i in picks]
    for i, rt in zip(picks, ref):
        c.newton_schulz([mats[i]], [rt], w.mats[i].head_rows, ns_params(fuse="off"))
    torch.cuda.synchronize()
    for i, rt in zip(picks, ref):
        assert torch.equal(out[i], rt)
    worst = check_oracle(mats, out, head_rows=128, picks=[0, len(mats) - 1])
    say(f"  fused per-head workload: max rel err {worst:.3e}")
    assert worst <= BF16_TOL
    c.close()


def test_step_merges_head_units_bit_identical():
    """MuonStep passes the heads of a micro-bucket's per-head q and k/v
    projections as one call of 128 x 2560 units (one fused launch instead of
    one per shape); the update it applies equals per-matrix calls with
    head_rows, bit for bit, momentum and apply included."""
    from newton_schulz_amd import MuonStep
    w = synth.qwen3_4b_heads(layers=6)
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    ms = MuonStep(shapes, DEV, lr=w.lr, beta=w.beta, nesterov=w.nesterov, cap_bytes=w.cap_bytes,
                  keep_bf16_weights=True)
    assert len(ms._work) == 1
    _, _, groups, _ = ms._work[0]
    assert len(groups) == 1 and groups[0][0] == 0 and len(groups[0][1]) == 6 * 48
    g = gen(w.seed)
    ms.grad.copy_(synth.normal((ms.numel,), w.grad_std, g, DEV, torch.bfloat16))
    ms.master.copy_(synth.normal((ms.numel,), 0.02, g, DEV, torch.float32))
    ms.momentum.copy_(synth.normal((ms.numel,), w.grad_std, g, DEV, torch.float32))
    grad, mom, master = ms.grad.clone(), ms.momentum.clone(), ms.master.clone()
    c = Context(DEV, ms.plan.max_workspace)
    c.timing_enable(True, 64)
    ms.ctx.timing_enable(True, 64)
    ms.ctx.timing_reset()
    ms.step()
    # the same step by hand: one call per shape with head_rows
    upd = torch.empty(ms.numel, dtype=torch.bfloat16, device=DEV)
    sq = torch.empty(-(-ms.numel // 4096), dtype=torch.float64, device=DEV)
    c.momentum_update(grad, mom, upd, w.beta, w.nesterov, sq_partials=sq)
    by_shape = {}
    for i, s in enumerate(shapes):
        by_shape.setdefault(s, []).append(i)
    c.timing_reset()
    for (r, cl, h), idx in by_shape.items():
        mats = [upd[ms.offset[i]:ms.offset[i] + r * cl].view(r, cl) for i in idx]
        c.newton_schulz(mats, None, h, ns_params(), sq=(sq, upd))
    wb = torch.empty(ms.numel, dtype=torch.bfloat16, device=DEV)
    c.apply(master, upd, w.lr, 1.0, 0.0, wb)
    torch.cuda.synchronize()
    # 128 x 2560 units fuse at any count: one fused launch for the 288 units
    # of the merged call, one per shape for the per-matrix calls
    assert ms.ctx.timing_read()["fused"][1] == 1
    assert c.timing_read()["fused"][1] == len(by_shape)
    assert torch.equal(ms.momentum, mom)
    assert torch.equal(ms.master, master)
    assert torch.equal(ms.weight_bf16, wb)
    c.close()
