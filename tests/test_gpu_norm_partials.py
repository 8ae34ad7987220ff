"""Norms from the momentum pass (muon_momentum_update_sq + sq_partials).

The momentum kernel leaves, per block of 4096 elements, the binary64 sum of
squares of the update as stored; Newton-Schulz then takes each unit's
Frobenius norm from its blocks instead of reading the update again.  Bars:
momentum and update bit-exact against the oracle as for the plain entry
point; every partial within 1e-12 (relative) of the exactly rounded sum of
its block's squares (oracle.sumsq_blocks over the stored values), and bit-identical
from call to call; Newton-Schulz with partials within 1e-3 of the call that
reads its input for the norm (the two sums differ only in rounding order,
so the float scales almost always agree bit for bit) and within the oracle
bar.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_amd import Context, MuonError, MuonStep, ns_params
from newton_schulz_amd import synth
from newton_schulz_amd.api import SQ_BLOCK, sq_blocks

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
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
    return torch.Generator(device=DEV).manual_seed(seed)


@pytest.mark.parametrize("gdt,udt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.float32, torch.bfloat16)])
# vector path: whole blocks, a partial last block, a scalar tail that opens a
# block of its own (4096 * 256 + 3), a large range; scalar path: offsets that
# break 16-byte alignment
@pytest.mark.parametrize("numel,offset", [(1, 0), (4099, 0), (3 * 4096, 0), (4096 * 256 + 3, 0),
                                          (1 << 20, 0), (100003, 1), (8 * 1000 + 5, 3)])
def test_momentum_sq_partials(ctx, gdt, udt, numel, offset):
    say(f"momentum_sq {gdt} -> {udt} numel={numel} offset={offset}")
    g = gen(numel + offset + 7)
    grad = synth.normal((numel + offset,), 1e-3, g, DEV, gdt)[offset:]
    mom0 = synth.normal((numel + offset,), 1e-3, g, DEV, torch.float32)[offset:]
    mom = mom0.clone()
    upd = torch.empty(numel + offset, dtype=udt, device=DEV)[offset:]
    sq = torch.full((sq_blocks(numel),), float("nan"), dtype=torch.float64, device=DEV)
    g_h, m_h = host(grad), host(mom0)
    ctx.momentum_update(grad, mom, upd, 0.95, True, sq_partials=sq)
    torch.cuda.synchronize()
    m_ref, u_ref = oracle.momentum_ref(g_h, m_h, 0.95, True)
    assert np.array_equal(host(mom), m_ref)
    stored = oracle.bf16_round(u_ref) if udt == torch.bfloat16 else u_ref
    assert np.array_equal(host(upd), stored)
    got = sq.cpu().numpy()
    want = oracle.sumsq_blocks(stored, SQ_BLOCK)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
    # reproducible bit for bit
    mom2 = mom0.clone()
    sq2 = torch.empty_like(sq)
    ctx.momentum_update(grad, mom2, upd, 0.95, True, sq_partials=sq2)
    torch.cuda.synchronize()
    assert torch.equal(sq, sq2)


def flat_update(ctx, shapes_counts, seed, pad=SQ_BLOCK, udt=torch.bfloat16):
    """One flat update buffer (after `pad` leading elements) holding the
    matrices back to back, written by momentum_sq; returns views and partials."""
    total = pad + sum(r * c * n for (r, c), n in shapes_counts)
    g = gen(seed)
    grad = synth.normal((total,), 1e-3, g, DEV, torch.bfloat16)
    mom = synth.normal((total,), 1e-3, g, DEV, torch.float32)
    upd = torch.empty(total, dtype=udt, device=DEV)
    sq = torch.empty(sq_blocks(total), dtype=torch.float64, device=DEV)
    ctx.momentum_update(grad, mom, upd, 0.95, True, sq_partials=sq)
    groups = []
    off = pad
    for (r, c), n in shapes_counts:
        mats = []
        for _ in range(n):
            mats.append(upd[off:off + r * c].view(r, c))
            off += r * c
        groups.append(mats)
    torch.cuda.synchronize()
    return upd, sq, groups


@pytest.mark.parametrize("rows,cols,count,head_rows,method,fuse", [
    (512, 1024, 3, 0, "quintic", "auto"),
    (1024, 512, 2, 0, "quintic", "auto"),     # tall
    (768, 2048, 3, 0, "gram", "auto"),
    (128, 2560, 40, 0, "quintic", "on"),      # fused small units
    (4096, 2560, 1, 128, "quintic", "on"),    # per-head units
    (2560, 4096, 2, 0, "quintic", "auto"),
])
def test_ns_norms_from_partials(ctx, rows, cols, count, head_rows, method, fuse):
    upd, sq, (mats,) = flat_update(ctx, [((rows, cols), count)], seed=rows + cols + count)
    p = ns_params(method=method, fuse=fuse)
    with_sq = [torch.empty_like(m) for m in mats]
    plain = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, with_sq, head_rows, p, sq=(sq, upd))
    ctx.newton_schulz(mats, plain, head_rows, p)
    torch.cuda.synchronize()
    d = max(oracle.rel_fro(host(a), host(b)) for a, b in zip(with_sq, plain))
    x = host(mats[0])
    ref = oracle.ns_ref_heads(x, head_rows)
    err = oracle.rel_fro(host(with_sq[0]), ref)
    say(f"  ns from partials {rows}x{cols} x{count} h={head_rows} {method} fuse={fuse}: "
        f"vs norm pass {d:.2e}, vs oracle {err:.3e}")
    # the two fp64 sums differ only in order, so the float scales agree except
    # in the rare case of a sum on a rounding boundary
    assert d <= 1e-3
    assert err <= BF16_TOL


@pytest.mark.parametrize("rows,cols,count,udt,tol", [
    (512, 1024, 2, torch.float32, 1e-4),    # fp32 verification mode
    (4096, 3, 4, torch.bfloat16, BF16_TOL),  # generic kernels (m = 3), three blocks per unit
    (4096, 3, 4, torch.float32, 1e-4),
])
def test_ns_partials_other_paths(ctx, rows, cols, count, udt, tol):
    upd, sq, (mats,) = flat_update(ctx, [((rows, cols), count)], seed=rows * cols + count, udt=udt)
    p = ns_params(compute="bf16" if udt == torch.bfloat16 else "f32")
    with_sq = [torch.empty_like(m) for m in mats]
    plain = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, with_sq, 0, p, sq=(sq, upd))
    ctx.newton_schulz(mats, plain, 0, p)
    torch.cuda.synchronize()
    d = max(oracle.rel_fro(host(a), host(b)) for a, b in zip(with_sq, plain))
    err = max(oracle.rel_fro(host(o), oracle.ns_ref(host(m))) for o, m in zip(with_sq, mats))
    say(f"  ns from partials {rows}x{cols} x{count} {udt}: vs norm pass {d:.2e}, vs oracle {err:.3e}")
    assert d <= 1e-3 and err <= tol


def test_ns_partials_in_place_and_tables(ctx):
    """In place, and through the device pointer table (irregular order)."""
    upd, sq, (mats,) = flat_update(ctx, [((256, 512), 6)], seed=31)
    p = ns_params()
    ref = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, ref, 0, p, sq=(sq, upd))
    shuffled = [mats[i] for i in (4, 0, 5, 2, 1, 3)]
    out = [torch.empty_like(m) for m in shuffled]
    ctx.newton_schulz(shuffled, out, 0, p, sq=(sq, upd))
    torch.cuda.synchronize()
    for o, i in zip(out, (4, 0, 5, 2, 1, 3)):
        assert torch.equal(o, ref[i])
    ctx.newton_schulz(mats, None, 0, p, sq=(sq, upd))
    torch.cuda.synchronize()
    for m, r in zip(mats, ref):
        assert torch.equal(m, r)


def test_ns_partials_rejected_when_not_on_blocks(ctx):
    upd, sq, (mats,) = flat_update(ctx, [((256, 512), 2)], seed=5)
    p = ns_params()
    out = [torch.empty_like(m) for m in mats]
    # a matrix that starts 8 elements past a block boundary
    shifted = upd[SQ_BLOCK + 8:SQ_BLOCK + 8 + 256 * 512].view(256, 512)
    with pytest.raises(MuonError):
        ctx.newton_schulz([shifted], [out[0]], 0, p, sq=(sq, upd))
    # partials that end before the last matrix does
    with pytest.raises(MuonError):
        ctx.newton_schulz(mats, out, 0, p, sq=(sq[:sq.numel() - 1], upd))
    # a base past the matrices
    with pytest.raises(MuonError):
        ctx.newton_schulz(mats, out, 0, p, sq=(sq, upd.data_ptr() + 2 * SQ_BLOCK * 2 * 512))
    # units that do not span whole blocks (96 x 96 = 9216 elements)
    small = upd[:96 * 96].view(96, 96)
    with pytest.raises(MuonError):
        ctx.newton_schulz([small], [torch.empty_like(small)], 0, p, sq=(sq, upd))


def test_zero_and_nonfinite_from_partials(ctx):
    total = SQ_BLOCK + 2 * 256 * 512
    grad = torch.zeros(total, dtype=torch.bfloat16, device=DEV)
    mom = torch.zeros(total, dtype=torch.float32, device=DEV)
    grad[SQ_BLOCK + 256 * 512:] = synth.normal((256 * 512,), 1e-3, gen(2), DEV, torch.bfloat16)
    upd = torch.empty(total, dtype=torch.bfloat16, device=DEV)
    sq = torch.empty(sq_blocks(total), dtype=torch.float64, device=DEV)
    ctx.momentum_update(grad, mom, upd, 0.95, True, sq_partials=sq)
    mats = [upd[SQ_BLOCK + k * 256 * 512:SQ_BLOCK + (k + 1) * 256 * 512].view(256, 512) for k in range(2)]
    out = [torch.full_like(m, 3.0) for m in mats]
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctx.newton_schulz(mats, out, 0, ns_params(), nonfinite_flag=flag, sq=(sq, upd))
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0]) == 0          # zero unit: exactly zero
    assert torch.count_nonzero(out[1]) > 0
    assert int(flag.item()) == 0
    grad[SQ_BLOCK + 256 * 512 + 77] = float("inf")
    mom.zero_()
    ctx.momentum_update(grad, mom, upd, 0.95, True, sq_partials=sq)
    ctx.newton_schulz(mats, out, 0, ns_params(), nonfinite_flag=flag, sq=(sq, upd))
    torch.cuda.synchronize()
    assert int(flag.item()) == 1


def test_muon_step_norms_from_momentum(ctx):
    """A whole step with and without the partials: same momentum bits, weights
    within the rounding of the two norm sums."""
    w = synth.qwen3_4b_layer()
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    steps = []
    for use in (True, False):
        ms = MuonStep(shapes, DEV, lr=w.lr, beta=w.beta, nesterov=w.nesterov, compute=w.compute,
                      grad_dtype=w.grad_dtype, cap_bytes=w.cap_bytes, cap_kind=w.cap_kind,
                      ns_steps=w.ns_steps, norms_from_momentum=use)
        g = gen(w.seed)
        for i, W0 in enumerate(synth.draw_weights(w, g, DEV)):
            ms.view(ms.master, i).copy_(W0)
        synth.draw_grads(w, g, DEV, out=[ms.view(ms.grad, i) for i in range(len(w.mats))])
        init = ms.master.clone()
        ms.step()
        torch.cuda.synchronize()
        assert all(grp[3] == use for _, _, groups, _ in ms._work for grp in groups)
        steps.append((ms, ms.master - init))
    (a, da), (b, db) = steps
    assert torch.equal(a.momentum, b.momentum)
    d = oracle.rel_fro(da.cpu().numpy(), db.cpu().numpy())
    say(f"  step with / without partials: relative difference of the weight steps {d:.3e}")
    assert d <= 1e-3
