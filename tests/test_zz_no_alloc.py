"""The allocation-free Newton-Schulz entry point (needs a gfx950 GPU).

muon_newton_schulz_batched_noalloc runs the kernels of
muon_newton_schulz_batched with a static device scratch instead of a
context's workspace; on the same inputs the two give the same bits.  Two
calls in a row, the second smaller, share the scratch: the second must not
see anything of the first.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_amd import Context, MuonError, newton_schulz_noalloc, ns_params, synth
from newton_schulz_amd._lib import MUON_NOALLOC_SCRATCH_BYTES

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Context(DEV, 1 << 30)
    yield c
    c.close()


def stack(count, rows, cols, seed, dtype=torch.bfloat16, std=1e-3):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return synth.normal((count, rows, cols), std, g, DEV, dtype)


# (rows, cols, count, head_rows, params): the second of each pair smaller
CALLS = [
    [(768, 2048, 6, 0, {}), (256, 512, 2, 0, {})],                        # 256-tiles, then 128-tiles
    [(128, 2560, 40, 0, {"fuse": "on"}), (128, 640, 3, 0, {"fuse": "on"})],  # fused small units
    [(1024, 512, 4, 0, {}), (384, 256, 2, 0, {})],                        # tall
    [(512, 1024, 3, 128, {}), (256, 640, 2, 128, {})],                    # per-head
    [(520, 1048, 2, 0, {"method": "gram"}), (264, 520, 2, 0, {"coeffs": "minimax"})],
    [(96, 160, 3, 0, {"compute": "f32"}), (40, 72, 2, 0, {"compute": "f32"})],
    [(8, 64, 5, 0, {}), (24, 40, 2, 4, {})],                              # units under 16: fp32 iteration
]


@pytest.mark.parametrize("calls", CALLS, ids=lambda c: f"{c[0][0]}x{c[0][1]}")
def test_two_calls_match_context_entry_point(ctx, calls):
    for k, (rows, cols, count, h, kw) in enumerate(calls):
        dt = torch.float32 if kw.get("compute") == "f32" else torch.bfloat16
        x = stack(count, rows, cols, seed=rows + cols + k, dtype=dt, std=1.0 if dt == torch.float32 else 1e-3)
        p = ns_params(**kw)
        want = torch.empty_like(x)
        ctx.newton_schulz(list(x.unbind(0)), list(want.unbind(0)), h, p)
        got = torch.full_like(x, float("nan"))
        newton_schulz_noalloc(list(x.unbind(0)), list(got.unbind(0)), h, p)
        torch.cuda.synchronize()
        say(f"  call {k}: {count} x {rows}x{cols} h={h} {kw}")
        assert torch.equal(got, want)
        # and within the oracle's bar (first matrix)
        ref = oracle.ns_ref_heads(x[0].float().cpu().numpy().astype(np.float64), h,
                                  **({"coeffs": oracle.minimax_schedule(5)[0]} if kw.get("coeffs") else {}))
        err = oracle.rel_fro(got[0].float().cpu().numpy(), ref)
        assert err <= (1e-4 if dt == torch.float32 else 2e-2), err


def test_in_place(ctx):
    x = stack(3, 512, 1024, seed=7)
    want = torch.empty_like(x)
    ctx.newton_schulz(list(x.unbind(0)), list(want.unbind(0)))
    newton_schulz_noalloc(list(x.unbind(0)), None)
    torch.cuda.synchronize()
    assert torch.equal(x, want)


def test_rejections(ctx):
    # a call whose workspace exceeds the static scratch
    big = torch.empty((4, 2560, 9728), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(MuonError) as e:
        newton_schulz_noalloc(list(big.unbind(0)), None)
    assert e.value.status == 4 and "static scratch" in str(e.value)
    assert MUON_NOALLOC_SCRATCH_BYTES == 256 << 20
    # unevenly spaced inputs
    buf = torch.zeros(5 * 256 * 512, dtype=torch.bfloat16, device=DEV)
    mats = [buf[o * 256 * 512:(o + 1) * 256 * 512].view(256, 512) for o in (0, 1, 3)]
    with pytest.raises(MuonError) as e:
        newton_schulz_noalloc(mats, None)
    assert e.value.status == 1
    # outputs overlapping the inputs other than in place
    x = stack(3, 256, 512, seed=3)
    with pytest.raises(MuonError) as e:
        newton_schulz_noalloc([x[0], x[1]], [x[1], x[2]])
    assert e.value.status == 1
