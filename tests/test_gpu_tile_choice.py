"""Tile side of the product launches: 128 x 128 where few 256-tiles would
leave most CUs idle, 256 x 256 otherwise.  Each accumulator sums the same
products in the same order at either side, so a unit's result must not depend
on the tile side its call picked (needs a gfx950 GPU).

A call of one unit runs its products on 128-tiles (one 1024 x 2560 unit: 10
upper 256-tiles for 256 CUs); the same unit as the first of 72 runs on
256-tiles.  The first unit's bits must agree, for the quintic (the residual
plane and B's diagonal correction included), per-iteration coefficients and
the Gram form, wide and tall.
"""
import sys

import pytest
import torch

from newton_schulz_amd import Context, ns_params
from newton_schulz_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Context(DEV, 3 << 30)
    yield c
    c.close()


def first_unit_both_ways(ctx, shape, many, params, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    mats = [synth.normal(shape, 1e-3, g, DEV, torch.bfloat16) for _ in range(many)]
    alone = [torch.empty_like(mats[0])]
    ctx.newton_schulz(mats[:1], alone, params=params)
    batch = [torch.empty_like(m) for m in mats]
    ctx.newton_schulz(mats, batch, params=params)
    torch.cuda.synchronize()
    return alone[0], batch[0]


@pytest.mark.parametrize("shape,many", [((1024, 2560), 72), ((2560, 1024), 72), ((2560, 4096), 12)])
def test_quintic_same_bits_at_either_tile_side(ctx, shape, many):
    say(f"  quintic {shape}: one unit against the first of {many}")
    a, b = first_unit_both_ways(ctx, shape, many, ns_params(compute="bf16"), shape[0] + shape[1])
    assert torch.equal(a, b)
    assert a.abs().max().item() > 0


def test_per_iteration_coefficients_same_bits(ctx):
    say("  minimax 1024x2560: one unit against the first of 72")
    p = ns_params(compute="bf16", steps=4, coeffs="minimax")
    a, b = first_unit_both_ways(ctx, (1024, 2560), 72, p, 7)
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(1024, 2560), (2560, 1024)])
def test_gram_form_same_bits(ctx, shape):
    say(f"  gram form {shape}: one unit against the first of 72")
    a, b = first_unit_both_ways(ctx, shape, 72, ns_params(compute="bf16", method="gram"), 11)
    assert torch.equal(a, b)
