"""Units at the size limit of the MFMA path (needs a gfx950 GPU).

The MFMA product kernels address a unit through 32-bit buffer offsets, so a
bf16 unit must stay under 2 GiB; a unit of 2 GiB or more runs on the generic
kernels (64-bit offsets).  One 512 x n unit just under the limit and one at
it, each zero except a Gaussian 512-column block at either end: the
Newton-Schulz of [G1 | 0 | G2] is the Newton-Schulz of [G1 | G2] with the zero
columns kept (XX^T = G1 G1^T + G2 G2^T, and every product keeps a zero column
zero), so the two blocks are checked against the oracle on the 512 x 1024
matrix [G1 | G2], and the columns between them must come out exactly zero.
The second block sits in the unit's last bytes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_amd import Context, ns_params, ns_workspace_bytes
from newton_schulz_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16_TOL = 2e-2
ROWS = 512


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("cols,path", [((1 << 21) - 8, "MFMA, offsets just under 2 GiB"),
                                       (1 << 21, "generic, a 2 GiB unit")])
def test_unit_at_the_size_limit(cols, path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    unit_bytes = ROWS * cols * 2
    say(f"  {ROWS}x{cols} bf16 ({unit_bytes} bytes): {path}")
    g = torch.Generator(device=DEV).manual_seed(cols)
    x = torch.zeros((ROWS, cols), dtype=torch.bfloat16, device=DEV)
    x[:, :ROWS] = synth.normal((ROWS, ROWS), 1e-3, g, DEV, torch.bfloat16)
    x[:, cols - ROWS:] = synth.normal((ROWS, ROWS), 1e-3, g, DEV, torch.bfloat16)
    out = torch.empty_like(x)
    ctx = Context(DEV, ns_workspace_bytes(ROWS, cols, 1))
    try:
        ctx.newton_schulz([x], [out], params=ns_params(compute="bf16"))
        torch.cuda.synchronize()
    finally:
        ctx.close()
    assert out[:, ROWS:cols - ROWS].abs().max().item() == 0.0
    ends = torch.cat([x[:, :ROWS], x[:, cols - ROWS:]], dim=1).float().cpu().numpy()
    got = torch.cat([out[:, :ROWS], out[:, cols - ROWS:]], dim=1).float().cpu().numpy()
    ref = oracle.ns_ref(ends)
    err = oracle.rel_fro(got, ref)
    say(f"    relative error of the nonzero blocks {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= BF16_TOL
