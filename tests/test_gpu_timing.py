"""Per-kernel-class timing (muon_timing_enable / _select / _read) on a GPU.

With a class selection only the selected classes record events; the other
launches still run (same results) but add no event markers to the stream.
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
    c = Context(DEV, 1 << 30)
    c.timing_enable(True, 1024)
    yield c
    c.close()


def run(ctx, classes):
    g = torch.Generator(device=DEV).manual_seed(5)
    mats = [synth.normal((1024, 2560), 1e-3, g, DEV, torch.bfloat16) for _ in range(4)]
    out = [torch.empty_like(m) for m in mats]
    ctx.timing_select(classes)
    ctx.timing_reset()
    ctx.newton_schulz(mats, out, params=ns_params(compute="bf16"))
    torch.cuda.synchronize()
    return ctx.timing_read(), out


def test_only_selected_classes_are_timed(ctx):
    t, a = run(ctx, ["update"])
    say(f"  update only: {t}")
    assert t["update"][1] == 5 and t["update"][0] > 0
    for k in ("norm", "gram", "symsq", "momentum", "apply", "prod", "fused"):
        assert t[k] == (0.0, 0), k
    t, b = run(ctx, None)
    say(f"  every class: {t}")
    assert t["norm"][1] == 1 and t["gram"][1] == 5 and t["symsq"][1] == 5 and t["update"][1] == 5
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    t, _ = run(ctx, [])
    assert all(v == (0.0, 0) for v in t.values())
    ctx.timing_select(None)


def test_unknown_class_name_is_rejected(ctx):
    with pytest.raises(ValueError):
        ctx.timing_select(["nope"])
