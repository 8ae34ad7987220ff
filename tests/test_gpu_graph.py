"""A whole step recorded into a HIP graph and replayed (needs a gfx950 GPU).

Two MuonStep instances start from the same state; one steps eagerly, the
other replays its recorded step.  Every replay is checked against the eager
step, bit for bit, with fresh gradients, unrelated eager work and
synchronisations between the replays (a recorded graph must not depend on
what ran before it).
"""
import sys

import pytest
import torch

from newton_schulz_amd import Context, MuonStep, ns_params
from newton_schulz_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# wide, tall, per-head (fused when a call has a unit per CU: not here), a
# unit under 16 rows (fp32 iteration), a shape off the MFMA path
SHAPES = [(256, 512, 0), (512, 256, 0), (512, 640, 128), (8, 64, 0), (130, 202, 0), (256, 512, 0)]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def make(inflight):
    return MuonStep(SHAPES, DEV, cap_bytes=1 << 20, inflight=inflight, keep_bf16_weights=True)


@pytest.mark.parametrize("inflight", [1, 2])
def test_replayed_step_matches_eager(inflight):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    a, b = make(inflight), make(inflight)
    assert len(a.plan.buckets) > 2
    g = torch.Generator(device=DEV).manual_seed(9)
    w0 = synth.normal((a.numel,), 2e-2, g, DEV, torch.float32)
    for s in (a, b):
        s.master.copy_(w0)
    b.capture()
    junk = torch.zeros(1 << 20, device=DEV)
    for t in range(3):
        gr = synth.normal((a.numel,), 1e-3, g, DEV, torch.bfloat16)
        a.grad.copy_(gr)
        b.grad.copy_(gr)
        a.step()
        junk.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        b.replay()
        torch.cuda.synchronize()
        for name in ("momentum", "master", "weight_bf16"):
            x, y = getattr(a, name), getattr(b, name)
            assert torch.equal(x, y), (t, name)
        say(f"  inflight={inflight} step {t}: replay bit-identical to the eager step")
    assert torch.all(junk == 3.0)
    for s in (a, b):
        for c in s.contexts:
            c.close()


def test_timing_skips_recorded_launches():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = make(1)
    c = s.contexts[0]
    c.timing_enable(True, 4096)
    c.timing_reset()
    s.capture()
    s.replay()
    torch.cuda.synchronize()
    t = c.timing_read()
    assert all(v == (0.0, 0) for v in t.values()), t
    s.step()
    torch.cuda.synchronize()
    assert c.timing_read()["update"][1] > 0
    c.close()


# the rejected call records nothing, so torch reports an empty graph
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_irregular_placement_cannot_be_recorded():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from newton_schulz_amd.api import MuonError
    ctx = Context(DEV, 64 << 20)
    g = torch.Generator(device=DEV).manual_seed(3)
    base = synth.normal((4, 128, 256), 1e-3, g, DEV, torch.bfloat16)
    mats = [base[0], base[3], base[1]]  # not evenly spaced: needs pointer tables
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with pytest.raises(MuonError):
        with torch.cuda.graph(graph, stream=side):
            ctx.newton_schulz(mats, None, params=ns_params(compute="bf16"), stream=side)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    ctx.close()
