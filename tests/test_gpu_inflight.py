"""Micro-buckets in flight on the resident step (needs a gfx950 GPU).

With inflight = k the step runs micro-bucket i on lane i % k, each lane with
its own stream, update buffer and workspace.  Micro-buckets touch disjoint
state and every lane keeps its micro-buckets in order, so momentum, master
weights, their bf16 copy and the non-finite flag must be bit-identical to the
one-lane step for every k, step after step; and once the caller's stream has
been synchronised every lane's work must be complete.
"""
import sys

import pytest
import torch

from newton_schulz_amd import MuonStep, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def workload():
    """One Qwen3-4B layer plus per-head q/k/v copies, cut by a small cap into
    micro-buckets of several shapes (wide, tall, fused small units)."""
    w = synth.qwen3_4b(layers=1, seed=5, cap_bytes=64 << 20)
    w.mats = w.mats + synth.qwen3_4b_heads(layers=1).mats
    return w


@pytest.mark.parametrize("inflight", [2, 3, 7])
def test_inflight_bit_identical(inflight):
    w = workload()
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    kw = dict(lr=w.lr, beta=w.beta, nesterov=w.nesterov, compute=w.compute, grad_dtype=w.grad_dtype,
              cap_bytes=w.cap_bytes, cap_kind=w.cap_kind, keep_bf16_weights=True)
    one = MuonStep(shapes, DEV, **kw)
    many = MuonStep(shapes, DEV, inflight=inflight, **kw)
    say(f"inflight={inflight}: {len(one.plan.buckets)} micro-buckets")
    # several micro-buckets per lane, or (7) more lanes than micro-buckets
    assert len(one.plan.buckets) >= 6
    assert len(many.contexts) == inflight
    g = synth.generator(w.seed, DEV)
    for i, W0 in enumerate(synth.draw_weights(w, g, DEV)):
        one.view(one.master, i).copy_(W0)
    many.master.copy_(one.master)
    f1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    f2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    for step in range(3):
        synth.draw_grads(w, g, DEV, out=[one.view(one.grad, i) for i in range(len(shapes))])
        many.grad.copy_(one.grad)
        if step == 0:
            one.momentum_only()
            many.momentum_only()
        else:
            # on a side stream of the caller's: the lanes must follow it
            s = torch.cuda.Stream(DEV)
            s.wait_stream(torch.cuda.current_stream(DEV))
            one.step(nonfinite_flag=f1)
            many.step(stream=s, nonfinite_flag=f2)
            s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(many.momentum, one.momentum), step
        assert torch.equal(many.master, one.master), step
        assert torch.equal(many.weight_bf16, one.weight_bf16), step
        assert torch.equal(f1, f2) and int(f1.item()) == 0, step


def test_inflight_sync_on_callers_stream():
    """After step() on the caller's stream and a synchronisation of that
    stream alone, the last micro-bucket (on the last lane) has been applied."""
    w = workload()
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    ms = MuonStep(shapes, DEV, inflight=2, cap_bytes=w.cap_bytes, lr=0.5)
    ms.grad.normal_()
    ms.momentum_only()
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        before = ms.master.clone()
        ms.step(stream=s)
        s.synchronize()
        lo, hi = ms._work[-1][0], ms._work[-1][1]
        assert not torch.equal(ms.master[lo:hi], before[lo:hi])
