"""The host-offloaded step against the resident one (needs a gfx950 GPU).

The offload pipeline moves the momentum (and the gradient) across PCIe per
micro-bucket and runs the same kernels on the same buffer layout, so every
result must be bit-identical to the resident step: momentum, master weights,
their bf16 copy, and the orthogonalised update that is copied back to the
host.  The update is also checked against the apply's definition: the master
after the step is the oracle's apply of that update to the master before.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_amd import MuonStep, synth
from newton_schulz_amd.offload import MuonOffloadStep

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def workload():
    """One Qwen3-4B layer plus per-head q/k/v copies, cut into several
    micro-buckets by a small cap, so slots are reused within a step."""
    w = synth.qwen3_4b(layers=1, seed=11, cap_bytes=64 << 20)
    heads = synth.qwen3_4b_heads(layers=1)
    w.mats = w.mats + heads.mats
    return w


def resident_step(ms: MuonStep):
    """MuonStep.step, keeping every micro-bucket's update."""
    upd = torch.empty(ms.numel, dtype=ms.cdtype, device=DEV)
    for lo, hi, groups, want_sq in ms._work:
        wb = ms.weight_bf16[lo:hi] if ms.weight_bf16 is not None else None
        ms._run_bucket(ms.grad[lo:hi], ms.momentum[lo:hi], ms.update[:hi - lo], ms.sq, groups, want_sq,
                       ms.master[lo:hi], wb, None, None)
        upd[lo:hi].copy_(ms.update[:hi - lo])
    return upd


@pytest.mark.parametrize("inflight,pin,grads_on_host", [(2, True, True), (1, True, True),
                                                         (2, False, True), (2, True, False),
                                                         (3, True, True)])
def test_offload_bit_identical_to_resident(inflight, pin, grads_on_host):
    say(f"offload inflight={inflight} pin={pin} grads_on_host={grads_on_host}")
    w = workload()
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    kw = dict(lr=w.lr, beta=w.beta, nesterov=w.nesterov, compute=w.compute, grad_dtype=w.grad_dtype,
              cap_bytes=w.cap_bytes, cap_kind=w.cap_kind, keep_bf16_weights=True)
    res = MuonStep(shapes, DEV, **kw)
    off = MuonOffloadStep(shapes, DEV, inflight=inflight, pin=pin, grads_on_host=grads_on_host, **kw)
    assert len(off.plan.buckets) >= 4
    assert off.grad.is_cuda != grads_on_host and not off.momentum.is_cuda
    assert off.momentum.is_pinned() == pin
    g = synth.generator(w.seed, DEV)
    for i, W0 in enumerate(synth.draw_weights(w, g, DEV)):
        res.view(res.master, i).copy_(W0)
    off.master.copy_(res.master)
    # the momentum pre-fill and three steps, each with a fresh gradient
    for step in range(4):
        synth.draw_grads(w, g, DEV, out=[res.view(res.grad, i) for i in range(len(shapes))])
        off.grad.copy_(res.grad)
        W_before = off.master.cpu()
        if step == 0:
            res.momentum_only()
            off.momentum_only()
        else:
            u = resident_step(res)
            off.step()
        torch.cuda.synchronize()
        assert torch.equal(off.momentum, res.momentum.cpu()), step
        if step == 0:
            continue
        assert torch.equal(off.master, res.master), step
        assert torch.equal(off.weight_bf16, res.weight_bf16), step
        assert torch.equal(off.update_host.view(torch.int16), u.cpu().view(torch.int16)), step
        # the copied-back update is the one that was applied
        Wn = oracle.apply_ref(W_before.numpy(), off.update_host.float().numpy(), w.lr, 1.0, 0.0)
        Wn = Wn[0] if isinstance(Wn, tuple) else Wn
        assert np.array_equal(np.asarray(Wn, dtype=np.float32).view(np.uint32),
                              off.master.cpu().numpy().view(np.uint32)), step
        assert off.update_host.abs().amax() > 0


def test_offload_timing_and_device_bytes():
    w = workload()
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    off = MuonOffloadStep(shapes, DEV, inflight=2, timing=True, cap_bytes=w.cap_bytes)
    off.step()
    torch.cuda.synchronize()
    st = off.copy_stats()
    nb = len(off.plan.buckets)
    # copy-in per micro-bucket; momentum kernel + Newton-Schulz/apply; the
    # momentum and the update copied out separately
    assert st["h2d"]["ops"] == nb and st["compute"]["ops"] == st["d2h"]["ops"] == 2 * nb
    # gradient (bf16) + momentum in; momentum + update (bf16) out
    assert st["h2d"]["bytes"] == off.numel * 6 and st["d2h"]["bytes"] == off.numel * 6
    assert all(st[k]["ms"] > 0 for k in st)
    # the slots: two micro-buckets of gradient, momentum, update, partials
    mb = max(b.numel for b in off.plan.buckets)
    per = mb * (2 + 4 + 2) + 8 * -(-mb // 4096)
    assert off.device_bytes() == 2 * per + off.plan.max_workspace
    assert off.copy_stats()["h2d"]["ops"] == 0
