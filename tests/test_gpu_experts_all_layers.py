"""Qwen3-30B-A3B experts at the stated scale (needs a gfx950 GPU).

One Muon step over all 48 layers of experts (18432 matrices, 25% of the
experts without gradient), or as many layers as the device's free memory
holds, with the workload's 1 GiB workspace cap: the first and the last matrix
of every eighth micro-bucket and seeded picks against the oracle (momentum
bit-exact, Newton-Schulz + apply within the bf16 bar per matrix), and every
expert without gradient untouched -- its momentum still zero and its
weights' bit patterns summing to what they summed to before the step.
"""
import gc
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_amd import MuonStep, synth

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_TOL = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def bits_sums(ms, idx):
    """Per matrix, the sum of its fp32 bit patterns (int64, on the device): a
    change of any bit changes it."""
    return torch.stack([ms.view(ms.master, i).view(torch.int32).sum(dtype=torch.int64) for i in idx])


def test_experts_all_layers_one_step():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.empty_cache()
    free = torch.cuda.mem_get_info(DEV)[0]
    L = bench.expert_layers_that_fit(free)
    say(f"experts: {L} of 48 layers fit in {free / 1e9:.1f} GB")
    assert L >= 2
    w = synth.qwen3_30b_experts(layers=L)
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    ms = MuonStep(shapes, DEV, lr=w.lr, beta=w.beta, nesterov=w.nesterov, compute=w.compute,
                  grad_dtype=w.grad_dtype, cap_bytes=w.cap_bytes, cap_kind=w.cap_kind,
                  ns_steps=w.ns_steps)
    assert all(b.workspace_bytes <= w.cap_bytes for b in ms.plan.buckets)
    g = synth.generator(w.seed, DEV)
    for i, W0 in enumerate(synth.iter_weights(w, g, DEV)):
        ms.view(ms.master, i).copy_(W0)
    synth.draw_grads(w, g, DEV, out=[ms.view(ms.grad, i) for i in range(len(w.mats))])
    n = len(w.mats)
    zero = [i for i in range(n) if w.mats[i].zero_grad]
    assert len(zero) == L * 32 * 3
    picks = set()
    for b in ms.plan.buckets[::8]:
        picks |= {b.indices[0], b.indices[-1]}
    rng = np.random.default_rng(7)
    picks |= set(rng.integers(0, n, 8).tolist()) | set(zero[:2])
    picks = sorted(picks)
    G = {i: host(ms.view(ms.grad, i)) for i in picks}
    M0 = {i: host(ms.view(ms.momentum, i)) for i in picks}
    W0 = {i: host(ms.view(ms.master, i)).astype(np.float64) for i in picks}
    zsum = bits_sums(ms, zero)
    ms.step()
    torch.cuda.synchronize()
    say(f"  {len(ms.plan.buckets)} micro-buckets; checking {len(picks)} matrices against the oracle")
    for i in picks:
        m_ref, u_ref = oracle.momentum_ref(G[i], M0[i], w.beta, w.nesterov)
        assert np.array_equal(host(ms.view(ms.momentum, i)).view(np.uint32), m_ref.view(np.uint32)), i
        dW = host(ms.view(ms.master, i)).astype(np.float64) - W0[i]
        if w.mats[i].zero_grad:
            assert not np.any(dW), i
            continue
        O = oracle.ns_ref(oracle.bf16_round(u_ref))
        err = oracle.rel_fro(dW, -np.float32(w.lr) * O)
        assert err <= BF16_TOL, (i, err)
    nz = torch.stack([torch.count_nonzero(ms.view(ms.momentum, i)) for i in zero])
    assert int(nz.sum().item()) == 0
    assert torch.equal(bits_sums(ms, zero), zsum)
    say(f"  {len(zero)} experts without gradient untouched")
    # hand the ~290 GB back before the next test allocates
    for c in ms.contexts:
        c.close()
    del ms
    gc.collect()
    torch.cuda.empty_cache()
