"""Host logic of bench.py (no GPU): flop accounting, unit lists, the refusal
of more than one GPU.

The algorithmic count per m x n unit (m <= n) and iteration is
m(m+1)n (Gram, upper triangle) + m^2(m+1) (symmetric square) + 2m^2 n
(update); the dense-equivalent count is 2m^2 n + 2m^3 + 2m^2 n.  The totals
below are those closed forms summed by hand over each workload's shapes.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from newton_schulz_amd import synth  # noqa: E402


def per_unit(m, n, steps=5):
    return steps * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)


def dense_unit(m, n, steps=5):
    return steps * (2 * m * m * n + 2 * m ** 3 + 2 * m * m * n)


def totals(w):
    units = bench.unit_list(w)
    alg = sum(sum(bench.ns_flops(m, n, w.ns_steps)) for m, n in units)
    dense = sum(dense_unit(m, n, w.ns_steps) for m, n in units)
    return units, alg, dense


def test_one_layer_counts():
    units, alg, dense = totals(synth.qwen3_4b_layer())
    # q, o -> (2560, 4096) x2; k, v -> (1024, 2560) x2; gate, up, down -> (2560, 9728) x3
    assert sorted(units) == sorted([(2560, 4096)] * 2 + [(1024, 2560)] * 2 + [(2560, 9728)] * 3)
    want = 2 * per_unit(2560, 4096) + 2 * per_unit(1024, 2560) + 3 * per_unit(2560, 9728)
    assert alg == want
    assert round(alg / 1e12, 3) == 4.186 and round(dense / 1e12, 3) == 5.867


def test_full_model_counts():
    w = synth.qwen3_4b()
    units, alg, dense = totals(w)
    assert len(w.mats) == 252 and len(units) == 252
    assert sum(m.numel for m in w.mats) == 3633315840
    assert round(alg / 1e12, 2) == 150.68 and round(dense / 1e12, 1) == 211.2


def test_per_head_counts():
    w = synth.qwen3_4b_heads()
    units, alg, dense = totals(w)
    assert len(units) == 1728 and set(units) == {(128, 2560)}
    assert alg == 1728 * per_unit(128, 2560)
    assert round(alg / 1e12, 3) == 1.108 and round(dense / 1e12, 3) == 1.486


def test_expert_counts_skip_zero_experts():
    w = synth.qwen3_30b_experts(layers=48)
    units, alg, _ = totals(w)
    assert len(w.mats) == 48 * 128 * 3
    assert len(units) == len(w.mats) * 3 // 4        # 25% of experts carry zero gradients
    assert set(units) == {(768, 2048)}
    assert round(alg / 1e12, 1) == 281.9


def test_tiny_counts():
    units, alg, _ = totals(synth.tiny())
    assert sorted(units) == sorted([(64, 128), (128, 128), (64, 256), (96, 96)])
    assert alg == 86272000


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_4b_layer", "qwen3_4b_heads",
                                  "qwen3_30b_experts:2"])
def test_workload_names(name):
    assert bench.workload_by_name(name).mats


def read_golden(name):
    vals = {}
    for line in open(os.path.join(ROOT, "tests", "golden", name)):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_qwen3_4b_muon_parameters_match_the_pages():
    """The pages put Qwen3-4B's Muon momentum at 4 B per parameter, ~14.5 GB:
    the 36-layer shape inventory (q, k, v, o, gate, up, down) must give that."""
    g = read_golden("qwen3_4b_momentum_bytes.txt")
    params = sum(m.numel for m in synth.qwen3_4b().mats)
    assert round(params * g["bytes_per_param"] / 1e9, 1) == g["total_gb"]
    # a plausible slip in the inventory (another FFN width, a missing layer,
    # full-width k/v projections) lands elsewhere
    assert round((params - 3 * 2560 * (9728 - 9216) * 36) * 4 / 1e9, 1) != g["total_gb"]
    assert round(params * 35 / 36 * 4 / 1e9, 1) != g["total_gb"]
    assert round((params + 2 * 2560 * (2560 - 1024) * 36) * 4 / 1e9, 1) != g["total_gb"]


def test_fused_bytes_count_the_iterate_and_residual_passes():
    # quintic, 5 iterations: the input once for A_0, then 5 reads and 5
    # writes of the iterate, and the residual written by iterations 0..2
    # and read by iterations 1..3: 17 passes of 2 m n bytes
    assert bench.fused_bytes(128, 2560, 5, gram=False) == 17 * 2 * 128 * 2560
    # two iterations carry no residual: input + 2 reads + 2 writes
    assert bench.fused_bytes(128, 2560, 2, gram=False) == 5 * 2 * 128 * 2560
    assert bench.fused_bytes(128, 2560, 3, gram=False) == 9 * 2 * 128 * 2560
    # the Gram form reads the input twice and writes once
    assert bench.fused_bytes(96, 4096, 5, gram=True) == 3 * 2 * 96 * 4096


def test_expert_layers_that_fit():
    per = 128 * 3 * 768 * 2048 * 10
    gib = 1 << 30
    assert bench.expert_layers_that_fit(48 * per + 6 * gib) == 48
    assert bench.expert_layers_that_fit(10 ** 15) == 48
    assert bench.expert_layers_that_fit(45 * per + 6 * gib + per - 1) == 45
    assert bench.expert_layers_that_fit(0) == 1
    # each further lane of micro-buckets in flight reserves 2 GiB more
    assert bench.expert_layers_that_fit(48 * per + 6 * gib, lanes=2) == 47
    assert bench.expert_layers_that_fit(48 * per + 8 * gib, lanes=2) == 48


def test_traffic_record_guards():
    """A counter record is used only for the kernel code and the launches per
    step it was taken on."""
    csrc = os.path.join(bench.ROOT, "newton_schulz_amd", "csrc")
    src = [os.path.join(csrc, f) for f in ("ns_gemm_mfma.hip", "ns_mfma_common.h", "muon_device.h")]
    name = "update_kernel_traffic_qwen3_4b_36l"
    rec = json.load(open(os.path.join(bench.ROOT, "profiles", name + ".json")))
    n = rec["dispatches"]
    assert bench.traffic_record(name, n + 1, *src) is None
    assert bench.traffic_record(name, n / 2, *src) is None
    assert bench.traffic_record("no_such_record", n, *src) is None
    from newton_schulz_amd.prof import source_fingerprint
    if rec["source_code_sha256_16"] == source_fingerprint(*src):
        assert bench.traffic_record(name, n, *src) == round(rec["hbm_bytes_per_launch"])
    else:
        assert bench.traffic_record(name, n, *src) is None
