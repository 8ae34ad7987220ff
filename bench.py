#!/usr/bin/env python3
"""Benchmark: one full Muon optimizer step on Qwen3-4B-shaped matrices.

A step = momentum (+ Nesterov) -> batched Newton-Schulz (5 quintic
iterations, bf16 MFMA) -> apply (fp32 master + bf16 copy) over all 252 Muon
matrices of a 36-layer Qwen3-4B (3.63B parameters), in 512 MiB micro-buckets.
Inputs are synthetic and already resident in HBM (bf16 gradients ~ N(0, 1e-3),
fp32 momentum pre-filled by two momentum steps, fp32 masters ~ N(0, 0.02)).

Prints ONE JSON line.  `value` is Newton-Schulz algorithmic TFLOP per step
divided by the whole step's wall time; ms_per_step is the full step.  Per-
kernel durations come from HIP events the library records on the launch
stream around every kernel during the timed steps.  --ns-method gram runs
the Gram form instead; `value` then still counts the quintic's flops
(quintic-equivalent throughput) and the breakdown the executed ones.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Newton–Schulz TFLOP/s (% bf16 MFMA peak); full Muon step ms, Qwen3-4B shapes"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def ns_flops(m: int, n: int, steps: int = 5):
    """Algorithmic flops of one unit (m <= n): symmetric Gram m(m+1)n, symmetric
    square m^2(m+1), update 2 m^2 n, per iteration."""
    gram = m * (m + 1) * n
    symsq = m * m * (m + 1)
    upd = 2 * m * m * n
    return steps * gram, steps * symsq, steps * upd


def ns_flops_gram(m: int, n: int, steps: int = 5):
    """Algorithmic flops of one unit in the Gram form: A_0 = X X^T (symmetric,
    m(m+1)n), steps symmetric squares P_k, 3 (steps - 1) symmetric m x m
    products (Q_{k+1} = P_k Q_k, P_k A_k, (P_k A_k) P_k), one final 2 m^2 n."""
    if steps == 0:
        return 0, 0, 0, 0
    sq = m * m * (m + 1)
    return m * (m + 1) * n, steps * sq, 3 * (steps - 1) * sq, 2 * m * m * n


def uses_gram_form(m: int, n: int, compute: str) -> bool:
    """bf16 runs the Gram form on units with 2 m <= n (the library's rule)."""
    return compute == "f32" or 2 * m <= n


def workload_by_name(name):
    from newton_schulz_amd import synth
    if name == "qwen3_4b":
        return synth.qwen3_4b()
    if name == "tiny":
        return synth.tiny()
    if name == "qwen3_4b_layer":
        return synth.qwen3_4b_layer()
    if name == "qwen3_4b_heads":
        return synth.qwen3_4b_heads()
    if name.startswith("qwen3_30b_experts"):
        layers = int(name.split(":")[1]) if ":" in name else 4
        return synth.qwen3_30b_experts(layers=layers)
    raise SystemExit(f"unknown workload {name}")


def unit_list(w, wide_flag: bool = False):
    """(m, n) of every Newton-Schulz unit with a nonzero gradient (with
    wide_flag: (m, n, rows <= cols))."""
    units = []
    for m in w.mats:
        if m.zero_grad:
            continue
        ur = m.head_rows or m.rows
        for _ in range(m.rows // ur):
            u = (min(ur, m.cols), max(ur, m.cols))
            units.append(u + (ur <= m.cols,) if wide_flag else u)
    return units


def fused_bytes(m: int, n: int, steps: int, gram: bool) -> int:
    """HBM bytes the whole-iteration kernel must move for one m x n unit: the
    quintic reads the input once for A_0, then per iteration reads the iterate
    and writes the next, and the bf16 iterate's rounding residual is written
    by iterations 0 .. steps-3 and read by iterations 1 .. steps-2; the Gram
    form reads the input twice and writes the result once."""
    if gram:
        return 3 * 2 * m * n
    return 2 * m * n * (1 + 2 * steps + 2 * max(0, steps - 2))


def traffic_record(name: str, launches_per_step: float, *kernel_src: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary profiles/<name>.json, or None when missing, taken on
    different kernel code (the kernel file and its local headers), or taken
    when a step cut the work into a different number of launches (the record
    covers one step: its dispatch count is the launches of that step)."""
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    from newton_schulz_amd.prof import source_fingerprint
    rec = json.load(open(path))
    if rec.get("source_code_sha256_16") != source_fingerprint(*kernel_src):
        return None
    if rec.get("dispatches") != round(launches_per_step):
        return None
    return round(rec.get("hbm_bytes_per_launch"))


def cpu_baseline(seconds_budget: float = 20.0, ns_steps: int = 5, minimax: bool = False):
    """The oracle (numpy fp64 Newton-Schulz, binary32 momentum/apply) on one
    Qwen3-4B layer, timed on this host's cores, with the same iteration count
    and coefficients as the timed GPU run."""
    import numpy as np
    import oracle
    from newton_schulz_amd import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    # BLAS threads: the CPUs this process may run on, capped at 16 (the share
    # of one GPU's host); the host's own count is reported beside it
    cores = min(len(os.sched_getaffinity(0)), 16)
    ctxm = threadpool_limits(limits=cores, user_api="blas") if threadpool_limits else None
    w = synth.qwen3_4b_layer()
    rng = np.random.default_rng(0)
    mats = [(m.rows, m.cols) for m in w.mats]
    ns_kw = {"steps": ns_steps}
    if minimax:
        ns_kw["coeffs"] = oracle.minimax_schedule(ns_steps)[0]
    t_ns = t_el = 0.0
    flops = 0
    done = 0
    try:
        for (r, c) in mats:
            g = oracle.bf16_round((rng.standard_normal((r, c)) * 1e-3).astype(np.float32))
            M = np.zeros((r, c), np.float32)
            W = (rng.standard_normal((r, c)) * 0.02).astype(np.float32)
            t0 = time.perf_counter()
            M, U = oracle.momentum_ref(g, M, 0.95, True)
            t1 = time.perf_counter()
            O = oracle.ns_ref(oracle.bf16_round(U), **ns_kw)
            t2 = time.perf_counter()
            oracle.apply_ref(W, oracle.bf16_round(O.astype(np.float32)), 0.02, bf16_copy=True)
            t3 = time.perf_counter()
            t_el += (t1 - t0) + (t3 - t2)
            t_ns += t2 - t1
            flops += sum(ns_flops(min(r, c), max(r, c), ns_steps))
            done += 1
            if t_ns + t_el > seconds_budget:
                break
        blas = None
        if threadpool_limits:
            info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
            blas = info[0].get("internal_api") if info else None
            cores_used = info[0].get("num_threads", cores) if info else cores
        else:
            cores_used = cores
    finally:
        if ctxm is not None:
            ctxm.__exit__(None, None, None)
    tot = t_ns + t_el
    return {
        "value": round(flops / tot / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores_used),
        "kind": "oracle",
        "sample": f"{done} of the 7 matrices of one Qwen3-4B layer (q, k, v, o, gate, up, down): "
                  f"momentum + fp64 Newton-Schulz + apply; {tot:.1f} s on the host "
                  f"(NS {t_ns:.1f} s); BLAS {blas}",
        "blas_thread_cap": cores,
        **host_cores(),
    }


EXPERT_LAYER_ELEMS = 128 * 3 * 768 * 2048   # one Qwen3-30B-A3B layer's expert matrices
EXPERT_STATE_BYTES = 2 + 4 + 4              # bf16 gradient, fp32 momentum, fp32 master
GIB = 1 << 30


def expert_layers_that_fit(free_bytes: int, layers: int = 48, lanes: int = 1) -> int:
    """Largest layer count (<= layers) whose expert state fits in free device
    memory with 4 GiB to spare beyond the step's own buffers (per lane of
    micro-buckets in flight: an update buffer and a workspace, each bounded by
    the 1 GiB cap)."""
    per = EXPERT_LAYER_ELEMS * EXPERT_STATE_BYTES
    return max(1, min(layers, (free_bytes - 4 * GIB - 2 * GIB * lanes) // per))


def step_times(run, steps: int):
    """Run `steps` steps between HIP events on the current stream: mean, median
    and min ms per step, the host wall time and every step's ms."""
    import statistics
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, statistics.median(per), min(per), wall, per


def host_cores():
    return {"host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def link_probe(dev, nbytes: int = GIB, reps: int = 3):
    """Host<->device copy rates of `nbytes`: pinned and pageable, each
    direction alone, and pinned both directions at once on two streams."""
    import torch
    d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    d2 = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = {}
    for pin in (True, False):
        h = torch.ones(nbytes, dtype=torch.uint8, pin_memory=pin)
        h2 = torch.empty(nbytes, dtype=torch.uint8, pin_memory=pin)
        for name, fn in (("h2d", lambda: d.copy_(h, non_blocking=pin)),
                         ("d2h", lambda: h2.copy_(d, non_blocking=pin))):
            best = None
            for _ in range(reps):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
                best = dt if best is None else min(best, dt)
            out[f"{name}_{'pinned' if pin else 'pageable'}_GBps"] = round(nbytes / best / 1e9, 2)
        if pin:
            s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
            best = None
            for _ in range(reps):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                with torch.cuda.stream(s1):
                    d2.copy_(h, non_blocking=True)
                with torch.cuda.stream(s2):
                    h2.copy_(d, non_blocking=True)
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
                best = dt if best is None else min(best, dt)
            out["duplex_pinned_GBps_each_way"] = round(nbytes / best / 1e9, 2)
        del h, h2
    out["bytes"] = nbytes
    return out


def run_library_gemm(args, w, dev):
    """The vendor library's batched GEMM (torch.bmm -> hipBLASLt) on the
    products of one Newton-Schulz iteration, per canonical unit shape, with
    the batch of the workload's largest micro-bucket of that shape: the update
    B'X (m x m times m x n) and the Gram X X^T (dense: the library computes
    both triangles).  Random bf16 operands (the MFMA rate depends on the
    data); transposed operands are made contiguous first."""
    import torch
    from newton_schulz_amd.api import Plan
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    plan = Plan(shapes, w.cap_bytes, w.cap_kind, w.compute)
    batch = {}
    for b in plan.buckets:
        batch[(b.m, b.n)] = max(batch.get((b.m, b.n), 0), b.units)
    dt = torch.bfloat16 if w.compute == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(0)
    rows = []
    for (m, n), U in batch.items():
        X = torch.randn((U, m, n), generator=g, device=dev).to(dt)
        B = torch.randn((U, m, m), generator=g, device=dev).to(dt)
        Xt = X.transpose(1, 2).contiguous()
        res = {"m": m, "n": n, "batch": U}
        for name, fn, flops in (("update", lambda: torch.bmm(B, X), 2 * m * m * n * U),
                                ("gram", lambda: torch.bmm(X, Xt), 2 * m * m * n * U)):
            for _ in range(3):
                fn()
            mean, med, mn, _, _ = step_times(fn, max(args.steps, 5))
            res[name] = {"ms_median": round(med, 4), "tflops_median": round(flops / (med * 1e-3) / 1e12, 1),
                         "tflops_best": round(flops / (mn * 1e-3) / 1e12, 1)}
        rows.append(res)
        del X, B, Xt
    print(json.dumps({"library_gemm": "torch.bmm (hipBLASLt), dense flops 2 m^2 n per product",
                      "dtype": w.compute, "workload": w.name, "shapes": rows,
                      "torch": torch.__version__}), flush=True)


def run_offload(args, w, dev):
    """The Muon step with momentum and gradient in host memory (pinned unless
    --pageable), `--inflight` micro-buckets on the device at a time."""
    import torch
    from newton_schulz_amd import synth
    from newton_schulz_amd.offload import MuonOffloadStep
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    t0 = time.perf_counter()
    off = MuonOffloadStep(shapes, dev, inflight=args.inflight, pin=not args.pageable,
                          lr=w.lr, beta=w.beta, nesterov=w.nesterov, compute=w.compute,
                          grad_dtype=w.grad_dtype, cap_bytes=w.cap_bytes, cap_kind=w.cap_kind,
                          ns_steps=w.ns_steps, keep_bf16_weights=True)
    t_alloc = time.perf_counter() - t0
    g = torch.Generator(device=dev).manual_seed(w.seed)
    for i, W0 in enumerate(synth.iter_weights(w, g, dev)):
        off.view(off.master, i).copy_(W0)
    grads = [off.view(off.grad, i) for i in range(len(w.mats))]
    for _ in range(w.warmup_momentum_steps):
        synth.draw_grads(w, g, dev, out=grads)
        off.momentum_only()
    synth.draw_grads(w, g, dev, out=grads)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        off.step()
    mean, med, mn, wall, per = step_times(off.step, args.steps)
    # one more step with events around every copy and compute stage
    off.timing = True
    off.step()
    torch.cuda.synchronize()
    st = off.copy_stats()
    off.timing = False
    numel = off.numel

    def rate(k):
        return round(st[k]["bytes"] / (st[k]["ms"] * 1e-3) / 1e9, 2) if st[k]["ms"] > 0 else None

    probe = link_probe(dev)
    units = unit_list(w)
    f_ns = sum(sum(ns_flops(m, n, w.ns_steps)) for (m, n) in units)
    out = {
        "metric": "Muon step with momentum and gradient in host memory, ms per step (Qwen3-4B shapes)",
        "value": round(mean, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean, 3),
        "ms_per_step_median": round(med, 3),
        "ms_per_step_min": round(mn, 3),
        "ms_steps": [round(t, 2) for t in per],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1e-3) bf16 gradients, fp32 state; no checkpoint)",
        "config": {"workload": w.name + "_offload", "matrices": len(w.mats), "muon_params": numel,
                   "inflight_micro_buckets": args.inflight, "host_memory": "pageable" if args.pageable else "pinned",
                   "grads_on_host": True, "update_to_host": True,
                   "micro_bucket_cap_bytes": w.cap_bytes, "micro_buckets": len(off.plan.buckets),
                   "parallelism": "single GPU"},
        "ns_tflops_pcie_inclusive": round(f_ns / (mean * 1e-3) / 1e12, 2),
        "copies_per_step": {
            "h2d_bytes": st["h2d"]["bytes"], "d2h_bytes": st["d2h"]["bytes"],
            "h2d_ms": round(st["h2d"]["ms"], 2), "d2h_ms": round(st["d2h"]["ms"], 2),
            "compute_ms": round(st["compute"]["ms"], 2),
            "h2d_GBps": rate("h2d"), "d2h_GBps": rate("d2h"),
            "pages_pinned_GBps": {"h2d": 43, "d2h": 57, "pageable": 10}},
        "link_probe": probe,
        "device_bytes_beyond_master": off.device_bytes(),
        "ns_workspace_bytes": off.plan.max_workspace,
        "host_alloc_s": round(t_alloc, 2),
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_4b",
                    help="qwen3_4b, qwen3_4b_layer, qwen3_4b_heads, qwen3_30b_experts:L "
                         "(L layers, or 'fit': the most of 48 that fit in device memory)")
    ap.add_argument("--ns-method", default="quintic", choices=["quintic", "gram"],
                    help="Newton-Schulz evaluation; value stays the quintic's flops / step time")
    ap.add_argument("--ns-coeffs", default="fixed", choices=["fixed", "minimax"],
                    help="fixed quintic (a, b, c), or the per-iteration minimax schedule")
    ap.add_argument("--ns-steps", type=int, default=0,
                    help="Newton-Schulz iterations (default: the workload's)")
    ap.add_argument("--ns-fuse", default="auto", choices=["auto", "off", "on"],
                    help="whole-iteration fusion of small units (muon_fuse_t)")
    ap.add_argument("--norms", default="momentum", choices=["momentum", "pass"],
                    help="Frobenius norms from the momentum pass's partials, or a separate read")
    ap.add_argument("--compute", default=None, choices=["bf16", "f32"],
                    help="override the workload's Newton-Schulz compute mode (f32: verification mode)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="instead of the step: the vendor library's batched GEMM (torch.bmm) on the "
                         "Newton-Schulz products of the workload's micro-buckets, as a yardstick")
    ap.add_argument("--offload", action="store_true",
                    help="momentum and gradient in host memory, copied per micro-bucket")
    ap.add_argument("--inflight", type=int, default=None,
                    help="micro-buckets in flight: lanes of the resident step (default 1), "
                         "device slots with --offload (default 2)")
    ap.add_argument("--pageable", action="store_true", help="--offload: pageable host memory")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-timing", action="store_true", help="skip per-kernel event timing")
    ap.add_argument("--graph", action="store_true",
                    help="record the step into a HIP graph once and time its replays (no per-kernel timing)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from newton_schulz_amd import MuonStep, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        # also a same-box reference for the streaming kernels: the median
        # rate of the plain device copy (read + write bytes per second)
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        times = []
        for i in range(3 + 10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.copy_(src)
            b.record()
            b.synchronize()
            if i >= 3:
                times.append(a.elapsed_time(b))
        times.sort()
        med = times[len(times) // 2]
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy, "copy_ms_median": round(med, 4),
                          "copy_gbs_read_plus_write": round(2 * args.calibrate_copy / (med * 1e-3) / 1e9, 1)}),
              flush=True)
        return
    if args.inflight is None:
        args.inflight = 2 if args.offload else 1
    if args.inflight < 1:
        print("--inflight must be >= 1", file=sys.stderr)
        sys.exit(2)
    if args.graph and (args.offload or args.library_gemm):
        print("--graph records the resident step only", file=sys.stderr)
        sys.exit(2)
    layers_note = None
    if args.workload in ("qwen3_30b_experts:fit", "qwen3_30b_experts:48"):
        free = torch.cuda.mem_get_info(dev)[0]
        L = expert_layers_that_fit(free, lanes=1 if args.offload else args.inflight)
        layers_note = {"layers_run": L, "layers_model": 48, "free_device_bytes": free,
                       "state_bytes_per_layer": EXPERT_LAYER_ELEMS * EXPERT_STATE_BYTES}
        args.workload = f"qwen3_30b_experts:{L}"
    w = workload_by_name(args.workload)
    if args.ns_steps:
        w = dataclasses.replace(w, ns_steps=args.ns_steps)
    if args.compute:
        w = dataclasses.replace(w, compute=args.compute)
    if args.library_gemm:
        run_library_gemm(args, w, dev)
        return
    if args.offload:
        run_offload(args, w, dev)
        return
    shapes = [(m.rows, m.cols, m.head_rows) for m in w.mats]
    keep_bf16 = not args.workload.startswith("qwen3_30b_experts")
    ms = MuonStep(shapes, dev, lr=w.lr, beta=w.beta, nesterov=w.nesterov, compute=w.compute,
                  grad_dtype=w.grad_dtype, cap_bytes=w.cap_bytes, cap_kind=w.cap_kind,
                  ns_steps=w.ns_steps, keep_bf16_weights=keep_bf16, ns_method=args.ns_method,
                  ns_coeffs=None if args.ns_coeffs == "fixed" else args.ns_coeffs,
                  norms_from_momentum=args.norms == "momentum", ns_fuse=args.ns_fuse,
                  inflight=args.inflight)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    for i, W0 in enumerate(synth.iter_weights(w, g, dev)):
        ms.view(ms.master, i).copy_(W0)
    grads = [ms.view(ms.grad, i) for i in range(len(w.mats))]
    for _ in range(w.warmup_momentum_steps):
        synth.draw_grads(w, g, dev, out=grads)
        ms.momentum_only()
    synth.draw_grads(w, g, dev, out=grads)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        ms.step()
    torch.cuda.synchronize()
    run = ms.step
    if args.graph:
        # the whole step as one recorded graph; replays record no per-kernel
        # events, so this line carries no breakdown or roofline
        ms.capture()
        ms.replay()
        torch.cuda.synchronize()
        run = ms.replay

    timing = not args.no_timing and not args.graph
    ns_classes = ("gram", "symsq", "prod", "update", "fused")
    breakdown_steps = min(args.steps, 5)
    if timing:
        # one event pair per launch: size the pool from one step's launches
        # (launches beyond the pool would go untimed); one pool per lane
        def timing_read():
            tot = {}
            for c in ms.contexts:
                for k, (t, n) in c.timing_read().items():
                    t0, n0 = tot.get(k, (0.0, 0))
                    tot[k] = (t0 + t, n0 + n)
            return tot
        for c in ms.contexts:
            c.timing_enable(True, capacity=1 << 14)
            c.timing_select(None)
            c.timing_reset()
        ms.step()
        pre = timing_read()
        per = sum(v[1] for v in pre.values())
        # the dominant Newton-Schulz kernel class by time in that step: the
        # timed steps record events around its launches only, so the other
        # launches' event markers stay out of the timed region
        dom = max(ns_classes, key=lambda k: pre[k][0])
        for c in ms.contexts:
            c.timing_enable(True, capacity=int(per * max(args.steps, breakdown_steps)) + 64)
            c.timing_select([dom])
            c.timing_reset()
    ms_per_step, ms_median, ms_min, wall, per = step_times(run, args.steps)
    kd = timing_read() if timing else {}
    if timing:
        # the per-class breakdown: a few steps after the timed region with
        # every launch between events
        for c in ms.contexts:
            c.timing_select(None)
            c.timing_reset()
        for _ in range(breakdown_steps):
            ms.step()
        torch.cuda.synchronize()
        kt = timing_read()
    else:
        kt = {}

    units = unit_list(w)
    fl = [ns_flops(m, n, w.ns_steps) for (m, n) in units]
    f_gram = sum(f[0] for f in fl)
    f_symsq = sum(f[1] for f in fl)
    f_upd = sum(f[2] for f in fl)
    f_ns = f_gram + f_symsq + f_upd
    dense = sum(w.ns_steps * (2 * m * m * n + 2 * m ** 3 + 2 * m * m * n) for (m, n) in units)
    # `value` counts the quintic iteration's algorithmic flops in both modes
    # (for the Gram form: quintic-equivalent throughput); the per-class rates
    # use the flops each class actually executed
    value = f_ns / (ms_per_step * 1e-3) / 1e12
    ex = {"gram": 0, "symsq": 0, "prod": 0, "update": 0, "fused": 0}
    fused_hbm = 0
    # units the library ran as fused launches (wide bf16 units with 16 <= m <=
    # 128: in these workloads every such call fuses, by its unit count or its
    # width)
    fused_ran = timing and kt["fused"][1] > 0
    for (m, n, wide) in unit_list(w, wide_flag=True):
        if args.ns_method == "gram" and uses_gram_form(m, n, w.compute):
            fg, fs, fp, fu = ns_flops_gram(m, n, w.ns_steps)
        else:
            (fg, fs, fu), fp = ns_flops(m, n, w.ns_steps), 0
        if fused_ran and w.compute == "bf16" and wide and 16 <= m <= 128:
            ex["fused"] += fg + fs + fp + fu
            fused_hbm += fused_bytes(m, n, w.ns_steps, args.ns_method == "gram")
            continue
        ex["gram"] += fg
        ex["symsq"] += fs
        ex["prod"] += fp
        ex["update"] += fu
    numel = sum(m.numel for m in w.mats)
    gdt_b = 2 if w.grad_dtype == torch.bfloat16 else 4
    cdt_b = 2 if w.compute == "bf16" else 4
    mom_bytes = numel * (gdt_b + 4 + 4 + cdt_b)
    app_bytes = numel * (4 + 4 + cdt_b + (2 if keep_bf16 else 0))

    breakdown = {}
    roofline = None
    if timing:
        per_step = {k: (v[0] / breakdown_steps, v[1] / breakdown_steps) for k, v in kt.items()}
        for k, (t, n) in per_step.items():
            breakdown[k] = {"ms_per_step": round(t, 4), "launches_per_step": n}
        def tf(f, k):
            t = per_step[k][0]
            return round(f / (t * 1e-3) / 1e12, 2) if t > 0 else None
        for k in ("gram", "symsq", "prod", "update", "fused"):
            if per_step[k][1] > 0:
                breakdown[k]["tflops"] = tf(ex[k], k)
        for k in ("gram", "symsq", "prod", "update", "fused"):
            if per_step[k][1] == 0:
                del breakdown[k]
        ns_ms = sum(per_step[k][0] for k in ("norm", "gram", "symsq", "prod", "update", "fused"))
        breakdown["newton_schulz"] = {"ms_per_step": round(ns_ms, 4),
                                      "tflops": round(sum(ex.values()) / (ns_ms * 1e-3) / 1e12, 2) if ns_ms else None}
        for k, b in (("momentum", mom_bytes), ("apply", app_bytes)):
            t = per_step[k][0]
            breakdown[k]["gbs"] = round(b / (t * 1e-3) / 1e9, 1) if t > 0 else None
            breakdown[k]["frac_hbm"] = round(b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if t > 0 else None
        # the roofline: the dominant class's launches inside the timed region.
        # The HBM counter records were taken on the default iteration (5 fixed
        # quintic steps, norms from the momentum pass, automatic fusion) and
        # apply to it only
        default_ns = (args.ns_method == "quintic" and args.ns_coeffs == "fixed" and w.ns_steps == 5
                      and args.norms == "momentum" and args.ns_fuse == "auto" and w.compute == "bf16")
        t_dom, n_dom = kd[dom][0] / args.steps, kd[dom][1] / args.steps
        csrc = os.path.join(ROOT, "newton_schulz_amd", "csrc")
        if dom == "fused" and t_dom > 0:
            achieved = fused_hbm / (t_dom * 1e-3) / 1e9
            if per_step["fused"][0] > 0:
                breakdown["fused"]["gbs"] = round(fused_hbm / (per_step["fused"][0] * 1e-3) / 1e9, 1)
            mfma_tf = ex["fused"] / (t_dom * 1e-3) / 1e12
            traffic = None if not default_ns else traffic_record(f"ns_small_kernel_traffic_{w.name}", n_dom,
                                     os.path.join(csrc, "ns_small.hip"), os.path.join(csrc, "ns_mfma_common.h"),
                                     os.path.join(csrc, "muon_device.h"))
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                        "kernel": "ns_small_kernel (every iteration of units with m <= 128 in one launch)",
                        "avg_launch_ms": round(t_dom / n_dom, 4),
                        "bytes_per_launch_avg": int(fused_hbm / n_dom),
                        "mfma_tflops": round(mfma_tf, 2),
                        "mfma_frac": round(mfma_tf / PEAK_BF16_TFLOPS, 4)}
        elif n_dom > 0 and t_dom > 0:
            achieved = ex[dom] / (t_dom * 1e-3) / 1e12
            traffic = None
            if dom == "update" and default_ns:
                traffic = traffic_record(f"update_kernel_traffic_{w.name}", n_dom,
                                         os.path.join(csrc, "ns_gemm_mfma.hip"),
                                         os.path.join(csrc, "ns_mfma_common.h"),
                                         os.path.join(csrc, "muon_device.h"))
            what = {"update": "update X' = B' X, B' = a I + b A + c A A", "gram": "Gram A = X X^T",
                    "symsq": "B' = a I + b A + c A A", "prod": "m x m products of the Gram form"}[dom]
            roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic, "kernel": f"ns_gemm_mfma_kernel ({what})",
                        "avg_launch_ms": round(t_dom / n_dom, 4),
                        "flop_per_launch_avg": int(ex[dom] / n_dom)}
        if args.inflight > 1:
            # lanes run concurrently: a launch's event interval includes time
            # it shares the GPU with the other lanes' launches, so per-kernel
            # rates understate the kernels and no roofline is claimed
            roofline = None
            breakdown["note"] = (f"{args.inflight} micro-buckets in flight: per-kernel event times "
                                 "overlap across lanes and sum to more than the step")

    out = {
        "metric": METRIC if args.ns_method == "quintic" else METRIC.replace(
            "Newton–Schulz TFLOP/s", "Newton–Schulz quintic-equivalent TFLOP/s, gram form"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(ms_median, 4),
        "ms_per_step_min": round(ms_min, 4),
        "ms_per_step_max": round(max(per), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.compute,
        "data": "synthetic (seeded N(0,1e-3) bf16 gradients, fp32 state; no checkpoint)",
        "config": {"workload": w.name, "matrices": len(w.mats), "muon_params": numel,
                   "ns_units": len(units), "ns_steps": w.ns_steps, "ns_method": args.ns_method,
                   "ns_coeffs": args.ns_coeffs, "norms": args.norms,
                   "ns_fuse": args.ns_fuse,
                   "micro_bucket_cap_bytes": w.cap_bytes, "cap_kind": w.cap_kind,
                   "micro_buckets": len(ms.plan.buckets), "workspace_bytes": ms.plan.max_workspace,
                   "inflight_micro_buckets": args.inflight, "graph_replay": bool(args.graph),
                   "parallelism": "single GPU"},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "ns_tflop_per_step_algorithmic": round(f_ns / 1e12, 4),
        "ns_tflop_per_step_dense_equiv": round(dense / 1e12, 4),
        "ns_tflop_per_step_executed": round(sum(ex.values()) / 1e12, 4),
        "matrices_per_s": round(len(units) / (ms_per_step * 1e-3), 1),
        "wall_s_timed": round(wall, 3),
        "breakdown": breakdown,
        "breakdown_from": (f"{breakdown_steps} steps after the timed region, every launch between HIP events; "
                           f"the timed steps record events around the {dom} launches only (the roofline's)")
        if timing else None,
        "roofline": roofline,
    }
    if layers_note is not None:
        L = layers_note["layers_run"]
        if L < 48:
            layers_note["ms_per_step_x48_over_L"] = round(ms_per_step * 48 / L, 2)
            layers_note["note"] = (f"{L} of the 48 layers fit in device memory; the 48-layer step time "
                                   f"is extrapolated as x48/{L}, not measured")
        else:
            layers_note["note"] = "all 48 layers measured"
        out["layers"] = layers_note
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ns_steps=w.ns_steps, minimax=args.ns_coeffs == "minimax")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
