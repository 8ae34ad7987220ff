"""Seeded synthetic workloads: matrix shapes and random draws only.

Shared by the tests, the smoke check and the benchmark; it holds no step of
the optimizer's arithmetic.  Every draw goes through one torch.Generator per
workload, in a fixed order, so a device run and a host copy see identical
values.  "N(0, s)" means standard deviation s.

Shapes stand in for real models (no checkpoints are used):
  * Qwen3-4B decoder layer: hidden 2560, 32 query heads and 8 key/value heads
    of 128, FFN 9728, 36 layers (the DeepSpeed PR "[Muon] CPU offload: pin the
    momentum and overlap the host writeback", section Performance, benchmarks
    these shapes).
  * Qwen3-30B-A3B routed experts: 48 layers x 128 experts with gate/up
    768x2048 and down 2048x768 (prime-rl PR "feat: overlap CPU optimizer with
    backward", section Results, names the model).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

QWEN3_4B_LAYER = [
    # name, rows, cols, head_rows (for the per-head workload)
    ("q_proj", 4096, 2560, 128),
    ("k_proj", 1024, 2560, 128),
    ("v_proj", 1024, 2560, 128),
    ("o_proj", 2560, 4096, 0),
    ("gate_proj", 9728, 2560, 0),
    ("up_proj", 9728, 2560, 0),
    ("down_proj", 2560, 9728, 0),
]
QWEN3_30B_EXPERT = [("gate_proj", 768, 2048), ("up_proj", 768, 2048), ("down_proj", 2048, 768)]


@dataclass
class MatrixSpec:
    name: str
    rows: int
    cols: int
    head_rows: int = 0      # 0: the whole matrix is one Newton-Schulz unit
    zero_grad: bool = False  # expert left without tokens: gradient is exactly 0

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclass
class Workload:
    name: str
    mats: List[MatrixSpec]
    seed: int
    grad_std: float
    weight_std: float = 0.02
    grad_dtype: torch.dtype = torch.bfloat16
    compute: str = "bf16"          # "bf16" or "f32"
    beta: float = 0.95
    nesterov: bool = True
    lr: float = 0.02
    ns_steps: int = 5
    steps: int = 1                 # optimizer steps the workload runs
    warmup_momentum_steps: int = 0  # momentum-only steps that pre-fill M
    cap_bytes: int = 1 << 30
    cap_kind: str = "full"         # "full": full-matrix bytes; "workspace": NS workspace bytes
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def numel(self) -> int:
        return sum(m.numel for m in self.mats)


def tiny() -> Workload:
    shapes = [(64, 128), (128, 128), (256, 64), (96, 96)]
    return Workload(
        name="tiny_fp32", seed=0, grad_std=1.0, grad_dtype=torch.float32, compute="f32",
        mats=[MatrixSpec(f"w{i}", r, c) for i, (r, c) in enumerate(shapes)], steps=3,
        description="4 matrices 64x128, 128x128, 256x64, 96x96; fp32; 3 optimizer steps")


def qwen3_4b(layers: int = 36, seed: int = 2, cap_bytes: int = 512 << 20,
             warmup: int = 2) -> Workload:
    mats = [MatrixSpec(f"layers.{l}.{n}", r, c) for l in range(layers) for (n, r, c, _) in QWEN3_4B_LAYER]
    return Workload(
        name=f"qwen3_4b_{layers}l", mats=mats, seed=seed, grad_std=1e-3, cap_bytes=cap_bytes,
        warmup_momentum_steps=warmup,
        description=f"Qwen3-4B-shaped Muon matrices, {layers} layer(s) x 7")


def qwen3_4b_layer() -> Workload:
    w = qwen3_4b(layers=1, seed=1, cap_bytes=1 << 30, warmup=0)
    w.name = "qwen3_4b_layer"
    return w


def qwen3_4b_heads(layers: int = 36) -> Workload:
    mats = [MatrixSpec(f"layers.{l}.{n}", r, c, h)
            for l in range(layers) for (n, r, c, h) in QWEN3_4B_LAYER if h]
    return Workload(
        name=f"qwen3_4b_heads_{layers}l", mats=mats, seed=3, grad_std=1e-3, cap_bytes=1 << 40,
        description=f"per-head Newton-Schulz on q/k/v, 128x2560 heads, {layers} layer(s)")


def qwen3_30b_experts(layers: int = 48, experts: int = 128, zero_frac: float = 0.25,
                      seed: int = 4) -> Workload:
    """Expert matrices, expert-major within each layer.  Which experts get a
    zero gradient is drawn per layer with torch.randperm on the workload's
    generator, before any matrix is drawn (see zero_experts())."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    nzero = int(round(zero_frac * experts))
    mats = []
    for l in range(layers):
        zero = set(torch.randperm(experts, generator=g)[:nzero].tolist())
        for e in range(experts):
            for (n, r, c) in QWEN3_30B_EXPERT:
                mats.append(MatrixSpec(f"layers.{l}.experts.{e}.{n}", r, c, 0, e in zero))
    return Workload(
        name=f"qwen3_30b_a3b_experts_{layers}l", mats=mats, seed=seed, grad_std=1e-3,
        cap_bytes=1 << 30, cap_kind="workspace",
        description=f"{layers} layers x {experts} experts x (768x2048, 768x2048, 2048x768); "
                    f"{nzero}/{experts} experts per layer with zero gradients")


def generator(seed: int, device) -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def normal(shape, std: float, gen: torch.Generator, device, dtype=torch.float32) -> torch.Tensor:
    """fp32 N(0, std) draw, then cast (round to nearest even) to `dtype`."""
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def draw_grads(w: Workload, gen: torch.Generator, device, out: Optional[List[torch.Tensor]] = None):
    """One gradient per matrix in workload order (zero for zero_grad matrices).

    With `out`, fills the given tensors in place (shapes must match)."""
    res = []
    for i, m in enumerate(w.mats):
        if m.zero_grad:
            t = torch.zeros((m.rows, m.cols), device=device, dtype=w.grad_dtype)
        else:
            t = normal((m.rows, m.cols), w.grad_std, gen, device, w.grad_dtype)
        if out is not None:
            out[i].copy_(t)
            res.append(out[i])
        else:
            res.append(t)
    return res


def iter_weights(w: Workload, gen: torch.Generator, device):
    """The fp32 master weights one matrix at a time, in workload order (the
    draws of draw_weights, without holding them all)."""
    for m in w.mats:
        yield normal((m.rows, m.cols), w.weight_std, gen, device, torch.float32)


def draw_weights(w: Workload, gen: torch.Generator, device):
    return list(iter_weights(w, gen, device))


# Spectra that Gaussian draws do not reach.  Newton-Schulz lifts every
# singular value towards 1, small ones by up to a^steps, so inputs whose
# spectrum spans many orders of magnitude exercise precision that an i.i.d.
# Gaussian matrix (singular values within about one order) does not.
STRUCTURED_KINDS = ("gauss", "rank1", "rank8_noise", "geometric")


def structured(kind: str, rows: int, cols: int, seed: int, std: float = 1e-3,
               scale: float = 1.0, device=None, dtype=torch.bfloat16) -> torch.Tensor:
    """A seeded rows x cols matrix with a chosen spectrum, drawn on the host in
    float64 (torch CPU generator, so the values do not depend on the device),
    multiplied by `scale`, cast to `dtype` (round to nearest even) and moved
    to `device`.

      gauss        i.i.d. N(0, std)
      rank1        std * u v^T, u and v i.i.d. N(0, 1)
      rank8_noise  std * L R / sqrt(8) (L rows x 8, R 8 x cols, N(0, 1)) plus
                   i.i.d. N(0, 1e-3 std) noise: eight large singular values
                   over a floor about 1e-3 below them
      geometric    std * Q1 diag(sigma) Q2^T with Haar-random orthonormal Q1,
                   Q2 (QR of Gaussian draws, signs fixed by R's diagonal) and
                   sigma_i = 10^(-6 i / (k - 1)), k = min(rows, cols): a
                   geometric spectrum over six decades
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    f64 = torch.float64
    if kind == "gauss":
        y = torch.randn(rows, cols, generator=g, dtype=f64) * std
    elif kind == "rank1":
        y = torch.outer(torch.randn(rows, generator=g, dtype=f64),
                        torch.randn(cols, generator=g, dtype=f64)) * std
    elif kind == "rank8_noise":
        L = torch.randn(rows, 8, generator=g, dtype=f64)
        R = torch.randn(8, cols, generator=g, dtype=f64)
        y = (L @ R) * (std / 8 ** 0.5) + torch.randn(rows, cols, generator=g, dtype=f64) * (1e-3 * std)
    elif kind == "geometric":
        k = min(rows, cols)

        def haar(n, p):
            q, r = torch.linalg.qr(torch.randn(n, p, generator=g, dtype=f64))
            return q * torch.sign(torch.diagonal(r))

        sig = 10.0 ** (-6.0 * torch.arange(k, dtype=f64) / max(k - 1, 1))
        y = (haar(rows, k) * sig) @ haar(cols, k).T * std
    else:
        raise ValueError(f"unknown spectrum kind {kind!r}")
    y = (y * scale).to(torch.float32).to(dtype)
    return y.to(device) if device is not None else y
