"""CPU oracle for the Muon optimizer step: momentum, Newton-Schulz, apply.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
HIP path is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never calls it
and shares no code with it (no kernels, headers, helpers or tables).

What it computes follows the update rule of the blog "Muon Optimizer + FSDP",
section "Background: the conflict between FSDP and Muon":

    M_t = momentum_update(grad)
    U_t = NewtonSchulz(M_t)
    W_t = W_t - lr * U_t

applied to whole 2D matrices (same page and section: orthogonalising shards
separately is not the same as orthogonalising the full matrix), with the
Newton-Schulz step being "the current quintic iteration" of the DeepSpeed RFC
"Enable Correct and High-Performance Muon Optimizer under ZeRO CPU Offload",
section 5 (Roadmap), run for 5 iterations (same RFC, section 2, Root Cause
Analysis, says 5~6).  The pages print neither the polynomial's coefficients
nor the momentum formula; the readings taken here are:

  * momentum (EMA form, Nesterov):  M' = beta*M + (1-beta)*g,
    U_in = (1-beta)*g + beta*M'.  Every multiply and add is a separate IEEE
    binary32 operation rounded to nearest-even (numpy float32), no fused
    multiply-add, denormals kept.
  * Newton-Schulz (float64 throughout): transpose a tall matrix, divide by
    (Frobenius norm + eps), then `steps` times
        A = X X^T ;  B = b A + c A A ;  X = a X + B X
    and undo the transpose.  Default (a, b, c) = (3.4445, -4.7750, 2.0315),
    eps = 1e-7.
  * per-head split: a rows x cols matrix with head_rows = h is treated as
    rows/h contiguous row blocks, each orthogonalised on its own (RFC section
    4D, "Per-Head Muon (MuonSplit)"; blog section "Chunked communication",
    splitting fused tensors into their logical matrices).
  * apply (binary32): eta = lr*scale; W1 = W*(1 - lr*wd) when wd != 0;
    W' = W1 - eta*u; optional bf16 copy of W' rounded to nearest-even.

Pins (tests/test_oracle_*.py, run without a GPU) tie each function to facts
other than itself: the SVD closed form of the odd matrix polynomial, diagonal
and rank-1 inputs, transpose / sign / scale / orthogonal symmetries, an
independent Gram-recursion evaluation, exact rational emulation of the
binary32 momentum and apply sequences, and torch's CPU bfloat16 cast.
"""
from __future__ import annotations

import numpy as np

# Quintic coefficients and iteration count of the default configuration.
NS_A = 3.4445
NS_B = -4.7750
NS_C = 2.0315
NS_STEPS = 5
NS_EPS = 1e-7


# ---------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even), on float32 bit patterns.
# ---------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.  NaN
    stays NaN (quiet), +-inf stay infinite, overflow past the largest finite
    bfloat16 rounds to infinity, as IEEE round-to-nearest-even requires.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    is_nan = np.isnan(f)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    r = np.where(is_nan, (u >> np.uint64(16)) | np.uint64(0x40), r)
    out = (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return out.reshape(f.shape)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16_round(x)."""
    return (bf16_round(x).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    """float32 values of bfloat16 bit patterns (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ---------------------------------------------------------------------------
# Momentum (first-order momentum with Nesterov look-ahead), binary32.
# ---------------------------------------------------------------------------
def momentum_ref(g, M, beta: float = 0.95, nesterov: bool = True):
    """One momentum update per element; returns (M_new, U_in), both float32.

    Follows M_t = momentum_update(grad) of the blog's Background section, in
    EMA form with Nesterov look-ahead.  Operation order (each step one
    binary32 rounding):  c1 = 1 - beta;  t = c1*g;  M' = beta*M + t;
    U_in = t + beta*M'  (or U_in = M' without Nesterov).
    """
    g = np.asarray(g, dtype=np.float32)
    M = np.asarray(M, dtype=np.float32)
    b = np.float32(beta)
    c1 = np.float32(np.float32(1.0) - b)
    t = np.multiply(c1, g, dtype=np.float32)
    bm = np.multiply(b, M, dtype=np.float32)
    M_new = np.add(bm, t, dtype=np.float32)
    if nesterov:
        bmn = np.multiply(b, M_new, dtype=np.float32)
        U = np.add(t, bmn, dtype=np.float32)
    else:
        U = M_new.copy()
    return M_new, U


# ---------------------------------------------------------------------------
# Newton-Schulz orthogonalisation, float64.
# ---------------------------------------------------------------------------
def ns_ref(Y, steps: int = NS_STEPS, a: float = NS_A, b: float = NS_B,
           c: float = NS_C, eps: float = NS_EPS) -> np.ndarray:
    """Quintic Newton-Schulz of one 2D matrix, in float64.

    The iteration drives every singular value of the normalised matrix
    towards the quintic's band around 1 (RFC section 2: the update should
    have unit spectral norm; section 5: the quintic iteration).  A tall
    matrix (rows > cols) is processed as its transpose so that the Gram
    matrix is the small side; the result is transposed back.
    """
    X = np.array(Y, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError("ns_ref expects a 2D matrix")
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X, "fro") + eps)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    if tall:
        X = X.T
    return np.ascontiguousarray(X)


def split_heads(Y, head_rows: int):
    """Contiguous row blocks of `head_rows` rows (head k = rows [k*h, (k+1)*h))."""
    Y = np.asarray(Y)
    if head_rows <= 0:
        return [Y]
    if Y.shape[0] % head_rows:
        raise ValueError("rows must be a multiple of head_rows")
    return [Y[k * head_rows:(k + 1) * head_rows] for k in range(Y.shape[0] // head_rows)]


def ns_ref_heads(Y, head_rows: int = 0, **kw) -> np.ndarray:
    """Per-head Newton-Schulz: each row block on its own, stacked back."""
    if head_rows <= 0:
        return ns_ref(Y, **kw)
    return np.concatenate([ns_ref(blk, **kw) for blk in split_heads(Y, head_rows)], axis=0)


# ---------------------------------------------------------------------------
# Weight apply, binary32.
# ---------------------------------------------------------------------------
def apply_ref(W, u, lr: float, scale: float = 1.0, weight_decay: float = 0.0,
              bf16_copy: bool = False):
    """W' = W1 - (lr*scale)*u with W1 = W*(1 - lr*wd) when wd != 0.

    The blog's Background section writes the apply as W_t = W_t - lr * U_t;
    `scale` and `weight_decay` default to 1 and 0.  Each operation is one
    binary32 rounding.  Returns W' (float32) and, when asked, the bf16 bit
    patterns of W' rounded to nearest-even.
    """
    W = np.asarray(W, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    lr32 = np.float32(lr)
    eta = np.float32(lr32 * np.float32(scale))
    if weight_decay != 0.0:
        decay = np.float32(np.float32(1.0) - np.float32(lr32 * np.float32(weight_decay)))
        W1 = np.multiply(W, decay, dtype=np.float32)
    else:
        W1 = W
    step = np.multiply(eta, u, dtype=np.float32)
    Wn = np.subtract(W1, step, dtype=np.float32)
    if bf16_copy:
        return Wn, bf16_bits(Wn)
    return Wn


# ---------------------------------------------------------------------------
# One whole Muon step over a list of matrices (composition of the above).
# ---------------------------------------------------------------------------
def muon_step_ref(weights, grads, moms, lr: float, beta: float = 0.95,
                  nesterov: bool = True, head_rows=None, update_bf16: bool = False,
                  ns_kw=None):
    """Momentum -> Newton-Schulz -> apply for each matrix, in place on lists.

    `update_bf16` rounds U_in to bf16 before the Newton-Schulz (the bf16
    compute mode feeds bf16 matrices) and rounds the orthogonalised update to
    bf16 before the apply.  Returns the list of float64 Newton-Schulz outputs.
    """
    ns_kw = ns_kw or {}
    outs = []
    for i, (W, g) in enumerate(zip(weights, grads)):
        M_new, U = momentum_ref(g, moms[i], beta, nesterov)
        moms[i] = M_new
        if update_bf16:
            U = bf16_round(U)
        h = 0 if head_rows is None else head_rows[i]
        O = ns_ref_heads(U, h, **ns_kw)
        outs.append(O)
        u = O.astype(np.float32)
        if update_bf16:
            u = bf16_round(u)
        weights[i] = apply_ref(W, u, lr)
    return outs


def rel_fro(x, ref) -> float:
    """Relative Frobenius distance ||x - ref|| / ||ref|| in float64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
