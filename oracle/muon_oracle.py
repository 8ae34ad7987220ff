"""CPU oracle for the Muon optimizer step: momentum, Newton-Schulz, apply.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
HIP path is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never calls it
and shares no code with it (no kernels, headers, helpers or tables).

What it computes follows the update rule of the blog "Muon Optimizer + FSDP",
section "Background: the conflict between FSDP and Muon": the gradient first
refreshes a momentum buffer, the momentum is orthogonalised by Newton-Schulz,
and the weight moves against that orthogonalised update scaled by the
learning rate -- applied to whole 2D matrices (same page and section: orthogonalising shards
separately is not the same as orthogonalising the full matrix), with the
Newton-Schulz step being the quintic iteration that the DeepSpeed RFC
"Enable Correct and High-Performance Muon Optimizer under ZeRO CPU Offload"
names as its current one (section 5, Roadmap), run for 5 iterations (the
same RFC, section 2, Root Cause Analysis, gives five to six).  The pages print neither the polynomial's coefficients
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
  * per-iteration coefficients (RFC section 5, "Polar Express", named but
    not given): each iteration's quintic is the best one, in the maximum
    norm, on the interval that holds the singular values at that point
    (`minimax_schedule`, whose comment block lists the readings).

Pins (tests/test_oracle_*.py, run without a GPU) tie each function to facts
other than itself: the SVD closed form of the odd matrix polynomial, diagonal
and rank-1 inputs, transpose / sign / scale / orthogonal symmetries, an
independent Gram-recursion evaluation, exact rational emulation of the
binary32 momentum and apply sequences, torch's CPU bfloat16 cast, exact
rational sums of squares per block, and for the
per-iteration coefficients a linear-programme solution of the same best
approximation, the alternation property and the closed-form limit polynomial.
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

    The momentum refresh of the blog's Background section, read as an
    exponential moving average with Nesterov look-ahead.  Operation order (each step one
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
# Sums of squares per block (the Frobenius norms' raw material).
# ---------------------------------------------------------------------------
def sumsq_blocks(u, block: int = 4096):
    """Sum of squares of each run of `block` consecutive values (the last run
    may be short), correctly rounded to binary64.

    X_0 = Y / (||Y||_F + eps) needs ||Y||_F^2 = sum of squares of Y's
    elements (RFC section 2; blog "Muon Optimizer + FSDP", Memory control
    item 4 keeps such scalars in FP32 or wider).  Summed per block, a unit
    that spans whole blocks gets its norm from its blocks.  Squares of
    binary32 values are exact in binary64 and math.fsum rounds the exact sum
    once, so the result depends on the values only, not on any order.
    """
    import math
    v = np.asarray(u, dtype=np.float32).astype(np.float64).ravel()
    return np.array([math.fsum((v[b:b + block] ** 2).tolist()) for b in range(0, len(v), block)],
                    dtype=np.float64)


# ---------------------------------------------------------------------------
# Newton-Schulz orthogonalisation, float64.
# ---------------------------------------------------------------------------
def ns_ref(Y, steps: int = NS_STEPS, a: float = NS_A, b: float = NS_B,
           c: float = NS_C, eps: float = NS_EPS, coeffs=None) -> np.ndarray:
    """Quintic Newton-Schulz of one 2D matrix, in float64.

    The iteration drives every singular value of the normalised matrix
    towards the quintic's band around 1 (RFC section 2: the update should
    have unit spectral norm; section 5: the quintic iteration).  A tall
    matrix (rows > cols) is processed as its transpose so that the Gram
    matrix is the small side; the result is transposed back.

    `coeffs`: optional per-iteration coefficients, `steps` rows of (a, b, c);
    iteration k then uses row k instead of the fixed (a, b, c) (RFC section
    5: per-iteration optimised coefficients, see `minimax_schedule`).
    """
    X = np.array(Y, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError("ns_ref expects a 2D matrix")
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X, "fro") + eps)
    rows = [(a, b, c)] * steps
    if coeffs is not None:
        rows = [tuple(float(v) for v in r) for r in np.asarray(coeffs, dtype=np.float64)]
        if len(rows) != steps or any(len(r) != 3 for r in rows):
            raise ValueError("coeffs must hold `steps` rows of (a, b, c)")
    for ak, bk, ck in rows:
        A = X @ X.T
        B = bk * A + ck * (A @ A)
        X = ak * X + B @ X
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
# Per-iteration coefficients (DeepSpeed RFC, section 5 Roadmap: Newton-Schulz
# whose coefficients are optimised for each iteration, "Polar Express", so
# that fewer iterations reach the same accuracy).  The pages name the idea but
# give neither a table nor a derivation; the reading taken here:
#
#   * iteration t applies p_t(x) = a x + b x^3 + c x^5 to every singular
#     value, and p_t is the odd quintic closest to 1 in the maximum norm over
#     the interval [l_t, u_t (1 + margin)] that holds the singular values
#     (greedy: each step the best one for where the values are now);
#   * X_0 is normalised by its Frobenius norm, so u_0 = 1; l_0 = `lo` is the
#     smallest singular value the schedule is built to lift (a parameter);
#   * the values land in p_t's image [1 - E_t, 1 + E_t], the next interval;
#   * `margin` widens each interval at the top: above it the polynomial
#     climbs steeply, and bf16 rounding (2^-8 relative per rounding, a few
#     per iteration) would otherwise push the top values past it and let
#     them grow without bound over the later iterations; near the top the
#     polynomial is also steep inside the interval, so a wider margin lowers
#     how much rounding error the later iterations amplify (default 0.05);
#   * once an interval is narrower than 1e-3 the limit of the best
#     polynomial as the interval shrinks to {1} is used:
#     (a, b, c) = (15/8, -5/4, 3/8), which matches 1 to third order at 1 and
#     is increasing everywhere, p'(x) = (15/8) (1 - x^2)^2.
# ---------------------------------------------------------------------------
MINIMAX_LO = 1e-3
MINIMAX_MARGIN = 0.05
LIMIT_QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)


def minimax_quintic(lo: float, hi: float, iters: int = 100):
    """Odd quintic p minimising max over [lo, hi] of |1 - p(x)|, 0 < lo < hi.

    Remez exchange on four reference points.  The error 1 - p of the best p
    alternates in sign on four points (Chebyshev alternation for the Haar
    system x, x^3, x^5 on an interval away from 0); p has at most two
    interior critical points (p' is a quadratic in x^2), so the endpoints are
    two of them.  Each round solves p(x_i) + s_i E = 1 with s = (+, -, +, -)
    and moves the two interior points to the new critical points.
    Returns (a, b, c, E), E = max |1 - p| on [lo, hi].
    """
    lo, hi = float(lo), float(hi)
    if not (0.0 < lo < hi):
        raise ValueError("need 0 < lo < hi")
    x = np.array([lo, 0.0, 0.0, hi])
    x[1:3] = lo + (hi - lo) * (1.0 - np.cos(np.pi * np.array([1.0, 2.0]) / 3.0)) / 2.0
    sign = np.array([1.0, -1.0, 1.0, -1.0])
    for _ in range(iters):
        M = np.stack([x, x ** 3, x ** 5, sign], axis=1)
        a, b, c, E = np.linalg.solve(M, np.ones(4))
        disc = 9.0 * b * b - 20.0 * a * c
        if c == 0.0 or disc < 0.0:
            raise ArithmeticError("Remez lost the alternation")
        roots = np.sort([(-3.0 * b - np.sqrt(disc)) / (10.0 * c),
                         (-3.0 * b + np.sqrt(disc)) / (10.0 * c)])
        if not (lo * lo < roots[0] < roots[1] < hi * hi):
            raise ArithmeticError("Remez lost the alternation")
        xn = np.array([lo, np.sqrt(roots[0]), np.sqrt(roots[1]), hi])
        done = np.max(np.abs(xn - x)) <= 1e-15 * hi
        x = xn
        if done:
            break
    M = np.stack([x, x ** 3, x ** 5, sign], axis=1)
    a, b, c, E = np.linalg.solve(M, np.ones(4))
    return float(a), float(b), float(c), float(abs(E))


def quintic_eval(coef, x):
    """p(x) = a x + b x^3 + c x^5."""
    a, b, c = coef
    x = np.asarray(x, dtype=np.float64)
    return a * x + b * x ** 3 + c * x ** 5


def minimax_schedule(steps: int, lo: float = MINIMAX_LO, margin: float = MINIMAX_MARGIN):
    """Per-iteration (a, b, c) rows (steps x 3, float64) and the final bound.

    Returns (rows, E): every singular value of X_0 in [lo, 1] ends, in exact
    arithmetic, within [1 - E, 1 + E] after the `steps` iterations.
    """
    if steps < 1 or not (0.0 < lo < 1.0) or not (0.0 <= margin <= 0.5):
        raise ValueError("steps >= 1, 0 < lo < 1, 0 <= margin <= 0.5")
    l, u = float(lo), 1.0
    rows = []
    E = 1.0 - l
    for _ in range(steps):
        top = u * (1.0 + margin)
        if top - l < 1e-3:
            coef = LIMIT_QUINTIC
            # increasing everywhere: the extremes sit at the ends
            E = max(1.0 - float(quintic_eval(coef, l)), float(quintic_eval(coef, top)) - 1.0)
        else:
            a, b, c, E = minimax_quintic(l, top)
            coef = (a, b, c)
        rows.append(coef)
        l, u = 1.0 - E, 1.0 + E
    return np.array(rows, dtype=np.float64), float(E)


# ---------------------------------------------------------------------------
# Weight apply, binary32.
# ---------------------------------------------------------------------------
def apply_ref(W, u, lr: float, scale: float = 1.0, weight_decay: float = 0.0,
              bf16_copy: bool = False):
    """W' = W1 - (lr*scale)*u with W1 = W*(1 - lr*wd) when wd != 0.

    The blog's Background section moves the weight against the orthogonalised
    update times the learning rate; `scale` and `weight_decay` default to 1
    and 0.  Each operation is one
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
