"""Pins of oracle.muon_step_ref, the whole-step composition (momentum ->
Newton-Schulz -> apply, blog "Muon Optimizer + FSDP", section "Background"),
against closed forms it does not compute itself.

With a constant gradient G and momentum starting at zero, the moving average
after t steps is (1 - beta^t) G in real arithmetic and the Nesterov look-ahead
(1 - beta) G + beta M_t is (1 - beta^(t+1)) G.  For a diagonal G the Newton-
Schulz output is diagonal, each entry the scalar quintic recursion applied to
u_i / (||u|| + eps).  The weights must move by -lr times the sum of the
steps' outputs.  A step that forgets the momentum carry, drops Nesterov,
skips the bf16 rounding it is asked for, or applies with the wrong sign or
learning rate fails one of these.
"""
import math

import numpy as np
import pytest
import torch

import oracle

BETA, LR = 0.95, 0.02


def scalar_ns(u, steps=5, a=oracle.NS_A, b=oracle.NS_B, c=oracle.NS_C, eps=oracle.NS_EPS):
    """Newton-Schulz of diag(u) by the scalar recursion, in Python floats."""
    nrm = math.sqrt(sum(float(x) * float(x) for x in u)) + eps
    out = []
    for x in u:
        s = float(x) / nrm
        for _ in range(steps):
            s = a * s + b * s ** 3 + c * s ** 5
        out.append(s)
    return out


def diag_matrix(rows, cols, vals):
    G = np.zeros((rows, cols), np.float32)
    for i, v in enumerate(vals):
        G[i, i] = v
    return G


def torch_bf16(x):
    """bf16 rounding by torch's CPU cast (independent of oracle.bf16_round)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("rows,cols", [(6, 9), (10, 4), (5, 5)])
def test_two_steps_constant_diagonal_gradient(rows, cols):
    k = min(rows, cols)
    d = np.array([0.5, -1.25, 2.0, 0.75, -0.3, 1.1, 0.9, -2.2, 0.05, 1.7][:k], np.float32)
    G = diag_matrix(rows, cols, d)
    rng = np.random.default_rng(rows * cols)
    W0 = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    weights, moms = [W0.copy()], [np.zeros_like(G)]
    total = np.zeros((rows, cols))
    for t in (1, 2):
        outs = oracle.muon_step_ref(weights, [G], moms, LR, BETA, True)
        # the momentum is carried from step to step: (1 - beta^t) G
        np.testing.assert_allclose(moms[0], (1.0 - BETA ** t) * G.astype(np.float64), rtol=1e-6, atol=0)
        # Newton-Schulz of the look-ahead (1 - beta^(t+1)) G
        u = (1.0 - BETA ** (t + 1)) * d.astype(np.float64)
        exp = diag_matrix(rows, cols, scalar_ns(u)).astype(np.float64)
        O = outs[0]
        assert O.shape == (rows, cols)
        np.testing.assert_allclose(O, exp, rtol=0, atol=1e-6)
        total += O
        # apply: W_t - W_0 = -lr * (sum of outputs), to binary32 rounding of W
        np.testing.assert_allclose(weights[0].astype(np.float64) - W0, -LR * total, rtol=0, atol=4 * 2.0 ** -24 * 0.1)


def test_two_steps_without_nesterov():
    d = np.array([1.0, -0.5, 0.25], np.float32)
    G = diag_matrix(3, 7, d)
    weights, moms = [np.zeros_like(G)], [np.zeros_like(G)]
    for t in (1, 2):
        outs = oracle.muon_step_ref(weights, [G], moms, LR, BETA, False)
        np.testing.assert_allclose(moms[0], (1.0 - BETA ** t) * G.astype(np.float64), rtol=1e-6, atol=0)
        # without look-ahead the update is the momentum itself; its scale
        # cancels in the normalisation, so the output equals NS(diag(d))
        exp = diag_matrix(3, 7, scalar_ns((1.0 - BETA ** t) * d.astype(np.float64)))
        np.testing.assert_allclose(outs[0], exp, rtol=0, atol=1e-6)


def test_bf16_rounding_of_the_update():
    # look-ahead values chosen so that rounding to bf16 moves them: the
    # Newton-Schulz input must be the bf16-rounded U, and the applied update
    # the bf16-rounded output
    d = np.array([1.0 + 2.0 ** -10, -(3.0 + 2.0 ** -9), 0.7 + 2.0 ** -12, 0.0], np.float32)
    G = diag_matrix(4, 6, d)
    W0 = np.full((4, 6), 0.5, np.float32)
    weights, moms = [W0.copy()], [np.zeros_like(G)]
    outs = oracle.muon_step_ref(weights, [G], moms, LR, BETA, True, update_bf16=True)
    # U as binary32 from the momentum sequence, then bf16 by torch's cast
    c1 = np.float32(1.0) - np.float32(BETA)
    t = (c1 * d).astype(np.float32)
    M = t  # beta * 0 + t
    U = (t + (np.float32(BETA) * M).astype(np.float32)).astype(np.float32)
    Ub = torch_bf16(U)
    assert not np.array_equal(Ub, U)  # the rounding is visible
    exp = scalar_ns(Ub.astype(np.float64))
    np.testing.assert_allclose(np.diag(outs[0][:, :4]), exp, rtol=0, atol=1e-12)
    # the apply sees bf16(O) in binary32 arithmetic: W' = W - f32(lr) * bf16(O)
    ob = torch_bf16(np.asarray(exp, np.float32))
    for i in range(4):
        want = np.float32(np.float32(0.5) - np.float32(np.float32(LR) * ob[i]))
        assert weights[0][i, i] == want, i
    # entries off the diagonal have a zero update and keep their weight
    off = ~np.eye(4, 6, dtype=bool)
    assert np.array_equal(weights[0][off], W0[off])


def test_per_head_rows_are_independent():
    # two heads of 2 x 5, block-diagonal gradient: each head is its own
    # diagonal matrix with its own normalisation
    G = np.zeros((4, 5), np.float32)
    G[0, 0], G[1, 1] = 1.0, 0.5
    G[2, 2], G[3, 3] = 4.0, -0.25
    weights, moms = [np.zeros_like(G)], [np.zeros_like(G)]
    outs = oracle.muon_step_ref(weights, [G], moms, LR, BETA, True, head_rows=[2])
    u = (1.0 - BETA ** 2) * G.astype(np.float64)
    h0 = scalar_ns([u[0, 0], u[1, 1]])
    h1 = scalar_ns([u[2, 2], u[3, 3]])
    got = [outs[0][0, 0], outs[0][1, 1], outs[0][2, 2], outs[0][3, 3]]
    np.testing.assert_allclose(got, h0 + h1, rtol=0, atol=1e-6)
    # whole-matrix normalisation would differ
    whole = scalar_ns([u[0, 0], u[1, 1], u[2, 2], u[3, 3]])
    assert max(abs(x - y) for x, y in zip(got, whole)) > 1e-2
