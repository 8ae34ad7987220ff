"""Pins for the oracle's Newton-Schulz (CPU only).

Each check compares the oracle against something that is not the oracle:
the SVD closed form of an odd matrix polynomial, the scalar recursion on a
diagonal or rank-1 input, algebraic symmetries, an independent Gram-recursion
evaluation, and the band the quintic maps singular values into.  Mutation
tests plant plausible mistakes in a copy of the iteration and show that the
pins reject them.
"""
import numpy as np
import pytest

from oracle import NS_A, NS_B, NS_C, NS_EPS, NS_STEPS, ns_ref, ns_ref_heads, rel_fro

C1_SHAPES = [(64, 128), (128, 128), (256, 64), (96, 96)]


def p_scalar(s, steps=NS_STEPS, a=NS_A, b=NS_B, c=NS_C):
    """The quintic a*s + b*s^3 + c*s^5 iterated `steps` times (Python floats)."""
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def closed_form(Y, steps=NS_STEPS, eps=NS_EPS):
    """Each iteration is an odd polynomial in X acting on singular values:
    NS(Y) = U diag(p^steps(sigma_i / (||Y||_F + eps))) V^T."""
    U, s, Vt = np.linalg.svd(np.asarray(Y, dtype=np.float64), full_matrices=False)
    fro = float(np.sqrt(np.sum(s * s)))
    sig = s / (fro + eps)
    sig = np.array([p_scalar(float(v), steps) for v in sig])
    return (U * sig) @ Vt


def gaussian(rng, r, c):
    return rng.standard_normal((r, c))


def haar(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


# --------------------------------------------------------------------------
# pins used below and by the mutation tests
# --------------------------------------------------------------------------
def check_closed_form(fn, rng, shapes=C1_SHAPES + [(40, 200), (200, 40)], tol=1e-10):
    for (r, c) in shapes:
        Y = gaussian(rng, r, c)
        err = rel_fro(fn(Y), closed_form(Y))
        assert err < tol, f"{r}x{c}: closed-form error {err:.3e}"


def check_diagonal(fn, shapes=((5, 9), (9, 5), (7, 7))):
    for (r, c) in shapes:
        k = min(r, c)
        d = np.linspace(0.1, 2.0, k) * (-1.0) ** np.arange(k)
        Y = np.zeros((r, c))
        Y[np.arange(k), np.arange(k)] = d
        fro = float(np.sqrt(np.sum(d * d)))
        want = np.zeros((r, c))
        for i in range(k):
            want[i, i] = p_scalar(float(d[i]) / (fro + NS_EPS))
        got = fn(Y)
        assert np.max(np.abs(got - want)) < 1e-13, (r, c)


def check_square_transpose(fn, rng, n=48):
    Y = gaussian(rng, n, n) + 0.5 * np.eye(n)
    assert rel_fro(fn(Y.T), fn(Y).T) < 1e-12


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def test_coefficients_fixed_points():
    # p(1) = a + b + c; the quintic has fixed points 0, +-0.868.., +-1.2637..
    assert abs((NS_A + NS_B + NS_C) - 0.701) < 1e-12
    p = np.polynomial.Polynomial([0.0, NS_A - 1.0, 0.0, NS_B, 0.0, NS_C])
    roots = sorted(r.real for r in p.roots() if abs(r.imag) < 1e-12 and r.real > 0)
    assert abs(roots[0] - 0.8680) < 1e-3 and abs(roots[1] - 1.2637) < 1e-3


def test_closed_form_svd(rng):
    check_closed_form(ns_ref, rng)


def test_diagonal_scalar_recursion():
    check_diagonal(ns_ref)


def test_rank_one():
    rng = np.random.default_rng(7)
    u = rng.standard_normal(30); u /= np.linalg.norm(u)
    v = rng.standard_normal(70); v /= np.linalg.norm(v)
    for s in (1e-3, 1.0, 250.0):
        Y = s * np.outer(u, v)
        want = p_scalar(s / (s + NS_EPS)) * np.outer(u, v)
        assert rel_fro(ns_ref(Y), want) < 1e-12
    # hand value of p^5(1): 1 -> 0.701 -> ... (five applications of the quintic)
    assert abs(p_scalar(1.0) - 0.69644) < 5e-5


def test_zero_matrix_is_zero():
    for (r, c) in C1_SHAPES:
        out = ns_ref(np.zeros((r, c)))
        assert out.shape == (r, c) and not np.any(out)


def test_transpose_symmetry(rng):
    for (r, c) in C1_SHAPES:
        Y = gaussian(rng, r, c)
        assert rel_fro(ns_ref(Y.T), ns_ref(Y).T) < 1e-12
    check_square_transpose(ns_ref, rng)


def test_sign_and_scale(rng):
    for (r, c) in C1_SHAPES:
        Y = gaussian(rng, r, c)
        base = ns_ref(Y)
        assert np.array_equal(ns_ref(-Y), -base)
        for alpha in (1e-2, 3.0, 1e3):
            # invariant up to the eps term: O(eps / ||Y||)
            assert rel_fro(ns_ref(alpha * Y), base) < 1e-6


def test_orthogonal_equivariance(rng):
    for (r, c) in [(64, 128), (96, 96), (256, 64)]:
        Y = gaussian(rng, r, c)
        Q, R = haar(rng, r), haar(rng, c)
        assert rel_fro(ns_ref(Q @ Y @ R), Q @ ns_ref(Y) @ R) < 1e-10


def test_band_around_one(rng):
    # non-square Gaussian inputs: every singular value lands in the quintic's
    # attracting band [0.6818, 1.1344]
    for (r, c) in [(64, 128), (256, 64), (128, 2560), (768, 2048)]:
        s = np.linalg.svd(ns_ref(gaussian(rng, r, c)), compute_uv=False)
        assert s.min() > 0.68 and s.max() < 1.135, (r, c, s.min(), s.max())
    # so the spectral distance to the exact polar factor U V^T stays within 0.32
    Y = gaussian(rng, 64, 128)
    U, _, Vt = np.linalg.svd(Y, full_matrices=False)
    assert np.linalg.norm(ns_ref(Y) - U @ Vt, 2) < 0.32


def test_gram_recursion_second_path(rng):
    """X_k = P_{k-1} ... P_0 X_0 with P_k = aI + bA_k + cA_k^2 and
    A_{k+1} = P_k A_k P_k: an evaluation that never forms the X iterates."""
    for (r, c) in C1_SHAPES:
        Y = gaussian(rng, r, c)
        X0 = Y.T if r > c else Y
        X0 = X0 / (np.sqrt(np.sum(X0 * X0)) + NS_EPS)
        m = X0.shape[0]
        A = X0 @ X0.T
        Pacc = np.eye(m)
        for _ in range(NS_STEPS):
            P = NS_A * np.eye(m) + NS_B * A + NS_C * (A @ A)
            Pacc = P @ Pacc
            A = P @ A @ P
        X = Pacc @ X0
        X = X.T if r > c else X
        assert rel_fro(ns_ref(Y), X) < 1e-11


def test_per_head_blocks(rng):
    h, heads, cols = 16, 4, 80
    blocks = [gaussian(rng, h, cols) for _ in range(heads)]
    Y = np.concatenate(blocks, axis=0)
    per_head = ns_ref_heads(Y, h)
    for k, blk in enumerate(blocks):
        assert np.array_equal(per_head[k * h:(k + 1) * h], ns_ref(blk))
    # orthogonalising the stacked matrix is a different update (blog section
    # "Background": orthogonalising the shards is not the shard of the whole)
    assert rel_fro(ns_ref(Y), per_head) > 0.05
    # a shard of heads gives the same rows as the whole per-head result
    assert np.array_equal(ns_ref_heads(Y[h:3 * h], h), per_head[h:3 * h])


def test_steps_and_coefficients_are_parameters(rng):
    Y = gaussian(rng, 32, 48)
    for steps in (1, 3, 6):
        assert rel_fro(ns_ref(Y, steps=steps), closed_form(Y, steps=steps)) < 1e-10


# --------------------------------------------------------------------------
# mutation tests: plausible mistakes in the iteration fail the pins above
# --------------------------------------------------------------------------
def _mutant(kind):
    def fn(Y):
        X = np.array(Y, dtype=np.float64)
        tall = X.shape[0] > X.shape[1]
        if tall:
            X = X.T
        if kind == "spectral_norm":
            X = X / (np.linalg.norm(X, 2) + NS_EPS)
        else:
            X = X / (np.linalg.norm(X) + NS_EPS)
        for _ in range(NS_STEPS):
            A = X @ X.T
            if kind == "dropped_square":
                B = NS_B * A + NS_C * A
            elif kind == "swapped_bc":
                B = NS_C * A + NS_B * (A @ A)
            elif kind == "gram_wrong_side":
                A = X.T @ X
                B = NS_B * A + NS_C * (A @ A)
                X = NS_A * X + X @ B
                continue
            else:
                B = NS_B * A + NS_C * (A @ A)
            if kind == "minus_a":
                X = -NS_A * X + B @ X
            else:
                X = NS_A * X + B @ X
        if tall and kind != "no_untranspose":
            X = X.T
        return X
    return fn


@pytest.mark.parametrize("kind", ["dropped_square", "swapped_bc", "minus_a", "spectral_norm",
                                  "no_untranspose"])
def test_mutants_fail_closed_form(kind, rng):
    with pytest.raises((AssertionError, ValueError)):
        check_closed_form(_mutant(kind), rng)


def test_reference_passes_mutation_harness(rng):
    # the un-mutated iteration written the same way passes every pin
    fn = _mutant("none")
    check_closed_form(fn, rng)
    check_diagonal(fn)
    # and moving the Gram to the other side is equivalent in exact arithmetic
    check_closed_form(_mutant("gram_wrong_side"), rng)
