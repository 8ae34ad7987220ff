"""Pins for the oracle's momentum, apply and bfloat16 rounding (CPU only).

The binary32 operation sequences are checked against an exact rational
emulation of IEEE 754 binary32 round-to-nearest-even written here from the
standard's definition (Fractions, no floating point), on random and
edge-case elements; bfloat16 rounding is checked against torch's CPU cast.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import apply_ref, bf16_bits, bf16_from_bits, bf16_round, momentum_ref, sumsq_blocks

# ---------------------------------------------------------------------------
# exact binary32 rounding from the definition
# ---------------------------------------------------------------------------
_EMIN = -126
_P = 24
_MAXF = Fraction((1 << 24) - 1, 1) * Fraction(2) ** (127 - 23)


def _floor_log2(q: Fraction) -> int:
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round32(q: Fraction) -> Fraction:
    """Nearest binary32 value to q, ties to even; overflow -> inf (as None)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), _EMIN)
    ulp = Fraction(2) ** (e - (_P - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r > _MAXF:
        return None
    return sign * r


def F(x) -> Fraction:
    return Fraction(float(x))


def mul(x, y):
    return round32(x * y)


def add(x, y):
    return round32(x + y)


def sample_f32(rng, n):
    """Random float32 values over many binades, plus zeros and subnormals."""
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(-40, 20, n)
    sign = rng.choice([-1.0, 1.0], n)
    x = (sign * mant * np.exp2(exp)).astype(np.float32)
    x[:8] = np.array([0.0, -0.0, 1e-45, -3e-44, 1.17e-38, 2.0 ** -130, 1.0, -1.0], dtype=np.float32)
    return x


def test_round32_definition():
    # spot checks of the emulator itself against exactly known binary32 facts
    assert round32(Fraction(1, 3)) == F(np.float32(1.0 / 3.0))
    assert round32(Fraction(1) + Fraction(2) ** -24) == 1            # tie -> even
    assert round32(Fraction(1) + Fraction(3, 2 ** 25)) == 1 + Fraction(2) ** -23
    assert round32(Fraction(2) ** -149) == Fraction(2) ** -149       # smallest subnormal
    assert round32(Fraction(2) ** -151) == 0                         # below half of it
    assert round32(_MAXF * 2) is None


@pytest.mark.parametrize("nesterov", [True, False])
@pytest.mark.parametrize("beta", [0.95, 0.9, 0.5])
def test_momentum_matches_exact_binary32(nesterov, beta):
    rng = np.random.default_rng(1)
    n = 400
    g = sample_f32(rng, n)
    M = sample_f32(rng, n)[::-1].copy()
    Mn, U = momentum_ref(g, M, beta, nesterov)
    b = F(np.float32(beta))
    c1 = round32(1 - b)
    assert c1 == 1 - b  # Sterbenz: exact for beta in [0.5, 1]
    for i in range(n):
        t = mul(c1, F(g[i]))
        m_new = add(mul(b, F(M[i])), t)
        u = add(t, mul(b, m_new)) if nesterov else m_new
        assert F(Mn[i]) == m_new, i
        assert F(U[i]) == u, i


def test_momentum_constant_gradient_closed_form():
    # from M = 0 with a constant g, the EMA momentum is (1 - beta^t) g
    g = np.full(16, 0.37, dtype=np.float32)
    M = np.zeros(16, dtype=np.float32)
    for t in range(1, 8):
        M, _ = momentum_ref(g, M, 0.95, True)
        want = (1.0 - 0.95 ** t) * float(g[0])
        assert abs(float(M[0]) - want) <= 8 * np.spacing(np.float32(want)), t


def test_momentum_hand_values():
    # beta = 0.95, g = 1, M = 0 worked by hand in binary32:
    #   f32(0.95) = 15938355 / 2^24, so c1 = 1 - f32(0.95) = 838861 / 2^24 exactly;
    #   t = c1; M' = t; U = t + f32(f32(0.95) * t)
    b = np.float32(0.95)
    c1 = np.float32(1.0) - b
    assert F(b) == Fraction(15938355, 2 ** 24)
    assert F(c1) == Fraction(838861, 2 ** 24)
    Mn, U = momentum_ref(np.ones(1, np.float32), np.zeros(1, np.float32), 0.95, True)
    assert float(Mn[0]) == float(c1)
    assert float(U[0]) == float(np.float32(c1 + np.float32(b * c1)))
    assert abs(float(U[0]) - 0.0975) < 1e-7


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_apply_matches_exact_binary32(wd):
    rng = np.random.default_rng(2)
    n = 400
    W = sample_f32(rng, n)
    u = sample_f32(rng, n)[::-1].copy()
    lr, scale = 0.02, 1.5
    Wn = apply_ref(W, u, lr, scale, wd)
    eta = mul(F(np.float32(lr)), F(np.float32(scale)))
    if wd:
        decay = round32(1 - mul(F(np.float32(lr)), F(np.float32(wd))))
    for i in range(n):
        w1 = mul(F(W[i]), decay) if wd else F(W[i])
        want = round32(w1 - mul(eta, F(u[i])))
        assert F(Wn[i]) == want, i


def test_apply_zero_update_is_identity():
    rng = np.random.default_rng(3)
    W = sample_f32(rng, 300)
    Wn = apply_ref(W, np.zeros_like(W), 0.02)
    assert np.array_equal(Wn.view(np.uint32), W.view(np.uint32))


def test_apply_bf16_copy_matches_torch_cast():
    rng = np.random.default_rng(4)
    W = rng.standard_normal(1000).astype(np.float32) * 0.02
    u = rng.standard_normal(1000).astype(np.float32)
    Wn, bits = apply_ref(W, u, 0.02, bf16_copy=True)
    tb = torch.from_numpy(Wn).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, tb)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        sample_f32(rng, 5000),
        # exact ties: low 16 bits 0x8000 with even and odd kept lsb
        (np.arange(0x3F800000, 0x3F800000 + 64 * 0x10000, 0x10000, dtype=np.uint32) | 0x8000).view(np.float32),
        np.array([np.inf, -np.inf, np.finfo(np.float32).max, -np.finfo(np.float32).max,
                  np.finfo(np.float32).tiny, 1e-40, -1e-40], dtype=np.float32),
    ]).astype(np.float32)
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # round trip of bf16 values is exact
    assert np.array_equal(bf16_round(bf16_from_bits(ours)), bf16_from_bits(ours))
    # NaN stays NaN
    assert np.isnan(bf16_round(np.array([np.nan], dtype=np.float32)))[0]


# ---------------------------------------------------------------------------
# sums of squares per block
# ---------------------------------------------------------------------------
def test_sumsq_blocks_exact_rational():
    """Against exact rational arithmetic: the binary64 value nearest to the
    true sum of squares of each block."""
    rng = np.random.default_rng(11)
    u = (rng.standard_normal(3 * 64 + 17) * 10.0 ** rng.uniform(-8, 3, 3 * 64 + 17)).astype(np.float32)
    got = sumsq_blocks(u, 64)
    assert len(got) == 4
    for b in range(4):
        exact = sum((Fraction(float(x)) ** 2 for x in u[64 * b:64 * b + 64]), Fraction(0))
        assert got[b] == float(exact)        # float(Fraction) rounds to nearest


def test_sumsq_blocks_closed_forms():
    assert sumsq_blocks(np.ones(10000, np.float32)).tolist() == [4096.0, 4096.0, 1808.0]
    assert sumsq_blocks(np.zeros(5, np.float32)).tolist() == [0.0]
    x = np.arange(1, 4097, dtype=np.float32)
    n = 4096
    assert sumsq_blocks(x)[0] == n * (n + 1) * (2 * n + 1) / 6
    assert np.isinf(sumsq_blocks(np.array([1.0, np.inf], np.float32))[0])
    assert np.isnan(sumsq_blocks(np.array([1.0, np.nan], np.float32))[0])
