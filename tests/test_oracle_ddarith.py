"""Pins for the oracle's double-double Gram-Schmidt (oracle.ddarith and
oracle.gram_schmidt on ill-conditioned input).

Expected values come from exact rational arithmetic (fractions), from an independent
200-bit modified Gram-Schmidt (mpmath), and from what the method fixes for a matrix of
rank below r (M_hat = M', E = 0; "PowerSGD State", orthogonalization_epsilon)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ddarith as dd
from oracle import compress_matrix_step, gram_schmidt


def _doubles(rng, k):
    """Doubles of many magnitudes and both signs, plus values that stress the splits."""
    x = rng.standard_normal(k) * np.exp2(rng.integers(-60, 60, k).astype(np.float64))
    special = np.array([1.0, -1.0, 2.0 ** 52 + 1, 1.0 + 2.0 ** -52, 3.0, 1e-300, -7e290,
                        0.1, 1.0 / 3.0, 2.0 ** 27 + 1])
    return np.concatenate([x, special])


def test_two_sum_and_two_prod_are_exact():
    rng = np.random.default_rng(1)
    a = _doubles(rng, 2000)
    b = _doubles(rng, 2000)[::-1].copy()
    s, e = dd.two_sum(a, b)
    for ai, bi, si, ei in zip(a, b, s, e):
        assert Fraction(si) + Fraction(ei) == Fraction(ai) + Fraction(bi)
        assert si == ai + bi
    small = a / 2.0 ** 400 * (np.abs(a) < 1e250)  # products stay in range
    p, q = dd.two_prod(small, b)
    for ai, bi, pi, qi in zip(small, b, p, q):
        if not math.isfinite(pi) or abs(pi) < 1e-280:
            continue
        assert Fraction(pi) + Fraction(qi) == Fraction(ai) * Fraction(bi)


def test_dd_sum_and_dot_against_exact_rationals():
    rng = np.random.default_rng(2)
    for n in (1, 2, 3, 17, 1000, 4097):
        h = rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n).astype(np.float64))
        # heavy cancellation: append the negated values, shuffled, plus one small term
        h = np.concatenate([h, -h[rng.permutation(n)], [1e-20]])
        l = rng.standard_normal(h.size) * 1e-40
        exact = sum((Fraction(float(x)) for x in h), Fraction(0)) + \
            sum((Fraction(float(x)) for x in l), Fraction(0))
        sh, sl = dd.dd_sum(h, l)
        got = Fraction(sh) + Fraction(sl)
        scale = sum(abs(Fraction(float(x))) for x in h)
        assert abs(got - exact) <= Fraction(2) ** -100 * scale, n
    x = rng.standard_normal(500)
    y = rng.standard_normal(500)
    exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, y))
    ph, pl = dd.dd_dot(x, np.zeros_like(x), y, np.zeros_like(y))
    assert abs(Fraction(ph) + Fraction(pl) - exact) <= Fraction(2) ** -100 * 500


def test_inverse_norm_plus():
    h, l = dd.inverse_norm_plus(4.0, 0.0, 0.0)
    assert (h, l) == (0.5, 0.0)
    h, l = dd.inverse_norm_plus(2.0, 0.0, 0.0)
    # 1/sqrt(2) to about 106 bits
    assert abs((Fraction(h) + Fraction(l)) ** 2 * 2 - 1) < Fraction(2) ** -100
    assert dd.inverse_norm_plus(0.0, 0.0, 0.0)[0] == math.inf
    assert dd.inverse_norm_plus(0.0, 0.0, 0.5) == (2.0, 0.0)
    assert math.isnan(dd.inverse_norm_plus(math.nan, 0.0, 0.0)[0])


def _mp_mgs(x, eps, prec=200):
    """Modified Gram-Schmidt with epsilon in `prec`-bit arithmetic (mpmath)."""
    import mpmath
    with mpmath.workprec(prec):
        n, r = x.shape
        cols = [[mpmath.mpf(float(x[i, j])) for i in range(n)] for j in range(r)]
        e = mpmath.mpf(eps)
        for i in range(r):
            nrm = mpmath.sqrt(mpmath.fsum(v * v for v in cols[i]))
            inv = 1 / (nrm + e)
            cols[i] = [v * inv for v in cols[i]]
            for j in range(i + 1, r):
                c = mpmath.fsum(a * b for a, b in zip(cols[i], cols[j]))
                cols[j] = [b - c * a for a, b in zip(cols[i], cols[j])]
        return np.array([[float(cols[j][i]) for j in range(r)] for i in range(n)])


@pytest.mark.parametrize("eps", [0.0, 1e-8])
def test_gram_schmidt_on_a_condition_number_of_1e14(eps):
    """x = U diag(s) V^T with s from 1 down to 1e-14: binary64 modified Gram-Schmidt
    loses orthogonality in proportion to u * 1e14; the oracle's steps match a 200-bit
    run of the same steps and, with epsilon = 0, give orthonormal columns."""
    rng = np.random.default_rng(3)
    n, r = 60, 8
    u, _ = np.linalg.qr(rng.standard_normal((n, r)))
    v, _ = np.linalg.qr(rng.standard_normal((r, r)))
    s = np.logspace(0, -14, r)
    x = (u * s) @ v.T
    q = gram_schmidt(x, eps)
    ref = _mp_mgs(x, eps)
    assert np.abs(q - ref).max() <= 1e-12
    if eps == 0.0:
        assert np.abs(q.T @ q - np.eye(r)).max() <= 1e-12


def test_rank_deficient_trajectory_keeps_mhat_equal_to_mprime():
    """A rank-1 M (fp32 values) at r = 32 over four warm-started steps with error
    feedback: P has condition numbers beyond 1e12 after the first step, and the
    oracle's M_hat stays the projection of M', so E stays at the rounding level of the
    binary32 input (about 1e-8 of M') and P keeps orthonormal columns."""
    rng = np.random.default_rng(4)
    n, m, r = 120, 90, 32
    u = rng.standard_normal(n)
    v = rng.standard_normal(m)
    q = gram_schmidt(oracle.standard_normal_q0(m, r, 0, 0, 0, 0), 0.0)
    e = None
    for step in range(4):
        g = (np.outer(u, v) * (2.0 + step)).astype(np.float32).astype(np.float64)
        vr = compress_matrix_step(g, e, q, 0.0, True)
        e, q = vr.error, vr.q
        assert np.abs(vr.p.T @ vr.p - np.eye(r)).max() <= 1e-12, step
        assert np.linalg.norm(vr.error) <= 1e-6 * np.linalg.norm(vr.m_prime), step
