"""Pins for the oracle's decision rule, Gram-Schmidt and single compression step.

Every expected value here comes from the pages (golden files, hand-worked), from
exact rational arithmetic, from a textbook routine the oracle does not use
(Householder QR, SVD), or from a mathematical identity the method must satisfy.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (compress_matrix_step, effective_rank, gram_schmidt, matrix_view,
                    should_compress)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- decisions

def test_rate_decisions_hand_evaluated():
    for case in _golden("rate_decisions.json")["cases"]:
        nm = matrix_view(case["shape"])
        if nm is None:
            got = False
        else:
            n, m = nm
            got = should_compress(n, m, effective_rank(n, m, case["rank"]), case["rate"])
        assert got == case["compress"], case


def test_rate_decision_structure_brute_force():
    # The strict inequality is monotone in the rate and in the rank, symmetric in
    # (rows, cols), and a boundary case (equality) is never compressed.
    rates = [0.25, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]
    for n in range(1, 41):
        for m in range(1, 41):
            for r in (1, 2, 4, 32):
                rt = effective_rank(n, m, r)
                assert rt == min(r, n, m)
                prev = True
                for rate in rates:
                    d = should_compress(n, m, rt, rate)
                    assert d == should_compress(m, n, rt, rate)
                    assert not (d and not prev)     # once false, stays false
                    prev = d
                    lhs = Fraction(n + m) * rt * Fraction(rate)
                    if lhs == n * m:
                        assert not d


def test_rate_decision_uses_exact_rate_value():
    # 0.3 in binary64 is slightly below 3/10, so (2+3)*4*0.3 is exactly a little
    # under 6 and the 2 x 3 matrix passes the strict test; a binary64 product would
    # round to 6.0 and fail it. The reading is the exact comparison.
    assert Fraction(0.3) < Fraction(3, 10)
    assert (2 + 3) * 4 * 0.3 == 6.0
    assert should_compress(2, 3, 4, 0.3)
    # 0.1 is slightly above 1/10: 40 * 100 * 0.1 is a little over 400
    assert not should_compress(20, 20, 100, 0.1)


def test_every_workload_matrix_compresses_and_vectors_do_not():
    from synthetic import CONFIGS
    for cfg in CONFIGS.values():
        r = cfg.hparams["matrix_approximation_rank"]
        rate = cfg.hparams["min_compression_rate"]
        for _, shape in cfg.views():
            nm = matrix_view(shape)
            if len(shape) < 2:
                assert nm is None
            else:
                assert should_compress(nm[0], nm[1], effective_rank(*nm, r), rate), shape


# ---------------------------------------------------------------- Gram-Schmidt

def _householder_q(x):
    q, r = np.linalg.qr(x)          # LAPACK Householder QR
    s = np.sign(np.diag(r))
    return q * s


@pytest.mark.parametrize("n,r", [(5, 1), (7, 3), (64, 4), (300, 32), (33, 33)])
def test_gram_schmidt_is_the_unique_thin_qr(n, r):
    rng = np.random.default_rng(n * 100 + r)
    x = rng.standard_normal((n, r))
    q = gram_schmidt(x, 0.0)
    # orthonormal columns
    assert np.abs(q.T @ q - np.eye(r)).max() < 1e-12
    # R = Q^T X is upper triangular with a positive diagonal and Q R = X
    rr = q.T @ x
    assert np.abs(np.tril(rr, -1)).max() < 1e-12 * np.abs(x).max()
    assert np.all(np.diag(rr) > 0)
    assert np.abs(q @ rr - x).max() < 1e-12 * np.abs(x).max()
    # and it equals LAPACK's Householder QR with the diagonal of R made positive
    assert np.abs(q - _householder_q(x)).max() < 1e-10


def test_gram_schmidt_epsilon_on_orthogonal_columns():
    # For mutually orthogonal columns no projection is removed, so each column is
    # simply divided by (its norm + epsilon).
    x = np.array([[3.0, 0.0, 0.0], [4.0, 0.0, 0.0], [0.0, 2.0, 0.0], [0.0, 0.0, -1.0]])
    eps = 0.5
    q = gram_schmidt(x, eps)
    assert np.allclose(q[:, 0], x[:, 0] / 5.5, rtol=0, atol=1e-15)
    assert np.allclose(q[:, 1], x[:, 1] / 2.5, rtol=0, atol=1e-15)
    assert np.allclose(q[:, 2], x[:, 2] / 1.5, rtol=0, atol=1e-15)


def test_gram_schmidt_zero_column():
    x = np.zeros((6, 2))
    x[:, 1] = 1.0
    # epsilon > 0: the zero column stays zero and nothing becomes NaN
    q = gram_schmidt(x, 1e-8)
    assert np.all(q[:, 0] == 0.0)
    assert np.allclose(q[:, 1], 1.0 / (math.sqrt(6) + 1e-8))
    # epsilon = 0: IEEE 0/0 propagates into every later column
    with np.errstate(invalid="ignore"):
        q0 = gram_schmidt(x, 0.0)
    assert np.all(np.isnan(q0))


def test_gram_schmidt_order_matters():
    # the first output column is the first input column normalized
    x = np.array([[1.0, 1.0], [0.0, 1.0]])
    q = gram_schmidt(x, 0.0)
    assert np.allclose(q, [[1, 0], [0, 1]])
    q2 = gram_schmidt(x[:, ::-1], 0.0)
    assert np.allclose(q2[:, 0], np.array([1, 1]) / math.sqrt(2))


# ---------------------------------------------------------------- one step

def _frac_matrix(rows):
    return [[Fraction(v) for v in row] for row in rows]


def _fmat(a, b):
    return [[sum(a[i][k] * b[k][j] for k in range(len(b))) for j in range(len(b[0]))]
            for i in range(len(a))]


def _ftrans(a):
    return [list(col) for col in zip(*a)]


def _finv(a):
    n = len(a)
    aug = [list(row) + [Fraction(int(i == j)) for j in range(n)] for i, row in enumerate(a)]
    for c in range(n):
        piv = next(r for r in range(c, n) if aug[r][c] != 0)
        aug[c], aug[piv] = aug[piv], aug[c]
        pv = aug[c][c]
        aug[c] = [v / pv for v in aug[c]]
        for r in range(n):
            if r != c and aug[r][c] != 0:
                f = aug[r][c]
                aug[r] = [v - f * w for v, w in zip(aug[r], aug[c])]
    return [row[n:] for row in aug]


def _exact_projection(m, q):
    """M_hat = X (X^T X)^-1 X^T M with X = M Q, in exact rational arithmetic:
    the orthogonal projection of M's columns onto span(M Q)."""
    mf, qf = _frac_matrix(m), _frac_matrix(q)
    x = _fmat(mf, qf)
    xt = _ftrans(x)
    return _fmat(_fmat(_fmat(x, _finv(_fmat(xt, x))), xt), mf)


def _parse(v):
    return float(Fraction(v))


def test_worked_examples():
    for case in _golden("worked_steps.json")["cases"]:
        m = np.array(case["M"], dtype=np.float64)
        q = np.array(case["Q"], dtype=np.float64)
        vr = compress_matrix_step(m, None, q, case["epsilon"])
        if "P" in case:
            p_exp = np.vectorize(_parse)(np.array(case["P"]))
            q_exp = np.vectorize(_parse)(np.array(case["Q_new"]))
        else:
            scale = 1.0 / math.sqrt(5.0)
            p_exp = np.vectorize(_parse)(np.array(case["P_scaled"])) * scale
            q_exp = np.vectorize(_parse)(np.array(case["Q_new_scaled"])) * scale
        assert np.allclose(vr.p, p_exp, rtol=0, atol=1e-14), case["name"]
        assert np.allclose(vr.q, q_exp, rtol=0, atol=1e-14), case["name"]
        assert np.allclose(vr.m_hat, np.vectorize(_parse)(np.array(case["M_hat"])),
                           rtol=0, atol=1e-14), case["name"]
        assert np.allclose(vr.error, np.vectorize(_parse)(np.array(case["E"])),
                           rtol=0, atol=1e-14), case["name"]


@pytest.mark.parametrize("n,m,r,seed", [(4, 3, 1, 0), (5, 4, 2, 1), (6, 5, 3, 2),
                                        (3, 7, 2, 3), (6, 6, 4, 4)])
def test_step_is_projection_onto_span_of_mq(n, m, r, seed):
    rng = np.random.default_rng(seed)
    mm = rng.integers(-5, 6, size=(n, m))
    q = rng.integers(-3, 4, size=(m, r))
    exact = _exact_projection(mm.tolist(), q.tolist())
    vr = compress_matrix_step(mm.astype(np.float64), None, q.astype(np.float64), 0.0)
    exact_f = np.array([[float(v) for v in row] for row in exact])
    scale = np.abs(mm).max()
    assert np.abs(vr.m_hat - exact_f).max() < 1e-12 * scale
    assert np.abs(vr.error - (mm - exact_f)).max() < 1e-12 * scale


def _random_low_rank(rng, n, m, k, decay=1.0, noise=0.0):
    u = rng.standard_normal((n, k))
    v = rng.standard_normal((m, k))
    s = np.arange(1, k + 1, dtype=np.float64) ** -decay
    return (u * s) @ v.T + noise * rng.standard_normal((n, m))


@pytest.mark.parametrize("eps_zero", [True])
def test_step_invariants(eps_zero):
    rng = np.random.default_rng(11)
    for (n, m, r) in [(40, 30, 1), (64, 20, 4), (17, 90, 3), (128, 128, 8)]:
        g = _random_low_rank(rng, n, m, 12, noise=0.01)
        e_prev = 0.1 * rng.standard_normal((n, m))
        q = rng.standard_normal((m, r))
        vr = compress_matrix_step(g, e_prev, q, 0.0)
        scale = np.linalg.norm(vr.m_prime)
        # M' = G + E_prev
        assert np.array_equal(vr.m_prime, g + e_prev)
        # P has orthonormal columns
        assert np.abs(vr.p.T @ vr.p - np.eye(r)).max() < 1e-12
        # E is orthogonal to span(P)
        assert np.abs(vr.p.T @ vr.error).max() < 1e-12 * scale
        # Pythagoras: |M_hat|^2 + |E|^2 = |M'|^2
        lhs = np.linalg.norm(vr.m_hat) ** 2 + np.linalg.norm(vr.error) ** 2
        assert lhs == pytest.approx(scale ** 2, rel=1e-12)
        # M_hat + E_new = G + E_prev
        assert np.abs(vr.m_hat + vr.error - (g + e_prev)).max() < 1e-12 * np.abs(g).max()
        # M_hat = P P^T M'
        assert np.abs(vr.m_hat - vr.p @ (vr.p.T @ vr.m_prime)).max() < 1e-11 * scale


def test_rank1_exact_recovery():
    rng = np.random.default_rng(3)
    for n, m in [(256, 512), (7, 3), (1000, 20)]:
        mm = np.outer(rng.standard_normal(n), rng.standard_normal(m))
        q = rng.standard_normal((m, 1))
        vr = compress_matrix_step(mm, None, q, 0.0)
        assert np.linalg.norm(vr.m_hat - mm) / np.linalg.norm(mm) < 1e-14
        assert np.linalg.norm(vr.error) / np.linalg.norm(mm) < 1e-14


def test_warm_start_power_iteration_reaches_truncated_svd():
    # Fixed M, no error feedback, Q carried from step to step: M_hat converges to
    # the best rank-r approximation (Eckart-Young), computed here by LAPACK's SVD.
    rng = np.random.default_rng(8)
    n, m, r = 60, 45, 3
    u, _ = np.linalg.qr(rng.standard_normal((n, n)))
    v, _ = np.linalg.qr(rng.standard_normal((m, m)))
    s = np.array([10.0, 8.0, 6.0, 3.0, 2.5, 2.0] + [1.0 / k for k in range(1, m - 5)])
    mm = (u[:, :m] * s) @ v.T
    q = rng.standard_normal((m, r))
    for _ in range(80):
        vr = compress_matrix_step(mm, None, q, 0.0, use_error_feedback=False)
        q = vr.q
    uu, ss, vt = np.linalg.svd(mm)
    best = (uu[:, :r] * ss[:r]) @ vt[:r]
    assert np.linalg.norm(vr.m_hat - best) / np.linalg.norm(best) < 1e-10


def test_q_right_multiplied_by_triangular_gives_same_step():
    # GS(M' Q R) = GS(M' Q) for upper-triangular R with positive diagonal, so the
    # orthogonalized draw and the raw draw give the same P, Q and M_hat.
    rng = np.random.default_rng(4)
    g = _random_low_rank(rng, 50, 40, 10, noise=0.01)
    q = rng.standard_normal((40, 4))
    tri = np.triu(rng.standard_normal((4, 4)))
    np.fill_diagonal(tri, np.abs(np.diag(tri)) + 0.5)
    a = compress_matrix_step(g, None, q, 0.0)
    b = compress_matrix_step(g, None, q @ tri, 0.0)
    c = compress_matrix_step(g, None, gram_schmidt(q, 0.0), 0.0)
    for other in (b, c):
        assert np.abs(a.p - other.p).max() < 1e-10
        assert np.abs(a.q - other.q).max() < 1e-9 * np.abs(a.q).max()
        assert np.abs(a.m_hat - other.m_hat).max() < 1e-9 * np.abs(a.m_hat).max()


def test_without_error_feedback_no_error_is_kept():
    rng = np.random.default_rng(2)
    g = rng.standard_normal((9, 8))
    vr = compress_matrix_step(g, rng.standard_normal((9, 8)), rng.standard_normal((8, 2)),
                              0.0, use_error_feedback=False)
    assert vr.error is None
    assert np.array_equal(vr.m_prime, g)
