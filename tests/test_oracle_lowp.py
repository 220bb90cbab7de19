"""Pins of the oracle's 16-bit rounding and of the wrapped hook (fp16_compress_wrapper /
bf16_compress_wrapper around powerSGD_hook): hand-worked ties, torch's own conversion
of binary32 values, nearest-value brute force, exact cases where 16-bit storage loses
nothing, and error bounds against the fp64 hook."""
import numpy as np
import pytest
import torch

import oracle
from oracle.lowp import compress_matrix_step_lowp, round_bf16, round_f16

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
RND = {"f16": round_f16, "bf16": round_bf16}


def test_round_f16_hand_worked():
    cases = [
        (1 + 2 ** -11, 1.0),                     # tie -> even
        (1 + 3 * 2 ** -11, 1 + 2 ** -9),         # tie -> even (mantissa 2)
        (1 + 2 ** -11 + 2 ** -40, 1 + 2 ** -10),  # above the tie: one rounding, not two
        (65504.0, 65504.0), (65519.99, 65504.0), (65520.0, np.inf), (-7e4, -np.inf),
        (2.0 ** -25, 0.0),                       # half the smallest subnormal: tie -> 0
        (1.5 * 2 ** -24, 2.0 ** -23),            # tie between subnormals -> even
        (-0.0, -0.0),
    ]
    got = round_f16([c[0] for c in cases])
    np.testing.assert_array_equal(got, [c[1] for c in cases])
    assert np.signbit(round_f16([-0.0]))[0]
    assert np.isnan(round_f16([np.nan]))[0]


def test_round_bf16_hand_worked():
    cases = [
        (1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -7),
        (-(1 + 2 ** -8 + 2 ** -40), -(1 + 2 ** -7)),
        (float.fromhex("0x1.fep127"), float.fromhex("0x1.fep127")),
        (float.fromhex("0x1.fefffffp127"), float.fromhex("0x1.fep127")),
        (float.fromhex("0x1.ffp127"), np.inf),
        (2.0 ** -126, 2.0 ** -126), (2.0 ** -134, 0.0), (1.5 * 2 ** -133, 2.0 ** -132),
        (3 * 2 ** -134, 2.0 ** -132),           # 1.5 subnormal steps: tie -> even
        (100.0, 100.0), (257.0, 256.0), (259.0, 260.0),
    ]
    got = round_bf16([c[0] for c in cases])
    np.testing.assert_array_equal(got, [c[1] for c in cases])
    assert np.isnan(round_bf16([np.nan]))[0]
    np.testing.assert_array_equal(round_bf16([np.inf, -np.inf]), [np.inf, -np.inf])


def test_round_bf16_matches_torch_on_binary32_values():
    g = torch.Generator().manual_seed(0)
    bits = torch.randint(-2 ** 31, 2 ** 31, (200000,), generator=g, dtype=torch.int64)
    x32 = bits.to(torch.int32).view(torch.float32)
    x32 = x32[torch.isfinite(x32)]
    want = x32.to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x32.to(torch.float64).numpy())
    np.testing.assert_array_equal(got, want)


def _neighbours(r, dt):
    """The 16-bit values adjacent to the (finite, nonzero) 16-bit values r, from their
    bit patterns."""
    if dt == "f16":
        b = r.astype(np.float16).view(np.uint16).astype(np.int32)
        mk = lambda x: x.astype(np.uint16).view(np.float16).astype(np.float64)
    else:
        b = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        mk = lambda x: (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return mk(b - 1), mk(b + 1)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_rounding_is_nearest_with_ties_to_even(dt):
    rnd = RND[dt]
    rng = np.random.default_rng(1)
    lo, hi = (-13, 14) if dt == "f16" else (-100, 100)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(lo, hi, 20000))
    x = x[np.abs(x) > (2.0 ** -13 if dt == "f16" else 2.0 ** -110)]
    x = x[np.abs(x) < (6e4 if dt == "f16" else 1e30)]
    r = rnd(x)
    assert np.all(rnd(r) == r)                       # results are 16-bit values
    # the adjacent 16-bit values (same sign) are no closer; on a tie r is even
    for nb in _neighbours(np.abs(r), dt):
        d_r, d_nb = np.abs(np.abs(x) - np.abs(r)), np.abs(np.abs(x) - nb)
        assert np.all(d_r <= d_nb)
        tie = d_r == d_nb
        if np.any(tie):
            bits = (np.abs(r[tie]).astype(np.float16).view(np.uint16) if dt == "f16"
                    else np.abs(r[tie]).astype(np.float32).view(np.uint32) >> 16)
            assert np.all(bits % 2 == 0)
    # exact ties built on purpose: midpoints of adjacent values round to the even one
    a = rnd(np.abs(x[:2000]))
    lo_nb, hi_nb = _neighbours(a, dt)
    mid = (a + hi_nb) / 2
    got = rnd(mid)
    ab = (a.astype(np.float16).view(np.uint16) if dt == "f16"
          else a.astype(np.float32).view(np.uint32) >> 16)
    np.testing.assert_array_equal(got, np.where(ab % 2 == 0, a, hi_nb))


def _rank1_row(n, m, row, vals):
    g = np.zeros((n, m))
    g[row] = vals
    return g


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_single_nonzero_row_is_recovered_exactly(dt):
    """M = e_i v^T with small integers: P = +-e_i, Q = +-v, M_hat = M and E = 0 with
    no rounding anywhere, whatever the starting Q."""
    rnd = RND[dt]
    v = np.array([3.0, -7.0, 1.0, 0.0, 12.0, -2.0])
    g = _rank1_row(5, 6, 2, v)
    q0 = rnd(np.array([[0.3], [-1.2], [0.7], [0.1], [0.5], [-0.9]]))
    q0 = rnd(q0 / np.linalg.norm(q0))
    mp, p, q, mh, e = compress_matrix_step_lowp(g, None, q0, 0.0, True, rnd)
    np.testing.assert_array_equal(mh, g)
    np.testing.assert_array_equal(e, np.zeros_like(g))
    assert abs(p[2, 0]) == 1.0 and np.count_nonzero(p) == 1
    np.testing.assert_array_equal(np.abs(q[:, 0]), np.abs(v))


def _low_rank(n, m, k, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((n, k))
    w = rng.standard_normal((m, k))
    return (u * (1.0 / np.arange(1, k + 1))) @ w.T + 0.01 * rng.standard_normal((n, m))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_every_materialized_tensor_is_16_bit_and_feedback_holds(dt):
    rnd, u = RND[dt], U[dt]
    g = rnd(_low_rank(40, 30, 6, 2))
    e = rnd(0.1 * _low_rank(40, 30, 3, 3))
    q0 = rnd(oracle.gram_schmidt(rnd(np.random.default_rng(4).standard_normal((30, 4))), 0.0))
    mp, p, q, mh, err = compress_matrix_step_lowp(g, e, q0, 0.0, True, rnd)
    for name, a in (("M'", mp), ("P", p), ("Q", q), ("M_hat", mh), ("E", err)):
        assert np.all(rnd(a) == a), name
    np.testing.assert_array_equal(mp, rnd(g + e))
    # E = rnd(M' - M_hat): M_hat + E = M' up to one rounding of E
    assert np.all(np.abs(mp - (mh + err)) <= u * np.abs(err) + 1e-300)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_wrapped_hook_is_the_fp64_hook_within_the_16_bit_bound(dt):
    """The 16-bit hook against the fp64 hook on the same gradients: the outputs
    differ by a few units of 16-bit rounding, relative to the output."""
    u = U[dt]
    views = [(0, (48, 3, 2, 2)), (576, (16,)), (592, (4, 4)), (608, (40, 33))]
    hp = oracle.HParams(matrix_approximation_rank=3, start_powerSGD_iter=0)
    a, b = oracle.OracleState(hp), oracle.OracleState(hp)
    for t in range(4):
        x = np.zeros(608 + 40 * 33, dtype=np.float32)
        x[0:576] = _low_rank(48, 12, 8, 10 + t).reshape(-1)
        x[576:592] = np.random.default_rng(t).standard_normal(16)
        x[592:608] = np.arange(16) * 0.37
        x[608:] = _low_rank(40, 33, 8, 20 + t).reshape(-1)
        ra = a.compress_bucket(x, views)
        rb = b.compress_bucket_wrapped(x, views, dt)
        for vi, (off, shp) in enumerate(views):
            size = int(np.prod(shp))
            o64 = ra.output64[off:off + size]
            o16 = rb.output64[off:off + size]
            if not ra.views[vi].compressed:
                # the wrapper's cast only: bit-identical to numpy's / torch's casts
                want = (x[off:off + size].astype(np.float16).astype(np.float32) if dt == "f16"
                        else torch.from_numpy(x[off:off + size]).to(torch.bfloat16)
                        .to(torch.float32).numpy())
                np.testing.assert_array_equal(rb.output[off:off + size], want)
                continue
            rel = np.linalg.norm(o16 - o64) / np.linalg.norm(o64)
            assert rel < 16 * u, (t, vi, rel)  # measured <= 9.1u; no error feedback >= 127u


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_wrapped_pass_through_and_layout(dt):
    hp = oracle.HParams(matrix_approximation_rank=1, start_powerSGD_iter=2)
    st = oracle.OracleState(hp)
    views = [(0, (8, 8)), (64, (5,))]
    x = (np.arange(69, dtype=np.float32) * 0.1234567).astype(np.float32)
    r = st.compress_bucket_wrapped(x, views, dt)
    assert r.passthrough
    want = RND[dt](x.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(r.output, want)
    st.compress_bucket_wrapped(x, views, dt)
    st.compress_bucket_wrapped(x, views, dt)           # compresses: memorizes the layout
    with pytest.raises(oracle.LayoutChanged):
        st.compress_bucket(x, views)                    # the fp32 hook on the same index
    other = "bf16" if dt == "f16" else "f16"
    with pytest.raises(oracle.LayoutChanged):
        st.compress_bucket_wrapped(x, views, other)


# ------------------------------------------ the wrappers around batched_powerSGD_hook

@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_batched_wrapped_single_nonzero_row_is_exact(dt):
    """A 16-element bucket is one 4 x 4 matrix; a single nonzero row of small integers
    is recovered exactly at rank 1 (no rounding anywhere) and E is zero."""
    hp = oracle.HParams(matrix_approximation_rank=1, start_powerSGD_iter=0)
    st = oracle.OracleState(hp)
    x = np.zeros(16, dtype=np.float32)
    x[8:12] = [3.0, -7.0, 12.0, 1.0]
    for _ in range(2):
        r = st.compress_bucket_batched_wrapped(x, dt)
        np.testing.assert_array_equal(r.output, x)
        np.testing.assert_array_equal(r.views[0].error, np.zeros((4, 4)))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_batched_wrapped_padding_truncation_and_feedback(dt):
    rnd, u = RND[dt], U[dt]
    hp = oracle.HParams(matrix_approximation_rank=2, start_powerSGD_iter=0)
    st = oracle.OracleState(hp)
    rng = np.random.default_rng(5)
    numel, s = 90, 10
    e_prev = None
    for t in range(3):
        x = rng.standard_normal(numel).astype(np.float32)
        r = st.compress_bucket_batched_wrapped(x, dt)
        vr = r.views[0]
        assert r.output.shape == (numel,) and (vr.n, vr.m, vr.rank) == (s, s, 2)
        g = np.zeros(s * s)
        g[:numel] = rnd(x.astype(np.float64))
        want_mp = rnd(g + e_prev.reshape(-1)) if e_prev is not None else g
        np.testing.assert_array_equal(vr.m_prime.reshape(-1), want_mp)   # padding: G is 0
        for a in (vr.p, vr.q, vr.m_hat, vr.error):
            assert np.all(rnd(a) == a)
        assert np.all(np.abs(vr.m_prime - (vr.m_hat + vr.error)) <= u * np.abs(vr.error) + 1e-300)
        np.testing.assert_array_equal(r.output, vr.m_hat.reshape(-1)[:numel].astype(np.float32))
        e_prev = vr.error
    assert (st.numel_in, st.numel_comm) == (3 * numel, 3 * 2 * s * 2)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_batched_wrapped_is_the_fp64_batched_hook_within_the_16_bit_bound(dt):
    u = U[dt]
    hp = oracle.HParams(matrix_approximation_rank=2, start_powerSGD_iter=0)
    a, b = oracle.OracleState(hp), oracle.OracleState(hp)
    for t in range(4):
        x = _low_rank(30, 30, 8, 40 + t).reshape(-1)[:880].astype(np.float32)
        ra = a.compress_bucket_batched(x)
        rb = b.compress_bucket_batched_wrapped(x, dt)
        rel = np.linalg.norm(rb.output64 - ra.output64) / np.linalg.norm(ra.output64)
        assert rel < 16 * u, (t, rel)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_batched_wrapped_pass_through_and_layout(dt):
    hp = oracle.HParams(matrix_approximation_rank=1, start_powerSGD_iter=1)
    st = oracle.OracleState(hp)
    x = (np.arange(20, dtype=np.float32) * 0.1234567).astype(np.float32)
    r = st.compress_bucket_batched_wrapped(x, dt, bucket_index=2)
    assert r.passthrough
    np.testing.assert_array_equal(r.output, RND[dt](x.astype(np.float64)).astype(np.float32))
    st.compress_bucket_batched_wrapped(x, dt, bucket_index=2)
    assert st.buckets[2].layout == ("batched", 20, dt)
    with pytest.raises(oracle.LayoutChanged):
        st.compress_bucket_batched(x, bucket_index=2)
    with pytest.raises(oracle.LayoutChanged):
        st.compress_bucket_wrapped(x, [(0, (4, 5))], dt, bucket_index=2)
