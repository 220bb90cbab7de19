"""Pins of the oracle's batched variant (batched_powerSGD_hook, "DDP Communication
Hooks -- PyTorch 1.11.0", section "PowerSGD Hooks"): a hand-worked example, closed
forms and identities that hold whatever the rounding."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.powersgd import _BucketMemory

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hp(**kw):
    base = dict(matrix_approximation_rank=1, start_powerSGD_iter=0, min_compression_rate=2.0,
                use_error_feedback=True, warm_start=True, orthogonalization_epsilon=0.0,
                random_seed=0)
    base.update(kw)
    return oracle.HParams(**base)


def test_batched_side_is_the_smallest_square_that_holds_the_bucket():
    assert oracle.batched_side(0) == 0
    for n in range(1, 20001):
        s = oracle.batched_side(n)
        assert s * s >= n and (s - 1) * (s - 1) < n, n
    for s in (4315, 46341, 3037000499):
        assert oracle.batched_side(s * s) == s
        assert oracle.batched_side(s * s + 1) == s + 1


def test_hand_worked_two_steps_with_padding_in_the_error_memory():
    doc = json.load(open(os.path.join(GOLDEN, "batched_worked.json")))
    st = oracle.OracleState(_hp(matrix_approximation_rank=doc["rank"]))
    mem = _BucketMemory(layout=("batched", doc["numel"]))
    mem.q[0] = np.array(doc["q_start"], dtype=np.float64)
    st.buckets[0] = mem
    for step in doc["steps"]:
        res = st.compress_bucket_batched(np.array(step["gradient"], dtype=np.float32))
        np.testing.assert_allclose(res.output64, step["output"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(res.views[0].error.reshape(-1), step["error"], rtol=0,
                                   atol=1e-12)
        np.testing.assert_allclose(mem.q[0], step["q"], rtol=0, atol=1e-12)


def test_rank_one_square_bucket_is_recovered_exactly():
    rng = np.random.default_rng(3)
    s = 37
    # small integer factors: the float32 bucket is exactly rank one
    u = rng.integers(-8, 9, s).astype(np.float64)
    v = rng.integers(-8, 9, s).astype(np.float64)
    u[0] = v[0] = 1.0
    g = np.outer(u, v).reshape(-1)
    st = oracle.OracleState(_hp())
    res = st.compress_bucket_batched(g.astype(np.float32))
    np.testing.assert_allclose(res.output64, g, rtol=0, atol=1e-12 * np.abs(g).max())


def test_rank_at_least_the_side_is_lossless():
    rng = np.random.default_rng(4)
    g = rng.standard_normal(7).astype(np.float32)  # s = 3, padding of 2
    st = oracle.OracleState(_hp(matrix_approximation_rank=8))  # rank = min(8, 3) = 3
    res = st.compress_bucket_batched(g)
    assert res.views[0].rank == 3
    np.testing.assert_allclose(res.output64, g.astype(np.float64), rtol=0, atol=1e-12)
    np.testing.assert_allclose(res.views[0].error, 0.0, atol=1e-12)


def test_error_feedback_identity_covers_the_padding():
    rng = np.random.default_rng(5)
    numel = 50  # s = 8, 14 padded entries
    st = oracle.OracleState(_hp(matrix_approximation_rank=2))
    e_prev = np.zeros(64)
    for step in range(4):
        g = rng.standard_normal(numel).astype(np.float32)
        res = st.compress_bucket_batched(g)
        vr = res.views[0]
        padded = np.zeros(64)
        padded[:numel] = g
        # M_hat + E_new = pad(G) + E_prev entry by entry, padding included
        np.testing.assert_allclose(vr.m_hat.reshape(-1) + vr.error.reshape(-1), padded + e_prev,
                                   rtol=0, atol=1e-12)
        np.testing.assert_array_equal(res.output64, vr.m_hat.reshape(-1)[:numel])
        e_prev = vr.error.reshape(-1)
        if step > 0:
            assert np.abs(e_prev[numel:]).max() > 0  # the padding carries error


def test_square_bucket_matches_a_single_view_of_the_per_layer_hook():
    rng = np.random.default_rng(6)
    s = 16
    a = oracle.OracleState(_hp(matrix_approximation_rank=2, min_compression_rate=0.0))
    b = oracle.OracleState(_hp(matrix_approximation_rank=2, min_compression_rate=0.0))
    for _ in range(3):
        g = rng.standard_normal(s * s).astype(np.float32)
        ra = a.compress_bucket_batched(g, bucket_index=5)
        rb = b.compress_bucket(g, [(0, (s, s))], bucket_index=5)
        np.testing.assert_array_equal(ra.output64, rb.output64)
    assert (a.numel_in, a.numel_comm) == (b.numel_in, b.numel_comm) == (3 * s * s, 3 * 2 * s * 2)


def test_fp16_skip_unscale_and_passthrough():
    g = (np.arange(10, dtype=np.float32) - 4.5).astype(np.float16)
    st = oracle.OracleState(_hp(start_powerSGD_iter=1))
    res = st.compress_bucket_batched(g, inv_loss_scale=0.5)  # iteration 0 < 1: unscale only
    assert res.passthrough and st.iteration == 1 and not st.buckets
    np.testing.assert_array_equal(res.output, (g.astype(np.float64) * 0.5).astype(np.float16))
    bad = g.copy()
    bad[3] = np.inf
    res = st.compress_bucket_batched(bad, inv_loss_scale=0.5)
    assert res.skipped and st.iteration == 2 and not st.buckets
    np.testing.assert_array_equal(res.output, bad)
    res = st.compress_bucket_batched(g, inv_loss_scale=0.5)
    assert not res.skipped and res.output.dtype == np.float16
    np.testing.assert_array_equal(res.output, res.output64.astype(np.float16))


def test_layout_memory_is_shared_with_the_per_layer_hook():
    st = oracle.OracleState(_hp())
    g = np.ones(16, dtype=np.float32)
    st.compress_bucket(g, [(0, (4, 4))], bucket_index=0)
    with pytest.raises(oracle.LayoutChanged):
        st.compress_bucket_batched(g, bucket_index=0)
    st.compress_bucket_batched(g, bucket_index=1)
    with pytest.raises(oracle.LayoutChanged):
        st.compress_bucket_batched(np.ones(15, dtype=np.float32), bucket_index=1)
