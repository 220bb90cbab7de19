"""Pins for the oracle's bucket-level behaviour: classification, pass-through,
statistics, iteration counting, layout memory and the fp16 / AMP path."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import HParams, LayoutChanged, OracleState
from synthetic import CONFIGS, BucketGenerator, packed_views, shrink_config

SHAPES = [(12, 20), (30,), (8, 3, 3), (5,), (4, 4), (40, 10)]


def _bucket(seed=0, dtype=np.float32, shapes=SHAPES):
    rng = np.random.default_rng(seed)
    n = sum(int(np.prod(s)) for s in shapes)
    return rng.standard_normal(n).astype(dtype)


def _hp(**kw):
    base = dict(matrix_approximation_rank=2, start_powerSGD_iter=0)
    base.update(kw)
    return HParams(**base)


def test_classification_and_passthrough_of_uncompressed_views():
    st = OracleState(_hp())
    views = packed_views(SHAPES)
    b = _bucket()
    res = st.compress_bucket(b, views)
    flags = [v.compressed for v in res.views]
    # (12,20): 32*2*2=128 < 240; (8,3,3) is 8x9: 17*2*2=68 < 72; (4,4): 8*2*2=32 not < 16;
    # (40,10): 50*2*2=200 < 400; vectors never.
    assert flags == [True, False, True, False, False, True]
    for (off, shp), vr in zip(views, res.views):
        size = int(np.prod(shp))
        if not vr.compressed:
            # uncompressed views leave the bucket bit-identical
            assert np.array_equal(res.output[off:off + size].view(np.uint32),
                                  b[off:off + size].view(np.uint32))
        else:
            assert np.array_equal(res.output[off:off + size],
                                  vr.m_hat.reshape(-1).astype(np.float32))


def test_statistics_closed_form():
    st = OracleState(_hp())
    views = packed_views(SHAPES)
    st.compress_bucket(_bucket(), views)
    numel = sum(int(np.prod(s)) for s in SHAPES)
    comm = (12 + 20) * 2 + 30 + (8 + 9) * 2 + 5 + 16 + (40 + 10) * 2
    assert (st.numel_in, st.numel_comm) == (numel, comm)
    st.compress_bucket(_bucket(1), views, is_last=False)
    assert (st.numel_in, st.numel_comm) == (2 * numel, 2 * comm)


def test_iteration_advances_only_on_last_bucket():
    st = OracleState(_hp())
    views = packed_views(SHAPES)
    st.compress_bucket(_bucket(), views, bucket_index=0, is_last=False)
    assert st.iteration == 0
    st.compress_bucket(_bucket(), views, bucket_index=1, is_last=True)
    assert st.iteration == 1


def test_start_iter_is_vanilla_allreduce():
    st = OracleState(_hp(start_powerSGD_iter=2))
    views = packed_views(SHAPES)
    for it in range(2):
        b = _bucket(it)
        res = st.compress_bucket(b, views)
        assert res.passthrough
        assert np.array_equal(res.output.view(np.uint32), b.view(np.uint32))
        assert not st.buckets                    # no state before compression starts
    res = st.compress_bucket(_bucket(2), views)
    assert not res.passthrough and any(v.compressed for v in res.views)


def test_error_feedback_identity_over_steps():
    # M_hat_t + E_t = G_t + E_{t-1} for every compressed view and step
    st = OracleState(_hp())
    views = packed_views(SHAPES)
    prev = {}
    for step in range(4):
        b = _bucket(step)
        res = st.compress_bucket(b, views)
        for vi, ((off, shp), vr) in enumerate(zip(views, res.views)):
            if not vr.compressed:
                continue
            g = b[off:off + int(np.prod(shp))].astype(np.float64).reshape(vr.n, vr.m)
            lhs = vr.m_hat + vr.error
            rhs = g + prev.get(vi, 0.0)
            assert np.abs(lhs - rhs).max() < 1e-12
            prev[vi] = vr.error


def test_warm_start_memorizes_q_and_draw_happens_once():
    views = packed_views(SHAPES)
    st = OracleState(_hp(use_error_feedback=False))
    b = _bucket(0)
    r1 = st.compress_bucket(b, views)
    r2 = st.compress_bucket(b, views)
    # second call starts from the first call's Q: one more power-iteration step
    v1, v2 = r1.views[0], r2.views[0]
    p_expected = v1.m_prime @ v1.q
    # GS(M Q1) spans the same space as P2
    proj = v2.p @ (v2.p.T @ p_expected)
    assert np.abs(proj - p_expected).max() < 1e-10 * np.abs(p_expected).max()


def test_without_warm_start_a_fresh_q_each_iteration():
    views = packed_views(SHAPES)
    b = _bucket(0)
    st = OracleState(_hp(use_error_feedback=False, warm_start=False))
    a = st.compress_bucket(b, views).views[0].p
    c = st.compress_bucket(b, views).views[0].p
    assert not np.allclose(a, c)
    # and the same seed reproduces the same draws
    st2 = OracleState(_hp(use_error_feedback=False, warm_start=False))
    assert np.array_equal(st2.compress_bucket(b, views).views[0].p, a)


def test_layout_change_of_memorized_bucket_is_an_error():
    st = OracleState(_hp())
    st.compress_bucket(_bucket(), packed_views(SHAPES))
    other = [(20, 12)] + SHAPES[1:]
    with pytest.raises(LayoutChanged):
        st.compress_bucket(_bucket(shapes=other), packed_views(other))
    # without memory (no error feedback, no warm start) a new layout is accepted
    st2 = OracleState(_hp(use_error_feedback=False, warm_start=False))
    st2.compress_bucket(_bucket(), packed_views(SHAPES))
    st2.compress_bucket(_bucket(shapes=other), packed_views(other))


def test_batching_flag_does_not_change_results():
    views = packed_views(SHAPES)
    a = OracleState(_hp(batch_tensors_with_same_shape=False))
    b = OracleState(_hp(batch_tensors_with_same_shape=True))
    for step in range(3):
        ra = a.compress_bucket(_bucket(step), views)
        rb = b.compress_bucket(_bucket(step), views)
        assert np.array_equal(ra.output64, rb.output64)


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_fp16_inf_or_nan_skips_everything(bad):
    views = packed_views(SHAPES)
    st = OracleState(_hp())
    b16 = (_bucket(0) * 100).astype(np.float16)
    st.compress_bucket(b16, views, inv_loss_scale=2.0 ** -16)
    mem_e = {k: v.copy() for k, v in st.buckets[0].error.items()}
    mem_q = {k: v.copy() for k, v in st.buckets[0].q.items()}
    it = st.iteration
    b2 = (_bucket(1) * 100).astype(np.float16)
    b2[37] = bad                               # inside the vector view (30,)
    res = st.compress_bucket(b2, views, inv_loss_scale=2.0 ** -16)
    assert res.found_inf and res.skipped
    assert np.array_equal(res.output.view(np.uint16), b2.view(np.uint16))
    for k in mem_e:
        assert np.array_equal(st.buckets[0].error[k], mem_e[k])
        assert np.array_equal(st.buckets[0].q[k], mem_q[k])
    assert st.iteration == it + 1              # the iteration still advances


def test_fp16_unscale_is_exact_and_output_is_rounded_fp16():
    views = packed_views(SHAPES)
    st = OracleState(_hp())
    b16 = (_bucket(2) * 3000).astype(np.float16)
    scale = 2.0 ** 16
    res = st.compress_bucket(b16, views, inv_loss_scale=1.0 / scale)
    assert not res.found_inf
    for (off, shp), vr in zip(views, res.views):
        size = int(np.prod(shp))
        out = res.output[off:off + size]
        if not vr.compressed:
            # output = x / 2^16 rounded once to fp16; when that quotient is a normal
            # fp16 number with spare exponent range it is exact
            for x, y in zip(b16[off:off + size], out):
                exact = Fraction(float(x)) / Fraction(int(scale))
                if abs(exact) >= Fraction(2) ** -14:
                    assert Fraction(float(y)) == exact
        else:
            # compressed output: within half an fp16 ulp of the fp64 M_hat
            mh = vr.m_hat.reshape(-1)
            ulp = np.spacing(np.abs(mh).astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(out.astype(np.float64) - mh) <= 0.5 * ulp + 1e-300)
            # and M' is the unscaled fp16 input (plus E = 0 on the first step)
            g = b16[off:off + size].astype(np.float64) / scale
            assert np.array_equal(vr.m_prime.reshape(-1), g)


def test_config_generator_is_deterministic_and_matches_recipe():
    cfg = shrink_config(CONFIGS[1], [(64, 3, 7, 7), (96,), (40, 50)], steps=2)
    a = BucketGenerator(cfg).bucket(0)
    b = BucketGenerator(cfg).bucket(0)
    assert a.dtype == b.dtype and bool((a == b).all())
    c = BucketGenerator(cfg).bucket(1)
    assert not bool((a == c).all())
    # low rank persists across steps, noise does not: the difference of two steps
    # is pure noise with the recipe's standard deviation
    d = (a[:64 * 147] - c[:64 * 147]).double()
    assert abs(float(d.std()) - 0.01 * np.sqrt(2)) < 0.002
    f16 = shrink_config(CONFIGS[4], [(16, 32), (8,)], steps=1)
    g = BucketGenerator(f16)
    h = g.bucket(10)                           # a forced inf step
    assert bool(h.isinf().any())
    assert not bool(g.bucket(3, inject_inf=False).isinf().any())
