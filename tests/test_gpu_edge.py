"""GPU edge cases against the oracle: degenerate matrices, hyperparameter corners,
control flow (pass-through, layout memory, several buckets), alignment, statistics
and error paths."""
import numpy as np
import pytest
import torch

import oracle
from parity import BucketParity, log, numel, rel_fro
from rank_gradient_compression_amd import PowerSGDError, PowerSGDState
from rank_gradient_compression_amd import powersgd as api
from synthetic import CONFIGS, BucketGenerator, packed_views, shrink_config

pytestmark = pytest.mark.gpu


def _hp(**kw):
    base = dict(matrix_approximation_rank=2, start_powerSGD_iter=0, min_compression_rate=2.0,
                use_error_feedback=True, warm_start=True, orthogonalization_epsilon=0.0,
                random_seed=0, compression_stats_logging_frequency=0)
    base.update(kw)
    return base


def _rand_bucket(shapes, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    n = sum(numel(s) for s in shapes)
    return torch.randn(n, generator=g) * scale


def _run_parity(hp, shapes, steps=3, seed=0, dtype="f32", inv_scale=1.0, bucket_fn=None):
    views = packed_views(shapes)
    par = BucketParity(hp, views, dtype)
    for step in range(steps):
        b = bucket_fn(step) if bucket_fn else _rand_bucket(shapes, seed + step)
        if dtype == "f16":
            b = b.to(torch.float16)
        rep = par.step(b, step, inv_loss_scale=inv_scale)
        log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items()))
    return par


def test_zero_matrix_epsilon_zero_propagates_nan_like_the_oracle():
    log("case: all-zero matrix, eps = 0 -> NaN everywhere (IEEE 0/0)")
    shapes = [(64, 48), (32,)]
    views = packed_views(shapes)
    b = _rand_bucket(shapes, 1)
    b[:64 * 48] = 0.0
    st = PowerSGDState(**_hp())
    d = b.cuda()
    st.compress_bucket(d, views)
    orc = oracle.OracleState(oracle.HParams(**_hp()))
    with np.errstate(invalid="ignore", divide="ignore"):
        res = orc.compress_bucket(b.numpy(), views)
    torch.cuda.synchronize()
    vr = res.views[0]
    p, q = st.factors(0, 0)
    for got, exp in ((p, vr.p), (q, vr.q), (d[:64 * 48].reshape(64, 48), vr.m_hat),
                     (st.error(0, 0), vr.error)):
        assert np.array_equal(np.isnan(got.cpu().numpy()), np.isnan(exp))
        assert np.isnan(exp).all()
    # the vector view is untouched
    assert torch.equal(d[64 * 48:].cpu(), b[64 * 48:])


def test_zero_matrix_with_epsilon_gives_zeros():
    log("case: all-zero matrix, eps = 1e-8 -> zeros")
    shapes = [(64, 48), (40, 300)]

    def fn(step):
        b = _rand_bucket(shapes, 2 + step)
        b[:64 * 48] = 0.0
        return b
    _run_parity(_hp(orthogonalization_epsilon=1e-8), shapes, steps=2, bucket_fn=fn)


def test_rank_one_matrix_is_recovered_exactly_at_rank_one():
    log("case: rank-1 M at r = 1 -> M_hat = M, E = 0")
    n, m = 300, 170
    g = torch.Generator().manual_seed(5)
    u = torch.randn(n, 1, generator=g)
    v = torch.randn(1, m, generator=g)
    b = (u @ v).reshape(-1).contiguous()
    st = PowerSGDState(**_hp(matrix_approximation_rank=1))
    d = b.cuda()
    st.compress_bucket(d, [(0, (n, m))])
    torch.cuda.synchronize()
    assert rel_fro(d.cpu().double().numpy(), b.double().numpy()) < 1e-6
    e = st.error(0, 0).cpu().double().numpy()
    assert np.linalg.norm(e) / np.linalg.norm(b.double().numpy()) < 1e-6


def test_rank_deficient_matrix_keeps_the_error_feedback_identity():
    log("case: rank-1 M at r = 2: M_hat + E = M', finite like the oracle")
    n, m = 256, 96
    g = torch.Generator().manual_seed(6)
    b = (torch.randn(n, 1, generator=g) @ torch.randn(1, m, generator=g)).reshape(-1)
    hp = _hp(matrix_approximation_rank=2)
    st = PowerSGDState(**hp)
    d = b.clone().cuda()
    st.compress_bucket(d, [(0, (n, m))])
    orc = oracle.OracleState(oracle.HParams(**hp))
    res = orc.compress_bucket(b.numpy(), [(0, (n, m))])
    torch.cuda.synchronize()
    mh = d.cpu().double().numpy().reshape(n, m)
    e = st.error(0, 0).cpu().double().numpy()
    bb = b.double().numpy().reshape(n, m)
    assert np.abs(mh + e - bb).max() <= 1e-5 * np.abs(bb).max()
    assert np.isfinite(mh).all() == np.isfinite(res.views[0].m_hat).all()


def test_rank_above_matrix_size_with_small_rate():
    log("case: r = 4 > min(n, m) = 3 with rate 0.25 -> rank 3, exact recovery")
    shapes = [(3, 5), (7, 3), (16, 16)]
    _run_parity(_hp(matrix_approximation_rank=4, min_compression_rate=0.25), shapes, steps=2)


def test_rate_boundary_matches_oracle_decisions():
    log("case: rate-test boundary shapes")
    shapes = [(8, 8), (9, 9), (16, 16), (17, 15), (4, 4), (5, 5), (100,)]
    hp = _hp(matrix_approximation_rank=2)
    par = _run_parity(hp, shapes, steps=1)
    assert par.gpu.decisions(0, len(shapes)) == [0, 1, 1, 1, 0, 0, 0]


def test_without_error_feedback_and_without_warm_start():
    log("case: no error feedback, no warm start (fresh draw every iteration)")
    shapes = [(128, 96), (64,), (256, 40)]
    _run_parity(_hp(use_error_feedback=False, warm_start=False), shapes, steps=3)


def test_warm_start_without_error_feedback():
    log("case: warm start, no error feedback")
    shapes = [(128, 96), (256, 40)]
    _run_parity(_hp(use_error_feedback=False), shapes, steps=4)


def test_error_feedback_without_warm_start():
    log("case: error feedback, no warm start")
    shapes = [(128, 96), (256, 40)]
    _run_parity(_hp(warm_start=False), shapes, steps=3)


def test_other_random_seed_and_bucket_index():
    log("case: random_seed 12345, bucket_index 7")
    shapes = [(100, 60), (70, 33)]
    views = packed_views(shapes)
    par = BucketParity(_hp(random_seed=12345), views, "f32", bucket_index=7)
    for step in range(2):
        par.step(_rand_bucket(shapes, 40 + step), step)


def test_start_iter_passthrough_then_compression():
    log("case: start_powerSGD_iter = 2 (vanilla phase is the identity)")
    shapes = [(64, 64), (32,)]
    _run_parity(_hp(start_powerSGD_iter=2), shapes, steps=4)


def test_start_iter_passthrough_fp16_unscales():
    log("case: fp16 with start_powerSGD_iter = 2 (unscale only, then compress)")
    shapes = [(64, 64), (32,)]
    _run_parity(_hp(start_powerSGD_iter=2), shapes, steps=4, dtype="f16",
                inv_scale=2.0 ** -10,
                bucket_fn=lambda s: _rand_bucket(shapes, 60 + s, scale=50.0))


@pytest.mark.parametrize("bad", [float("nan"), float("-inf")])
def test_fp16_nan_and_negative_inf_skip(bad):
    log(f"case: fp16 bucket with {bad}")
    shapes = [(64, 64), (32,)]

    def fn(step):
        b = _rand_bucket(shapes, 70 + step, scale=50.0)
        if step == 1:
            b[4100] = bad
        return b
    _run_parity(_hp(), shapes, steps=3, dtype="f16", inv_scale=2.0 ** -10, bucket_fn=fn)


@pytest.mark.parametrize("rank", [2, 32])
def test_fp16_skips_on_the_first_call_and_in_a_row(rank):
    """An fp16 bucket keeps M' in the error memory's place once a step has run; a step
    skipped for inf must leave every piece of state as it was, including on the very
    first call (the error memory still holds the error itself) and for two calls in a
    row. The oracle decides which steps are skipped."""
    log(f"case: fp16, r={rank}, inf at steps 0, 3 and 4 of 7")
    shapes = [(96, 160), (40,), (300, 64)]
    bad_steps = {0, 3, 4}

    def fn(step):
        b = _rand_bucket(shapes, 90 + step, scale=50.0)
        if step in bad_steps:
            b[100 + 7 * step] = float("inf")
        return b
    par = _run_parity(_hp(matrix_approximation_rank=rank, min_compression_rate=1.0), shapes,
                      steps=7, dtype="f16", inv_scale=2.0 ** -10, bucket_fn=fn)
    assert par.gpu.decisions(0, 3) == [1, 0, 1]


def test_fp16_skip_right_after_an_import():
    """Import puts the error itself back in the error memory's place; a skipped fp16
    step right after it must leave it there, and the next step continues from it."""
    log("case: fp16, r=2: 2 steps, export, import into a fresh state, inf, 2 more steps")
    shapes = [(128, 96), (24,)]
    views = packed_views(shapes)
    hp = _hp(min_compression_rate=1.0)
    par = BucketParity(hp, views, "f16")
    scale = 2.0 ** -10
    for step in range(2):
        par.step(_rand_bucket(shapes, 300 + step, scale=50.0).to(torch.float16), step,
                 inv_loss_scale=scale)
    blob = par.gpu.export_state()
    fresh = PowerSGDState(**hp)
    fresh.import_state(blob)
    par.gpu = fresh
    for step in range(2, 5):
        b = _rand_bucket(shapes, 300 + step, scale=50.0)
        if step == 2:
            b[5] = float("inf")
        rep = par.step(b.to(torch.float16), step, inv_loss_scale=scale)
        log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items())
            + (" (inf: skipped)" if rep.found_inf else ""))
        assert rep.found_inf == (step == 2)


@pytest.mark.parametrize("rank", [2, 32])
def test_fp16_two_mprime_places_match_one_checked_place(rank):
    """A state whose bucket plan was created by an fp16 call keeps M' in two
    alternating places and checks the bucket inside pass 1; a state restored from a
    snapshot keeps one place and checks the bucket before pass 1. Both must give the
    same bits through steps skipped for inf (two of them in a row) and the steps after
    them: outputs, found_inf, errors and snapshots. Rows of 160, 64, 77 and 2100 values
    take the aligned, unaligned and (rank 32) several-column-group paths."""
    log(f"case: fp16, r={rank}, two M' places against one, inf at steps 2, 3 and 5")
    shapes = [(96, 160), (40,), (300, 64), (130, 77), (40, 2100)]
    views = packed_views(shapes)
    hp = _hp(matrix_approximation_rank=rank, min_compression_rate=1.0)
    scale = 2.0 ** -10
    bad = {2, 3, 5}
    a = PowerSGDState(**hp)
    b = None
    for step in range(7):
        x = _rand_bucket(shapes, 500 + step, scale=50.0)
        if step in bad:
            x[11 + 3 * step] = float("inf")
        xh = x.to(torch.float16).cuda()
        if step == 1:
            b = PowerSGDState(**hp)
            b.import_state(a.export_state())
        outs = []
        for st in (a, b) if b is not None else (a,):
            xs = xh.clone()
            fi = torch.zeros(1, dtype=torch.int32, device="cuda")
            st.compress_bucket(xs, views, inv_loss_scale=scale, found_inf=fi)
            outs.append((xs, fi))
        torch.cuda.synchronize()
        assert outs[0][1].item() == (1 if step in bad else 0), step
        if b is None:
            continue
        (xa, fa), (xb, fb) = outs
        assert fa.item() == fb.item(), step
        assert torch.equal(xa.view(torch.int16), xb.view(torch.int16)), step
        for vi, (_, shp) in enumerate(views):
            if len(shp) < 2:
                continue
            assert torch.equal(a.error(0, vi).view(torch.int32),
                               b.error(0, vi).view(torch.int32)), (step, vi)
        assert a.export_state() == b.export_state(), step
    log("  7 steps: outputs, found_inf, errors and snapshots bitwise identical")


def test_misaligned_bucket_base_pointer():
    log("case: bucket starts 1 element into an allocation (scalar path)")
    shapes = [(64, 64), (48, 100), (7,)]
    views = packed_views(shapes)
    hp = _hp()
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle.HParams(**hp))
    for step in range(3):
        b = _rand_bucket(shapes, 80 + step)
        raw = torch.zeros(b.numel() + 1, device="cuda")
        raw[1:] = b.cuda()
        d = raw[1:]
        st.compress_bucket(d, views)
        res = orc.compress_bucket(b.numpy(), views)
        torch.cuda.synchronize()
        out = d.cpu().double().numpy()
        for (off, shp), vr in zip(views, res.views):
            if vr.compressed:
                got = out[off:off + numel(shp)].reshape(vr.n, vr.m)
                assert rel_fro(got, vr.m_hat) < 1e-4
        assert raw[0].item() == 0.0


def test_two_buckets_per_iteration():
    log("case: two buckets per iteration, is_last on the second")
    shapes_a = [(96, 80), (16,)]
    shapes_b = [(40, 120), (120, 40)]
    hp = _hp()
    par_a = BucketParity(hp, packed_views(shapes_a), "f32", bucket_index=0)
    par_b = BucketParity(hp, packed_views(shapes_b), "f32", bucket_index=1)
    # both sides share one state per run, as one hook state serves all buckets
    par_b.gpu = par_a.gpu
    par_b.oracle = par_a.oracle
    for step in range(3):
        par_a.step(_rand_bucket(shapes_a, 90 + step), step, is_last=False)
        par_b.step(_rand_bucket(shapes_b, 95 + step), step, is_last=True)
    it, nin, ncomm = par_a.gpu.stats()
    assert (it, nin, ncomm) == (par_a.oracle.iteration, par_a.oracle.numel_in,
                                par_a.oracle.numel_comm)


def test_layout_change_is_rejected_when_state_is_memorized():
    st = PowerSGDState(**_hp())
    d = torch.randn(64 * 64, device="cuda")
    st.compress_bucket(d, [(0, (64, 64))])
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket(d, [(0, (32, 128))])
    assert ei.value.status == api.POWERSGD_ERR_LAYOUT_CHANGED
    st2 = PowerSGDState(**_hp(use_error_feedback=False, warm_start=False))
    st2.compress_bucket(d, [(0, (64, 64))])
    st2.compress_bucket(d, [(0, (32, 128))])


def test_invalid_views_are_rejected():
    st = PowerSGDState(**_hp())
    d = torch.randn(100, device="cuda")
    for views in ([(0, (10, 11))], [(-1, (4, 4))], [(0, (8, 8)), (60, (8, 8))],
                  [(0, (2, -3))]):
        with pytest.raises(PowerSGDError) as ei:
            st.compress_bucket(d, views)
        assert ei.value.status == api.POWERSGD_ERR_INVALID_ARG
    h = torch.randn(100, device="cuda").half()
    with pytest.raises(PowerSGDError):
        api.powersgd_compress_bucket(st._state, 0, True, h.data_ptr(), api.POWERSGD_F16, 100,
                                     [(0, (10, 10))], 1.0, None, None)


def test_empty_and_vector_only_buckets():
    st = PowerSGDState(**_hp())
    d = torch.randn(50, device="cuda")
    ref = d.clone()
    st.compress_bucket(d, [(0, (50,)), (50, (0, 4))])
    st.compress_bucket(d, [], bucket_index=1)
    torch.cuda.synchronize()
    assert torch.equal(d, ref)


@pytest.mark.parametrize("rank,orth_launches", [(4, 1), (16, 4)])
def test_kernel_timing_reports_every_pass(rank, orth_launches):
    """Vector ranks orthogonalize P inside pass 2, so the orthogonalization kernel runs
    once (the initial Q); matrix-core ranks run it for Q and then for P every step."""
    log(f"case: kernel timing at rank {rank}")
    st = PowerSGDState(**_hp(matrix_approximation_rank=rank))
    st.set_timing(True)
    d = torch.randn(512 * 300, device="cuda")
    for _ in range(3):
        st.compress_bucket(d, [(0, (512, 300))])
    times = {name: (ms, n, by) for name, ms, n, by in st.kernel_times()}
    for k in ("pass1_mq", "pass2_mtp", "pass3_decompress_error"):
        assert times[k][1] == 3 and times[k][0] > 0, k
    assert times["orthogonalize"][1] == orth_launches
    assert times["pass1_mq"][2] == pytest.approx(3 * 512 * 300 * 12)


def test_full_rank_square_bucket_recovers_input():
    log("case: r = n (full rank) -> M_hat = M")
    shapes = [(8, 64)]
    par = _run_parity(_hp(matrix_approximation_rank=8, min_compression_rate=0.1), shapes,
                      steps=2)
    assert par.gpu.decisions(0, 1) == [1]


@pytest.mark.parametrize("rank", [16, 20, 32])
def test_matrix_core_ranks_with_ragged_shapes(rank):
    log(f"case: rank {rank} on matrix cores, ragged rows/columns, misaligned view")
    shapes = [(300, 520), (77, 1030), (37,), (130, 129), (1029, 64)]
    _run_parity(_hp(matrix_approximation_rank=rank, orthogonalization_epsilon=1e-8,
                    min_compression_rate=1.0), shapes, steps=3)


def test_matrix_core_rank32_fp16():
    log("case: rank 32, fp16 bucket")
    shapes = [(256, 320), (64,), (160, 512)]
    _run_parity(_hp(matrix_approximation_rank=32), shapes, steps=3, dtype="f16",
                inv_scale=2.0 ** -8, bucket_fn=lambda s: _rand_bucket(shapes, 110 + s, 20.0))


def test_tall_narrow_matrices_keep_their_p_rows_in_lds():
    """Row blocks of narrow matrices are capped so that a pass-2 workgroup holds its
    orthogonalized P rows in LDS (ranks 4 and 8, several row blocks, ragged tails)."""
    log("case: tall narrow matrices, r = 8, row blocks capped by the LDS staging")
    hp = _hp(matrix_approximation_rank=8, min_compression_rate=0.5)
    par = _run_parity(hp, [(5003, 4), (3001, 12), (2049, 9), (40,)], steps=3, seed=7)
    assert par.gpu.decisions(0, 4) == [1, 1, 1, 0]


def test_matrix_dimension_limit_is_rejected_before_device_work():
    """Rows and columns of a compressed matrix stop at 2^31 - 65537 (the kernels index
    rows in 32 bits with headroom past a work item's end). The sizes below are only
    claimed: every call returns its error before touching the 16-element buffer."""
    log("case: matrix dimension limit")
    lim = 2 ** 31 - 65537
    st = PowerSGDState(matrix_approximation_rank=1, start_powerSGD_iter=0,
                       compression_stats_logging_frequency=0)
    buf = torch.zeros(16, device="cuda")
    # a (lim + 1) x 8 view passes the rate test; the plan refuses it
    with pytest.raises(PowerSGDError) as ei:
        api.powersgd_compress_bucket(st._state, 0, True, buf.data_ptr(), api.POWERSGD_F32,
                                     (lim + 1) * 8, [(0, (lim + 1, 8))], 1.0, None, None)
    assert ei.value.status == api.POWERSGD_ERR_UNSUPPORTED
    # batched view: side lim + 1 is refused; side lim passes that check and stops at
    # the capacity check
    assert api.powersgd_batched_side(lim * lim + 1) == lim + 1
    with pytest.raises(PowerSGDError) as ei:
        api.powersgd_compress_bucket_batched(st._state, 1, True, buf.data_ptr(),
                                             api.POWERSGD_F32, lim * lim + 1, 2 ** 62, 1.0,
                                             None, None)
    assert ei.value.status == api.POWERSGD_ERR_UNSUPPORTED
    with pytest.raises(PowerSGDError) as ei:
        api.powersgd_compress_bucket_batched(st._state, 1, True, buf.data_ptr(),
                                             api.POWERSGD_F32, lim * lim, 16, 1.0, None, None)
    assert ei.value.status == api.POWERSGD_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf).item() == 0
    assert st.stats()[0] == 0  # no call got as far as the iteration counter
