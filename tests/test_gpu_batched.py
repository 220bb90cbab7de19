"""GPU parity of the batched variant (batched_powerSGD_hook: the whole bucket as one
zero-padded square matrix) against the oracle, element by element, through the C ABI.
Before every call the padding past the bucket is filled with NaN, so a library that did
not zero it would fail every comparison."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, log, rel_fro
from rank_gradient_compression_amd import PowerSGDError, PowerSGDState
from rank_gradient_compression_amd import powersgd as api
from synthetic import CONFIGS, BucketGenerator

pytestmark = pytest.mark.gpu


def _hp(**kw):
    base = dict(matrix_approximation_rank=1, start_powerSGD_iter=0, min_compression_rate=2.0,
                use_error_feedback=True, warm_start=True, orthogonalization_epsilon=0.0,
                random_seed=0, compression_stats_logging_frequency=0)
    base.update(kw)
    return base


def _low_rank_plus_noise(numel, step, seed, k=16):
    g = torch.Generator().manual_seed(seed)
    s = oracle.batched_side(numel)
    u = torch.randn(s, k, generator=g, dtype=torch.float64)
    v = torch.randn(s, k, generator=g, dtype=torch.float64)
    w = torch.tensor([1.0 / (j + 1) for j in range(k)], dtype=torch.float64)
    base = ((u * w) @ v.T).reshape(-1)[:numel]
    gs = torch.Generator().manual_seed(seed * 1000 + step + 1)
    return (base + 0.01 * torch.randn(numel, generator=gs, dtype=torch.float64)).float()


def _compare(st, buf, numel, res, tol, bucket_index=0):
    s = oracle.batched_side(numel)
    worst = {}
    out = buf[:numel].double().cpu().numpy()
    worst["out"] = rel_fro(out, res.output64)
    vr = res.views[0]
    p, q = st.factors(bucket_index, 0)
    worst["P"] = rel_fro(p.double().cpu().numpy(), vr.p)
    worst["Q"] = rel_fro(q.double().cpu().numpy(), vr.q)
    if vr.error is not None:
        e = st.error(bucket_index, 0).double().cpu().numpy()
        assert e.shape == (s, s)
        en = np.linalg.norm(vr.error)
        mn = np.linalg.norm(vr.m_prime)
        worst["E"] = rel_fro(e, vr.error, None if en >= 1e-3 * mn else mn)
    for k, v in worst.items():
        assert v <= tol, (k, v)
    return worst


def _run(hp, numel, steps, seed=0, dtype=torch.float32, inv=1.0, bucket_fn=None,
         capacity_extra=0):
    s = oracle.batched_side(numel)
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle.HParams(**{k: v for k, v in hp.items()
                                               if k in oracle.HParams.__dataclass_fields__}))
    buf = torch.empty(s * s + capacity_extra, dtype=dtype, device="cuda")
    found = torch.zeros(1, dtype=torch.int32, device="cuda") if dtype == torch.float16 else None
    tol = TOL["f16" if dtype == torch.float16 else "f32"]
    results = []
    for step in range(steps):
        # a spectrum of 2r terms: every column of P is well separated from the noise
        g = bucket_fn(step) if bucket_fn else _low_rank_plus_noise(
            numel, step, seed, k=max(16, 2 * hp["matrix_approximation_rank"]))
        g = g.to(dtype)
        buf[numel:].fill_(float("nan"))
        buf[:numel].copy_(g.cuda())
        if found is not None:
            found.zero_()
        st.compress_bucket_batched(buf, numel=numel, inv_loss_scale=inv, found_inf=found)
        res = orc.compress_bucket_batched(g.numpy(), inv_loss_scale=inv)
        torch.cuda.synchronize()
        if res.skipped or res.passthrough:
            np.testing.assert_array_equal(buf[:numel].cpu().numpy(), res.output)
            log(f"  step {step}: {'skipped' if res.skipped else 'passthrough'}, bit-exact")
        else:
            w = _compare(st, buf, numel, res, tol)
            log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in w.items()))
        results.append(res)
    return st, orc, results


@pytest.mark.parametrize("numel,rank", [(1000, 1), (5000, 4), (16284, 2), (20000, 8)])
def test_batched_parity_vector_ranks(numel, rank):
    s = oracle.batched_side(numel)
    log(f"case: batched, numel {numel} -> {s} x {s} ({s * s - numel} padded), r = {rank}")
    _run(_hp(matrix_approximation_rank=rank), numel, steps=4, seed=numel)


@pytest.mark.parametrize("numel,rank", [(16284, 32), (22400, 16), (150 * 150, 32)])
def test_batched_parity_matrix_core_ranks(numel, rank):
    s = oracle.batched_side(numel)
    log(f"case: batched, numel {numel} -> {s} x {s}, r = {rank} (matrix cores)")
    _run(_hp(matrix_approximation_rank=rank, orthogonalization_epsilon=1e-8), numel, steps=3,
         seed=numel)


@pytest.mark.parametrize("numel,rank", [(1, 4), (2, 1), (3, 4), (10, 3)])
def test_batched_tiny_buckets_at_full_rank(numel, rank):
    """Tiny buckets whose padded square has rank min(r, s): the step is lossless."""
    s = oracle.batched_side(numel)
    log(f"case: batched tiny bucket, numel {numel} -> {s} x {s}, r = {rank}")
    st, orc, res = _run(_hp(matrix_approximation_rank=rank), numel, steps=2, seed=numel)
    assert st.view_info(0, 0)[2] == min(rank, s)


def test_batched_rank_deficient_padding_keeps_the_error_feedback_identity():
    """numel 5 -> 3 x 3 with a zero row, rank 3 > rank(M') = 2: the last P column is
    rounding noise on both sides (parity unpinned there); M_hat + E = pad(G) holds."""
    log("case: batched rank-deficient padded square (numel 5, r = 4, eps 1e-8)")
    numel, s = 5, 3
    st = PowerSGDState(**_hp(matrix_approximation_rank=4, orthogonalization_epsilon=1e-8))
    g = torch.tensor([1.5, -2.0, 0.25, 3.0, -1.0])
    buf = torch.full((s * s,), float("nan"), device="cuda")
    buf[:numel].copy_(g.cuda())
    st.compress_bucket_batched(buf, numel=numel)
    torch.cuda.synchronize()
    m_hat = buf.double().cpu().numpy()
    e = st.error(0, 0).double().cpu().numpy().reshape(-1)
    padded = np.zeros(s * s)
    padded[:numel] = g.double().numpy()
    assert np.all(np.isfinite(m_hat)) and np.all(np.isfinite(e))
    np.testing.assert_allclose(m_hat + e, padded, rtol=0, atol=1e-5)


def test_batched_fp16_unscale_skip_and_passthrough():
    log("case: batched fp16: passthrough at iteration 0, inf skip at 2, compression after")
    numel = 3001
    scale = 2.0 ** 12

    def bucket(step):
        g = _low_rank_plus_noise(numel, step, 11) * scale
        if step == 2:
            g[17] = float("inf")
        return g

    st, orc, res = _run(_hp(matrix_approximation_rank=2, start_powerSGD_iter=1), numel, steps=5,
                        dtype=torch.float16, inv=1.0 / scale, bucket_fn=bucket)
    assert res[0].passthrough and res[2].skipped
    assert not res[3].skipped and not res[4].skipped


def test_batched_without_error_feedback_or_warm_start():
    log("case: batched without error feedback, fresh draw every call")
    _run(_hp(matrix_approximation_rank=2, use_error_feedback=False, warm_start=False), 777,
         steps=3, seed=3)


def test_batched_larger_buffer_and_stats():
    log("case: batched in a buffer larger than the padded square; statistics")
    numel = 2500  # s = 50, exact square
    st, orc, _ = _run(_hp(matrix_approximation_rank=3), numel, steps=2, seed=5,
                      capacity_extra=123)
    it, n_in, n_comm = st.stats()
    assert (it, n_in, n_comm) == (orc.iteration, orc.numel_in, orc.numel_comm) == (2, 5000, 600)


def test_batched_rejects_small_capacity_and_layout_changes():
    log("case: batched capacity and layout errors")
    st = PowerSGDState(**_hp())
    buf = torch.zeros(99, device="cuda")
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket_batched(buf, numel=82)  # s = 10 needs 100 elements
    assert ei.value.status == api.POWERSGD_ERR_INVALID_ARG
    st.compress_bucket(torch.zeros(64, device="cuda"), [(0, (8, 8))], bucket_index=0)
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket_batched(torch.zeros(64, device="cuda"), bucket_index=0)
    assert ei.value.status == api.POWERSGD_ERR_LAYOUT_CHANGED
    st.compress_bucket_batched(torch.zeros(64, device="cuda"), bucket_index=1)
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket_batched(torch.zeros(64, device="cuda"), numel=63, bucket_index=1)
    assert ei.value.status == api.POWERSGD_ERR_LAYOUT_CHANGED
    torch.cuda.synchronize()


def test_batched_resnet_bucket_full_size():
    """The benchmark's batched workload at full size: 18 614 912 elements as one 4315 x
    4315 matrix (4313 padded), rank 1, in the buffer layout the benchmark uses; the whole
    bucket is compared with the oracle on every step."""
    cfg = CONFIGS[5]
    gen = BucketGenerator(cfg, "cpu")
    log(f"case: {cfg.name} at full size, 3 steps")
    _run(dict(cfg.hparams, compression_stats_logging_frequency=0), cfg.numel, steps=3,
         bucket_fn=lambda step: gen.bucket(step))


def _random_batched_cases():
    """Seeded bucket sizes from 2 to 200 000 elements (squares, one past a square, primes
    and arbitrary sizes, so the padding runs from 0 to almost 2s) with ranks 1 to 8."""
    rng = np.random.default_rng(2024)
    sizes = [int(x) for x in rng.integers(2, 200_000, size=5)] + [317 * 317, 317 * 317 + 1,
                                                                   199_999, 65_521]
    ranks = [1, 2, 3, 4, 5, 8, 2, 4, 1]
    return list(zip(sizes, ranks))


@pytest.mark.parametrize("numel,rank", _random_batched_cases())
def test_batched_parity_seeded_sizes(numel, rank):
    s = oracle.batched_side(numel)
    log(f"case: batched, seeded size {numel} -> {s} x {s} ({s * s - numel} padded), r = {rank}")
    _run(_hp(matrix_approximation_rank=rank, orthogonalization_epsilon=0.0 if rank <= 4 else 1e-8),
         numel, steps=3, seed=numel % 9973)
