"""GPU parity on seeded random bucket layouts: up to nine views mixing vectors, matrices
of ragged sizes (1 to 699 rows, 1 to 1399 columns: widths below, at and above the
lane and column-block sizes, unaligned rows) and 4-D conv-like views, at padded and
unpadded ranks (1 to 8), rate thresholds 0.5 to 2 (0.5 admits 1 x m matrices, where
r = min(n, m)), fp32 and fp16 AMP, ranks 16 and 32 on the matrix cores, and the
fp16/bf16 wrapped hook checked step by step from the oracle's state. Values are low-rank plus noise with singular values falling
as 0.7^j, so P and Q are well determined and held to the same bound as M_hat and E."""
import math

import numpy as np
import pytest
import torch

from parity import BucketParity, log
from synthetic import packed_views

pytestmark = pytest.mark.gpu


def _layout(rng):
    shapes = []
    for _ in range(int(rng.integers(1, 10))):
        kind = rng.random()
        if kind < 0.25:
            shapes.append((int(rng.integers(1, 3000)),))
        elif kind < 0.8:
            shapes.append((int(rng.integers(1, 700)), int(rng.integers(1, 1400))))
        else:
            shapes.append((int(rng.integers(1, 130)), int(rng.integers(1, 40)),
                           int(rng.integers(1, 4)), int(rng.integers(1, 4))))
    return shapes


def _bucket(shapes, step, seed, scale=1.0, kmax=16, decay=0.7):
    """Per matrix view: a fixed part sum_j decay^j u_j v_j^T (j < min(kmax, n, m), u and
    v N(0, 1) per view) plus fresh N(0, 0.01^2) noise each step; vectors N(0, 1)."""
    parts = []
    for vi, shp in enumerate(shapes):
        size = math.prod(shp)
        gs = torch.Generator().manual_seed(seed * 7919 + step * 131 + vi)
        if len(shp) < 2:
            parts.append(torch.randn(size, generator=gs, dtype=torch.float64))
            continue
        n, m = shp[0], size // shp[0]
        k = min(kmax, n, m)
        g = torch.Generator().manual_seed(seed * 104729 + vi)
        u = torch.randn(n, k, generator=g, dtype=torch.float64)
        v = torch.randn(m, k, generator=g, dtype=torch.float64)
        w = decay ** torch.arange(k, dtype=torch.float64)
        parts.append(((u * w) @ v.T + 0.01 * torch.randn(n, m, generator=gs,
                                                         dtype=torch.float64)).reshape(-1))
    return (torch.cat(parts) * scale).float()


RANKS = [1, 2, 3, 4, 5, 8, 1, 2, 3, 4, 6, 7]
RATES = [2.0, 2.0, 1.0, 2.0, 0.5, 2.0, 0.5, 2.0, 2.0, 1.0, 2.0, 1.5]
CASES = [(seed, RANKS[seed], RATES[seed], "f32") for seed in range(12)] + \
        [(12, 2, 2.0, "f16"), (13, 4, 1.0, "f16"), (14, 1, 0.5, "f16")]


@pytest.mark.parametrize("seed,rank,rate,dtype", CASES)
def test_random_layout(seed, rank, rate, dtype):
    rng = np.random.default_rng(1000 + seed)
    shapes = _layout(rng)
    log(f"case: random layout {seed}, rank {rank}, rate {rate}, {dtype}: {shapes}")
    hp = dict(matrix_approximation_rank=rank, start_powerSGD_iter=0, min_compression_rate=rate,
              use_error_feedback=True, warm_start=True,
              orthogonalization_epsilon=0.0 if rank <= 4 else 1e-8, random_seed=seed,
              compression_stats_logging_frequency=0)
    par = BucketParity(hp, packed_views(shapes), dtype)
    scale = 1024.0 if dtype == "f16" else 1.0  # a power-of-two loss scale
    for step in range(3):
        b = _bucket(shapes, step, seed, scale)
        if dtype == "f16":
            b = b.to(torch.float16)
        rep = par.step(b, step, inv_loss_scale=1.0 / scale)
        log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items()))


WRAPPED_CASES = [(20, 2, 2.0, "bf16"), (21, 4, 1.0, "f16"), (22, 3, 0.5, "bf16"), (23, 8, 2.0, "f16")]


@pytest.mark.parametrize("seed,rank,rate,dt", WRAPPED_CASES)
def test_random_layout_wrapped_stepwise(seed, rank, rate, dt):
    """The wrapped hook (16-bit state) on random layouts, each step from the oracle's
    state (imported through the snapshot), so that one step's arithmetic is compared;
    gradients scaled by 1/16 keep P = M' Q, which grows like sigma^2 with the warm Q,
    inside the float16 range."""
    import oracle
    from parity import TOL_WRAPPED, oracle_hparams, rel_fro
    from rank_gradient_compression_amd import PowerSGDState
    rng = np.random.default_rng(1000 + seed)
    shapes = _layout(rng)
    log(f"case: random layout {seed}, wrapped {dt}, rank {rank}, rate {rate}: {shapes}")
    views = packed_views(shapes)
    hp = dict(matrix_approximation_rank=rank, start_powerSGD_iter=0, min_compression_rate=rate,
              use_error_feedback=True, warm_start=True,
              orthogonalization_epsilon=0.0 if rank <= 4 else 1e-8, random_seed=seed,
              compression_stats_logging_frequency=0)
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    tol = TOL_WRAPPED[dt]
    for t in range(3):
        x = _bucket(shapes, t, seed, 1.0 / 16)
        if t > 0:
            st.import_state(orc.export_state())
        dev = x.cuda()
        st.compress_bucket_wrapped(dev, views, dt)
        res = orc.compress_bucket_wrapped(x.numpy(), views, dt)
        torch.cuda.synchronize()
        out = dev.cpu().numpy()
        assert st.decisions(0, len(views)) == [int(v.compressed) for v in res.views]
        for vi, ((off, shp), vr) in enumerate(zip(views, res.views)):
            size = math.prod(shp)
            if not vr.compressed:
                np.testing.assert_array_equal(out[off:off + size], res.output[off:off + size])
                continue
            p, q = st.factors(0, vi)
            e = st.error(0, vi).double().cpu().numpy()
            errs = {"Mhat": rel_fro(out[off:off + size].reshape(vr.n, vr.m), vr.m_hat),
                    "P": rel_fro(p.double().cpu().numpy(), vr.p),
                    "Q": rel_fro(q.double().cpu().numpy(), vr.q),
                    "E": rel_fro(e, vr.error, np.linalg.norm(vr.m_prime))}
            for key, v in errs.items():
                assert v <= tol, (t, vi, key, v, shp)
        log(f"  step {t}: within {tol:.1e}")


MFMA_CASES = [(30, 16, 2.0, "f32"), (31, 32, 2.0, "f32"), (32, 32, 1.0, "f32"), (33, 16, 2.0, "f16")]


@pytest.mark.parametrize("seed,rank,rate,dtype", MFMA_CASES)
def test_random_layout_matrix_cores(seed, rank, rate, dtype):
    """Ranks 16 and 32 (the matrix-core passes) on random layouts; the spectrum falls as
    0.9^j over up to 64 components, so the 32nd value stays well above the noise."""
    rng = np.random.default_rng(1000 + seed)
    shapes = _layout(rng)
    log(f"case: random layout {seed}, rank {rank}, rate {rate}, {dtype}: {shapes}")
    hp = dict(matrix_approximation_rank=rank, start_powerSGD_iter=0, min_compression_rate=rate,
              use_error_feedback=True, warm_start=True, orthogonalization_epsilon=1e-8,
              random_seed=seed, compression_stats_logging_frequency=0)
    par = BucketParity(hp, packed_views(shapes), dtype)
    scale = 256.0 if dtype == "f16" else 1.0
    for step in range(3):
        b = _bucket(shapes, step, seed, scale, kmax=64, decay=0.9)
        if dtype == "f16":
            b = b.to(torch.float16)
        rep = par.step(b, step, inv_loss_scale=1.0 / scale)
        log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items()))
