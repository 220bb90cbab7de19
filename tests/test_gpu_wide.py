"""GPU parity on matrices four or more 256-column blocks wide: whole groups of four
blocks, a partial fifth block (1100 columns), rows that are not 16-byte multiples
(1030 and 4099 columns: unaligned access), several row blocks per matrix, every
vector rank, fp32, fp16 AMP and the 16-bit wrapped state (checked step by step from
the oracle's state), the matrix-core ranks' column groups, and a bucket that starts
one element into its allocation."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL_WRAPPED, log, oracle_hparams, rel_fro
from synthetic import CONFIGS, packed_views, shrink_config
from test_gpu_parity import _run
from test_gpu_wrapped import _bucket as wrapped_bucket
from test_gpu_wrapped import _hp as wrapped_hp
from rank_gradient_compression_amd import PowerSGDState

pytestmark = pytest.mark.gpu

WIDE = [(300, 1024), (64,), (200, 1100), (150, 1030), (1100, 2048), (7,), (33, 4099)]
# every matrix 16-byte aligned and at least 256 columns wide (the 16-bit state's pass 2
# then runs a kernel compiled for that access alone); odd-length vectors come last
WIDE_ALIGNED = [(300, 1024), (64,), (200, 1100), (1100, 2048), (96, 512), (40, 256), (7,)]


@pytest.mark.parametrize("rank", [1, 2, 4, 8])
def test_wide_fp32(rank):
    log(f"case: wide matrices, fp32, rank {rank}, 4 steps")
    _run(shrink_config(CONFIGS[2], WIDE, steps=4), hp_over={"matrix_approximation_rank": rank})


def test_wide_amp_fp16():
    log("case: wide matrices, fp16 AMP, rank 4, 4 steps")
    _run(shrink_config(CONFIGS[4], WIDE, steps=4))


@pytest.mark.parametrize("shapes", ["mixed", "aligned"])
@pytest.mark.parametrize("dt,rank", [("bf16", 2), ("f16", 4), ("f16", 8), ("bf16", 8)])
def test_wide_wrapped_stepwise(dt, rank, shapes):
    """Each step starts from the oracle's state (its snapshot imported into the
    library), so the comparison measures one step's arithmetic, not the drift of two
    trajectories: free-running, a one-ulp difference after the first step grows to 9u
    in P of the 150 x 1030 view at rank 8 with this 1/j spectrum, while one step from
    equal states stays within a fraction of u. Gradients are scaled by 1/16: with the
    warm-start Q carrying the singular values, P = M' Q grows like sigma^2 (about 2e6
    for the 1100 x 2048 view at scale 1), beyond the float16 range on both sides."""
    log(f"case: wide matrices ({shapes}), wrapped {dt}, rank {rank}, 3 steps from the "
        "oracle's state")
    views = packed_views(WIDE if shapes == "mixed" else WIDE_ALIGNED)
    hp = wrapped_hp(matrix_approximation_rank=rank)
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    tol = TOL_WRAPPED[dt]
    for t in range(3):
        x = wrapped_bucket(views, t, rank, rank, scale=1.0 / 16)
        if t > 0:
            st.import_state(orc.export_state())
        dev = x.cuda()
        st.compress_bucket_wrapped(dev, views, dt)
        res = orc.compress_bucket_wrapped(x.numpy(), views, dt)
        torch.cuda.synchronize()
        out = dev.cpu().numpy()
        worst = {}
        for vi, ((off, shp), vr) in enumerate(zip(views, res.views)):
            size = int(np.prod(shp))
            if not vr.compressed:
                np.testing.assert_array_equal(out[off:off + size], res.output[off:off + size])
                continue
            n, m = vr.n, vr.m
            p, q = st.factors(0, vi)
            e = st.error(0, vi).double().cpu().numpy()
            errs = {"Mhat": rel_fro(out[off:off + size].reshape(n, m), vr.m_hat),
                    "P": rel_fro(p.double().cpu().numpy(), vr.p),
                    "Q": rel_fro(q.double().cpu().numpy(), vr.q),
                    "E": rel_fro(e, vr.error, np.linalg.norm(vr.m_prime))}
            for key, v in errs.items():
                worst[key] = max(worst.get(key, 0.0), v)
                assert v <= tol, (t, vi, key, v, (n, m))
        log(f"  step {t}: " + ", ".join(f"{k}={v:.2e}" for k, v in worst.items())
            + f" (tol {tol:.1e})")


# Matrix-core ranks split each 32-row block into groups of 4096 columns whose partial P
# are summed in the Gram kernel: two and three groups with a short last one (4608 and
# 8452 columns), rows that are not 16-byte multiples (4099 and 6150 columns: the
# scalar-access body, also split into groups), one group over several row blocks with
# a ragged tail (2100 x 2060).
MC_WIDE = [(77, 4608), (64,), (40, 8452), (96, 4099), (9,), (300, 6150), (2100, 2060)]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("rank", [16, 32])
def test_wide_matrix_cores(rank, dtype):
    from test_gpu_edge import _hp as edge_hp, _rand_bucket, _run_parity
    log(f"case: matrix cores, rank {rank}, {dtype}, rows of up to 6150 columns, 3 steps")
    scale = 50.0 if dtype == "f16" else 1.0
    _run_parity(edge_hp(matrix_approximation_rank=rank, min_compression_rate=1.0,
                        orthogonalization_epsilon=1e-8), MC_WIDE, steps=3, dtype=dtype,
                inv_scale=2.0 ** -10 if dtype == "f16" else 1.0,
                bucket_fn=lambda t: _rand_bucket(MC_WIDE, 500 + t, scale))


@pytest.mark.parametrize("rank,shapes", [(4, WIDE), (32, MC_WIDE)], ids=["r4", "r32"])
def test_wide_misaligned_bucket(rank, shapes):
    log(f"case: wide matrices, bucket one element into its allocation, rank {rank}")
    views = packed_views(shapes)
    hp = dict(matrix_approximation_rank=rank, start_powerSGD_iter=0, min_compression_rate=2.0,
              use_error_feedback=True, warm_start=True, orthogonalization_epsilon=0.0,
              random_seed=5, compression_stats_logging_frequency=0)
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle.HParams(**hp))
    numel = views[-1][0] + int(np.prod(shapes[-1]))
    for step in range(3):
        g = torch.Generator().manual_seed(200 + step)
        b = torch.randn(numel, generator=g)
        raw = torch.zeros(numel + 1, device="cuda")
        raw[1:] = b.cuda()
        st.compress_bucket(raw[1:], views)
        res = orc.compress_bucket(b.numpy(), views)
        torch.cuda.synchronize()
        out = raw[1:].cpu().double().numpy()
        for (off, shp), vr in zip(views, res.views):
            if vr.compressed:
                got = out[off:off + vr.n * vr.m].reshape(vr.n, vr.m)
                assert rel_fro(got, vr.m_hat) < 1e-4, (step, shp)
        assert raw[0].item() == 0.0
        log(f"  step {step}: M_hat within 1e-4 of the oracle")
