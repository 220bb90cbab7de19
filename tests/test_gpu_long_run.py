"""Per-step parity over long warm-started trajectories: 60 steps in which every step
starts from the oracle's state (its snapshot imported into the library), so each
step's arithmetic is compared against the oracle at the fp32 bound however long the
run. Over a free-running trajectory two correct runs part beyond 1e-4 after some 20 to
40 steps (tests/test_oracle_trajectory.py shows it with the oracle against itself)."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, StepReport, compare_sampled, log, oracle_hparams, rel_fro
from rank_gradient_compression_amd import PowerSGDState
from synthetic import CONFIGS, BucketGenerator, shrink_config
from test_oracle_trajectory import SMALL_RESNET

pytestmark = pytest.mark.gpu

CASES = [("single 256x512, r = 1", 0, None), ("ResNet-shaped small bucket, r = 2", 1, SMALL_RESNET)]


@pytest.mark.parametrize("name,config,shapes", CASES, ids=[c[0] for c in CASES])
def test_sixty_steps_each_from_the_oracle_state(name, config, shapes):
    log(f"case: {name}, 60 steps from the oracle's state")
    base = CONFIGS[config]
    cfg = shrink_config(base, shapes or [s for _, s in base.views()], steps=60)
    hp = dict(cfg.hparams)
    hp["compression_stats_logging_frequency"] = 0
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    gen = BucketGenerator(cfg, "cpu")
    views = cfg.views()
    worst = 0.0
    for step in range(60):
        g = gen.bucket(step)
        if step > 0:
            st.import_state(orc.export_state())
        dev = g.cuda()
        st.compress_bucket(dev, views)
        res = orc.compress_bucket(g.numpy(), views)
        torch.cuda.synchronize()
        out = dev.cpu().double().numpy()
        for vi, ((off, shp), vr) in enumerate(zip(views, res.views)):
            if not vr.compressed:
                continue
            p, q = st.factors(0, vi)
            e = st.error(0, vi).double().cpu().numpy()
            errs = (rel_fro(out[off:off + vr.n * vr.m].reshape(vr.n, vr.m), vr.m_hat),
                    rel_fro(p.double().cpu().numpy(), vr.p),
                    rel_fro(q.double().cpu().numpy(), vr.q),
                    rel_fro(e, vr.error))
            assert max(errs) <= TOL["f32"], (step, vi, errs)
            worst = max(worst, max(errs))
    log(f"  worst over 60 steps: {worst:.2e} (bound {TOL['f32']:.0e})")


def test_sixty_amp_steps_each_from_the_oracle_state():
    """The fp16 AMP call (loss scale 65536, gradients x 2^-10 before it) over 60 steps of
    a ResNet-shaped bucket at r = 4, each step from the oracle's state; step 10 carries
    an inf, so both sides skip it and leave the state as it was."""
    log("case: AMP fp16, ResNet-shaped small bucket, r = 4, 60 steps from the oracle's state")
    cfg = shrink_config(CONFIGS[4], SMALL_RESNET, steps=60)
    hp = dict(cfg.hparams)
    hp["compression_stats_logging_frequency"] = 0
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    gen = BucketGenerator(cfg, "cpu")
    views = cfg.views()
    inv = 1.0 / cfg.loss_scale
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    worst, skipped = 0.0, []
    for step in range(60):
        g = gen.bucket(step)
        if step > 0:
            st.import_state(orc.export_state())
        dev = g.cuda()
        found.zero_()
        st.compress_bucket(dev, views, inv_loss_scale=inv, found_inf=found)
        res = orc.compress_bucket(g.numpy(), views, inv_loss_scale=inv)
        inf = oracle.any_nonfinite(g.numpy(), views)
        torch.cuda.synchronize()
        assert int(found.item()) == int(inf), step
        if inf:
            skipped.append(step)
            continue
        rep = StepReport(step=step)
        for vi, ((off, shp), vr) in enumerate(zip(views, res.views)):
            if vr.compressed:
                compare_sampled(st, 0, vi, vr, dev[off:off + vr.n * vr.m], TOL["f16"], rep)
        worst = max([worst] + list(rep.worst.values()))
    assert 10 in skipped
    log(f"  worst over 60 steps: {worst:.2e} (bound {TOL['f16']:.0e}); skipped {skipped}")
