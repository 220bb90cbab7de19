"""GPU parity: the HIP library against the fp64 oracle, element by element, on
seeded synthetic buckets of the benchmark workloads' shapes (oracle-sized), every
step of the trajectory. See tests/parity.py for the comparison rules."""
import pytest
import torch

from parity import BucketParity, log
from synthetic import CONFIGS, BucketGenerator, packed_views, shrink_config

pytestmark = pytest.mark.gpu


def _run(cfg, steps=None, hp_over=None, bucket_index=0):
    hp = dict(cfg.hparams)
    hp.update(hp_over or {})
    gen = BucketGenerator(cfg, "cpu")
    par = BucketParity(hp, cfg.views(), cfg.dtype, bucket_index)
    scale = cfg.loss_scale
    reports = []
    for step in range(cfg.steps if steps is None else steps):
        if cfg.dtype == "f16":
            b = gen.bucket(step, loss_scale=scale)
            rep = par.step(b, step, inv_loss_scale=1.0 / scale)
            if rep.found_inf:
                scale *= 0.5      # GradScaler backoff
        else:
            rep = par.step(gen.bucket(step), step)
        log(f"{cfg.name} step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items())
            + (" (inf: skipped)" if rep.found_inf else ""))
        reports.append(rep)
    return par, reports


def test_single_matrix_rank1_three_steps():
    log("case: workload 0 (256x512 fp32, r=1), 3 steps")
    _run(CONFIGS[0])


RESNET_SMALL = [(64, 3, 7, 7), (64,), (64, 64, 3, 3), (256, 64, 1, 1), (128, 128, 3, 3),
                (512, 128, 1, 1), (256,), (300, 2304), (1000, 260), (2048,), (17, 4099)]


def test_resnet_shapes_small_rank2():
    # misaligned rows (147 columns), vectors between matrices, ragged row and column
    # tails, several row tiles per matrix
    log("case: ResNet-shaped small bucket, r=2, 6 steps")
    _run(shrink_config(CONFIGS[1], RESNET_SMALL, steps=6))


def test_bert_shapes_small_rank4_batched():
    shapes = [(256, 256), (256, 256), (1024, 256), (256, 1024), (256,), (1024,), (256,)] * 2
    log("case: BERT-shaped small bucket, r=4, batched, 20 steps")
    _run(shrink_config(CONFIGS[2], shapes, steps=20))


def test_gpt_shapes_small_rank32():
    shapes = [(512, 512), (512, 2048), (2048, 512)]
    log("case: GPT-shaped small bucket, r=32, eps=1e-8, 10 steps")
    _run(shrink_config(CONFIGS[3], shapes, steps=10))


def test_amp_fp16_small_with_inf_steps():
    shapes = [(256, 256), (1024, 256), (256,), (256, 1024), (1024,)]
    log("case: fp16 AMP small bucket, r=4, 12 steps, inf at step 10")
    par, reps = _run(shrink_config(CONFIGS[4], shapes, steps=12))
    assert reps[10].found_inf and not reps[9].found_inf


def test_batched_equals_unbatched_bitwise():
    cfg = shrink_config(CONFIGS[2], [(256, 256), (128, 512), (256, 256), (64,), (128, 512)],
                        steps=3)
    gen = BucketGenerator(cfg, "cpu")
    outs = []
    for batched in (False, True):
        hp = dict(cfg.hparams)
        hp["batch_tensors_with_same_shape"] = batched
        from rank_gradient_compression_amd import PowerSGDState
        st = PowerSGDState(**hp)
        res = []
        for step in range(3):
            d = gen.bucket(step).cuda()
            st.compress_bucket(d, cfg.views())
            res.append(d.cpu())
        outs.append(res)
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_two_runs_are_bitwise_identical():
    cfg = shrink_config(CONFIGS[1], RESNET_SMALL, steps=3)
    gen = BucketGenerator(cfg, "cpu")
    from rank_gradient_compression_amd import PowerSGDState
    runs = []
    for _ in range(2):
        st = PowerSGDState(**cfg.hparams)
        res = []
        for step in range(3):
            d = gen.bucket(step).cuda()
            st.compress_bucket(d, cfg.views())
            res.append(d.cpu())
            p, q = st.factors(0, 7)
            res += [p.cpu(), q.cpu(), st.error(0, 7).cpu()]
        runs.append(res)
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
