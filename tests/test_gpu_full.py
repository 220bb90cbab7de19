"""GPU parity at the benchmark workloads' full sizes, with the benchmark's own
plans (same views, hyperparameters, launch configuration) and inputs generated on
the GPU. The ResNet-50-shaped bucket is compared whole against the oracle; for the
larger buckets the oracle follows a sample of views (one or two per shape) through
every step with its own per-matrix functions, every other view is checked through
properties that hold at any size (vectors untouched, M_hat + E = M' + E_prev)."""
import numpy as np
import pytest
import torch

import oracle
from parity import (TOL, TOL_WRAPPED, WRAPPED_ORACLE_STEPS, BucketParity, StepReport,
                    TensorTrack, TensorTrackWrapped, check_wrapped_properties, compare_sampled,
                    log, numel, oracle_hparams, rel_fro)
from rank_gradient_compression_amd import PowerSGDState
from synthetic import CONFIGS, BucketGenerator

pytestmark = pytest.mark.gpu


def test_resnet50_bucket_full_every_view_every_step():
    cfg = CONFIGS[1]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, whole-bucket oracle")
    gen = BucketGenerator(cfg, "cuda")
    par = BucketParity(cfg.hparams, cfg.views(), "f32")
    for step in range(cfg.steps):
        rep = par.step(gen.bucket(step).cpu(), step)
        log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items()))


def _sampled(cfg, sample_views, steps=None):
    views = cfg.views()
    gen = BucketGenerator(cfg, "cuda")
    hp = dict(cfg.hparams)
    hp["compression_stats_logging_frequency"] = 0
    gpu = PowerSGDState(**hp)
    tracks = {}
    tol = TOL[cfg.dtype]
    scale = cfg.loss_scale
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    e_prev_sum = None
    for step in range(cfg.steps if steps is None else steps):
        if cfg.dtype == "f16":
            bucket = gen.bucket(step, loss_scale=scale)
            inv = 1.0 / scale
        else:
            bucket = gen.bucket(step)
            inv = 1.0
        host_in = {vi: bucket[off:off + numel(shp)].cpu() for vi, (off, shp) in
                   enumerate(views) if vi in sample_views}
        vec_in = [(off, bucket[off:off + numel(shp)].clone()) for off, shp in views
                  if len(shp) < 2]
        inf = False
        if cfg.dtype == "f16":
            inf = oracle.any_nonfinite(bucket.cpu().numpy(), views)
        found.zero_()
        gpu.compress_bucket(bucket, views, inv_loss_scale=inv,
                            found_inf=found if cfg.dtype == "f16" else None)
        torch.cuda.synchronize()
        rep = StepReport(step=step, found_inf=inf)
        if cfg.dtype == "f16":
            assert bool(found.item()) == inf, step
        if inf:
            log(f"  step {step}: inf found, skipped")
            scale *= 0.5
            continue
        for vi in sample_views:
            off, shp = views[vi]
            n, m, r = gpu.view_info(0, vi)
            if vi not in tracks:
                tracks[vi] = TensorTrack(hp, vi, n, m, r)
            g = host_in[vi].double().numpy()
            if cfg.dtype == "f16":
                g = g * inv
            vr = tracks[vi].step(g, step)
            compare_sampled(gpu, 0, vi, vr, bucket[off:off + numel(shp)], tol, rep)
        for off, v in vec_in:
            got = bucket[off:off + v.numel()]
            if cfg.dtype == "f32":
                assert torch.equal(got, v)
            else:
                exp = (v.float() * inv).half()
                assert torch.equal(got.view(torch.int16), exp.view(torch.int16))
        log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items()))
    return gpu


def test_bert_large_bucket_full_sampled_views():
    cfg = CONFIGS[2]
    # first layer's Q, FFN-in, FFN-out and the last layer's attention output
    log(f"case: {cfg.name} full size, {cfg.steps} steps, sampled views")
    _sampled(cfg, sample_views=[0, 4, 5, 369])


def test_amp_bucket_full_sampled_views_with_inf_step():
    cfg = CONFIGS[4]
    log(f"case: {cfg.name} full size, {cfg.steps} steps (inf at step 10), sampled views")
    _sampled(cfg, sample_views=[0, 4, 5])


def test_gpt_bucket_full_sampled_views():
    cfg = CONFIGS[3]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, sampled views")
    _sampled(cfg, sample_views=[0, 3, 4, 39])


def test_resnet50_bucket_bf16_wrapper_full_every_view_every_step():
    cfg = CONFIGS[6]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, whole-bucket oracle for the first "
        f"{WRAPPED_ORACLE_STEPS}, properties at every step")
    views = cfg.views()
    gen = BucketGenerator(cfg, "cuda")
    hp = dict(cfg.hparams)
    hp["compression_stats_logging_frequency"] = 0
    gpu = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    tol = TOL_WRAPPED[cfg.wrap]
    e_prev = {}
    for step in range(cfg.steps):
        bucket = gen.bucket(step)
        host = bucket.cpu().numpy()
        gpu.compress_bucket_wrapped(bucket, views, cfg.wrap)
        with_oracle = step < WRAPPED_ORACLE_STEPS
        res = orc.compress_bucket_wrapped(host, views, cfg.wrap) if with_oracle else None
        out = bucket.cpu().numpy()
        rep = StepReport(step=step)
        dec = gpu.decisions(0, len(views))
        for vi, (off, shp) in enumerate(views):
            size = numel(shp)
            if not dec[vi]:  # the cast alone: bit-exact with numpy's / torch's
                want = torch.from_numpy(host[off:off + size]).to(torch.bfloat16).float().numpy()
                np.testing.assert_array_equal(out[off:off + size], want)
                continue
            e_prev[vi] = check_wrapped_properties(gpu, 0, vi, cfg.wrap, host[off:off + size],
                                                  e_prev.get(vi), out[off:off + size])
            if with_oracle:
                compare_sampled(gpu, 0, vi, res.views[vi], bucket[off:off + size], tol, rep)
        log(f"  step {step}: " + (", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items())
                                  if with_oracle else "properties hold"))


def _wrapped_properties_torch(gpu, vi, dt, g_in, e_prev, out_view):
    """check_wrapped_properties with torch's casts (round to nearest even) on the device,
    for views too large for the oracle's elementwise rounding: M_hat is 16-bit and
    E = M' - M_hat rounded once, with M' = rnd(rnd(G) + E_prev). Returns E."""
    t16 = torch.float16 if dt == "f16" else torch.bfloat16
    u = 2.0 ** -11 if dt == "f16" else 2.0 ** -8
    n, m, _ = gpu.view_info(0, vi)
    mh = out_view.reshape(n, m)
    assert torch.equal(mh.to(t16).float(), mh), (vi, "M_hat is not 16-bit")
    g16 = g_in.reshape(n, m).to(t16).double()
    mp = (g16 + e_prev).to(torch.float32).to(t16).double() if e_prev is not None else g16
    e = gpu.error(0, vi).double()
    assert bool(torch.all((e - (mp - mh.double())).abs() <= u * e.abs() + 1e-30)), \
        (vi, "E != rnd(M' - M_hat)")
    return e


def _wrapped_sampled(cfg, property_views, oracle_views, oracle_steps):
    """The wrapped hook at full size: the oracle follows oracle_views for the first
    oracle_steps steps; property_views are checked at every step; vectors are the
    16-bit cast and back."""
    views = cfg.views()
    gen = BucketGenerator(cfg, "cuda")
    hp = dict(cfg.hparams)
    hp["compression_stats_logging_frequency"] = 0
    gpu = PowerSGDState(**hp)
    tol = TOL_WRAPPED[cfg.wrap]
    t16 = torch.float16 if cfg.wrap == "f16" else torch.bfloat16
    tracks = {}
    e_prev = {}
    for step in range(cfg.steps):
        bucket = gen.bucket(step)
        g_in = {vi: bucket[off:off + numel(shp)].clone() for vi, (off, shp) in
                enumerate(views) if vi in property_views}
        vec_in = [(off, bucket[off:off + numel(shp)].clone()) for off, shp in views
                  if len(shp) < 2]
        gpu.compress_bucket_wrapped(bucket, views, cfg.wrap)
        torch.cuda.synchronize()
        rep = StepReport(step=step)
        for vi in property_views:
            off, shp = views[vi]
            n, m, r = gpu.view_info(0, vi)
            got = bucket[off:off + numel(shp)]
            e_prev[vi] = _wrapped_properties_torch(gpu, vi, cfg.wrap, g_in[vi],
                                                   e_prev.get(vi), got)
            if step < oracle_steps and vi in oracle_views:
                if vi not in tracks:
                    tracks[vi] = TensorTrackWrapped(hp, vi, n, m, r, cfg.wrap)
                vr = tracks[vi].step(g_in[vi].cpu().double().numpy(), step)
                compare_sampled(gpu, 0, vi, vr, got, tol, rep)
        for off, v in vec_in:  # vectors: the 16-bit cast and back
            got = bucket[off:off + v.numel()]
            assert torch.equal(got, v.to(t16).float())
        log(f"  step {step}: " + (", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items())
                                  if rep.worst else "properties hold"))


def test_bert_large_bucket_fp16_wrapper_full_sampled_views():
    cfg = CONFIGS[7]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, sampled views (oracle for the "
        f"first {WRAPPED_ORACLE_STEPS} steps, properties at every step)")
    _wrapped_sampled(cfg, [0, 4, 5, 369], [0, 4, 5, 369], WRAPPED_ORACLE_STEPS)


def test_gpt_bucket_bf16_wrapper_full_sampled_views():
    """Rank 32 on the 16-bit matrix-core passes at full size (1.48G elements, so the
    16-bit state runs past 2^31 bytes): the oracle follows the first 4096 x 4096 view
    for two steps; the first layer's 16384 x 4096 view and the last view (the bucket's
    end) are checked through the properties at every step."""
    cfg = CONFIGS[8]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, oracle on view 0 for 2 steps, "
        f"properties on views 0, 4, 39")
    _wrapped_sampled(cfg, [0, 4, 39], [0], 2)
