"""GPU parity at the benchmark workloads' full sizes, with the benchmark's own
plans (same views, hyperparameters, launch configuration) and inputs generated on
the GPU. The ResNet-50-shaped bucket is compared whole against the oracle; for the
larger buckets the oracle follows a sample of views (one per shape, plus the last
layer's) through every step with its own per-matrix functions, and every compressed
view is checked at every step through properties that hold at any size: M_hat + E_new
= G + E_prev on the library's own state, vectors untouched (fp16: unscaled)."""
import numpy as np
import pytest
import torch

import oracle
from parity import (TOL, TOL_WRAPPED, WRAPPED_ORACLE_STEPS, BucketParity, StepReport,
                    TensorTrack, TensorTrackWrapped, check_wrapped_properties, compare_sampled,
                    device_to_tensor, log, numel, oracle_hparams, rel_fro)
from rank_gradient_compression_amd import PowerSGDState
from rank_gradient_compression_amd import powersgd as api
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


def _bucket_error(gpu, length):
    """The library's bucket-shaped error memory (powersgd_get_error), copied."""
    return device_to_tensor(api.powersgd_get_error(gpu._state, 0), (length,), torch.float32)


def _check_identity(views, dec, g_in, e_prev, out, e_new, inv, f16, step):
    """Every compressed view: M_hat + E_new = M' with M' = G + E_prev (the error-feedback
    identity; "PowerSGD Hooks", first warning), up to the rounding of the two fp32
    operations that form M' and E_new (and of the fp16 output cast). Returns the worst
    relative residual."""
    worst = 0.0
    u32 = 2.0 ** -24
    for vi, (off, shp) in enumerate(views):
        if not dec[vi]:
            continue
        size = numel(shp)
        g = g_in[off:off + size].double() * inv
        mp = g + e_prev[off:off + size].double()
        o = out[off:off + size].double()
        en = e_new[off:off + size].double()
        res = float((o + en - mp).norm())
        nmp, nen, no = float(mp.norm()), float(en.norm()), float(o.norm())
        bound = 2 * u32 * (nmp + nen) + (2.0 ** -11 * no if f16 else 0.0)
        assert res <= bound, (step, vi, res, bound, nmp)
        worst = max(worst, res / max(nmp, 1e-300))
    return worst


def _sampled(cfg, sample_views, steps=None):
    """The oracle follows sample_views through every step; every other compressed view
    is held at every step to the error-feedback identity on the library's own state
    (bucket-shaped E before and after the call)."""
    views = cfg.views()
    gen = BucketGenerator(cfg, "cuda")
    hp = dict(cfg.hparams)
    hp["compression_stats_logging_frequency"] = 0
    gpu = PowerSGDState(**hp)
    tracks = {}
    tol = TOL[cfg.dtype]
    scale = cfg.loss_scale
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    f16 = cfg.dtype == "f16"
    e_prev = torch.zeros(cfg.numel, dtype=torch.float32, device="cuda")
    for step in range(cfg.steps if steps is None else steps):
        if f16:
            bucket = gen.bucket(step, loss_scale=scale)
            inv = 1.0 / scale
        else:
            bucket = gen.bucket(step)
            inv = 1.0
        g_in = bucket.clone()
        host_in = {vi: bucket[off:off + numel(shp)].cpu() for vi, (off, shp) in
                   enumerate(views) if vi in sample_views}
        vec_in = [(off, bucket[off:off + numel(shp)].clone()) for off, shp in views
                  if len(shp) < 2]
        inf = False
        if f16:
            inf = oracle.any_nonfinite(bucket.cpu().numpy(), views)
        found.zero_()
        gpu.compress_bucket(bucket, views, inv_loss_scale=inv,
                            found_inf=found if f16 else None)
        torch.cuda.synchronize()
        rep = StepReport(step=step, found_inf=inf)
        if f16:
            assert bool(found.item()) == inf, step
        if inf:
            assert torch.equal(bucket.view(torch.int16), g_in.view(torch.int16)), step
            if step > 0:
                assert torch.equal(_bucket_error(gpu, cfg.numel), e_prev), (step, "E changed")
            log(f"  step {step}: inf found, skipped (bucket and E unchanged)")
            scale *= 0.5
            continue
        e_new = _bucket_error(gpu, cfg.numel)
        dec = gpu.decisions(0, len(views))
        ident = _check_identity(views, dec, g_in, e_prev, bucket, e_new, inv, f16, step)
        e_prev = e_new
        del g_in
        for vi in sample_views:
            off, shp = views[vi]
            n, m, r = gpu.view_info(0, vi)
            if vi not in tracks:
                tracks[vi] = TensorTrack(hp, vi, n, m, r)
            g = host_in[vi].double().numpy()
            if f16:
                g = g * inv
            vr = tracks[vi].step(g, step)
            compare_sampled(gpu, 0, vi, vr, bucket[off:off + numel(shp)], tol, rep)
        for off, v in vec_in:
            got = bucket[off:off + v.numel()]
            if not f16:
                assert torch.equal(got, v)
            else:
                exp = (v.float() * inv).half()
                assert torch.equal(got.view(torch.int16), exp.view(torch.int16))
        log(f"  step {step}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items())
            + f", identity on all {sum(dec)} matrices <= {ident:.1e}")
    return gpu


def test_bert_large_bucket_full_sampled_views():
    cfg = CONFIGS[2]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, sampled views")
    # one view per shape (first layer) and the last layer's FFN-out matrix
    _sampled(cfg, sample_views=[0, 4, 5, 373])


def test_amp_bucket_full_sampled_views_with_inf_step():
    cfg = CONFIGS[4]
    log(f"case: {cfg.name} full size, {cfg.steps} steps (inf at step 10), sampled views")
    _sampled(cfg, sample_views=[0, 4, 5, 373])


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


def _wrapped_sampled(cfg, oracle_views, oracle_steps):
    """The wrapped hook at full size: the oracle follows oracle_views for the first
    oracle_steps steps; every compressed view is checked through the properties at every
    step; vectors are the 16-bit cast and back."""
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
        g_all = bucket.clone()
        vec_in = [(off, bucket[off:off + numel(shp)].clone()) for off, shp in views
                  if len(shp) < 2]
        gpu.compress_bucket_wrapped(bucket, views, cfg.wrap)
        torch.cuda.synchronize()
        rep = StepReport(step=step)
        dec = gpu.decisions(0, len(views))
        for vi, (off, shp) in enumerate(views):
            if not dec[vi]:
                continue
            n, m, r = gpu.view_info(0, vi)
            got = bucket[off:off + numel(shp)]
            g_in = g_all[off:off + numel(shp)]
            e_prev[vi] = _wrapped_properties_torch(gpu, vi, cfg.wrap, g_in, e_prev.get(vi), got)
            if step < oracle_steps and vi in oracle_views:
                if vi not in tracks:
                    tracks[vi] = TensorTrackWrapped(hp, vi, n, m, r, cfg.wrap)
                vr = tracks[vi].step(g_in.cpu().double().numpy(), step)
                compare_sampled(gpu, 0, vi, vr, got, tol, rep)
        del g_all
        for off, v in vec_in:  # vectors: the 16-bit cast and back
            got = bucket[off:off + v.numel()]
            assert torch.equal(got, v.to(t16).float())
        log(f"  step {step}: " + (", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items())
                                  if rep.worst else "")
            + f" properties hold on all {sum(dec)} matrices")


def test_bert_large_bucket_fp16_wrapper_full_sampled_views():
    cfg = CONFIGS[7]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, oracle on one view per shape and "
        f"the last layer's for the first {WRAPPED_ORACLE_STEPS} steps, properties on every "
        f"matrix at every step")
    _wrapped_sampled(cfg, [0, 4, 5, 373], WRAPPED_ORACLE_STEPS)


def test_gpt_bucket_bf16_wrapper_full_sampled_views():
    """Rank 32 on the 16-bit matrix-core passes at full size (1.48G elements, so the
    16-bit state runs past 2^31 bytes): the oracle follows one view of each shape (4096 x
    4096, 4096 x 16384, 16384 x 4096) for the first steps; every matrix is checked
    through the properties at every step."""
    cfg = CONFIGS[8]
    log(f"case: {cfg.name} full size, {cfg.steps} steps, oracle on views 0, 3, 4 for "
        f"{WRAPPED_ORACLE_STEPS} steps, properties on every matrix")
    _wrapped_sampled(cfg, [0, 3, 4], WRAPPED_ORACLE_STEPS)
