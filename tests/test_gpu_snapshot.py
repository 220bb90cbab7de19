"""GPU tests of the state snapshot (powersgd_state_export / powersgd_state_import)
through the C ABI: the library's snapshot against the oracle's after the same steps,
a library state resumed from an oracle snapshot against the oracle resumed from it,
bitwise resumption from the library's own snapshot, rejection of malformed snapshots,
and the statistics of skipped fp16 calls."""
import struct

import numpy as np
import pytest
import torch

import oracle
from parity import TOL, BucketParity, log, oracle_hparams, rel_fro
from rank_gradient_compression_amd import PowerSGDError, PowerSGDState
from rank_gradient_compression_amd import powersgd as api
from snapshot_format import parse

pytestmark = pytest.mark.gpu

# per-layer bucket: a conv view, a vector, a matrix the rate test keeps whole, a
# 16-byte-aligned matrix and one with rows of 77 floats (unaligned row access)
VIEWS_SMALL_R = [(0, (64, 3, 3, 3)), (1728, (64,)), (1792, (4, 4)), (1808, (300, 260)),
                 (79808, (130, 77))]
# matrix-core ranks: views wide enough to compress at r = 32
VIEWS_LARGE_R = [(0, (256, 300)), (76800, (16,)), (76816, (200, 130)), (102816, (96, 97))]
BATCHED_NUMEL = 5000  # 71 x 71


def _numel(views):
    return max(off + int(np.prod(shp)) for off, shp in views)


def _hp(**kw):
    base = dict(matrix_approximation_rank=2, start_powerSGD_iter=0, min_compression_rate=2.0,
                use_error_feedback=True, warm_start=True, orthogonalization_epsilon=0.0,
                random_seed=11, compression_stats_logging_frequency=0)
    base.update(kw)
    return base


def _bucket(views, step, seed, rank):
    """Per view: a rank-k signal with a 1/j spectrum (k = max(16, 2r), fixed per view)
    plus fresh N(0, 0.01^2) noise per step; vectors are fresh N(0, 1)."""
    out = torch.zeros(_numel(views), dtype=torch.float64)
    k = max(16, 2 * rank)
    for vi, (off, shp) in enumerate(views):
        size = int(np.prod(shp))
        gs = torch.Generator().manual_seed(seed * 7919 + step * 131 + vi)
        if len(shp) < 2:
            out[off:off + size] = torch.randn(size, generator=gs, dtype=torch.float64)
            continue
        n, m = shp[0], size // shp[0]
        g = torch.Generator().manual_seed(seed * 104729 + vi)
        u = torch.randn(n, k, generator=g, dtype=torch.float64)
        v = torch.randn(m, k, generator=g, dtype=torch.float64)
        w = torch.tensor([1.0 / (j + 1) for j in range(k)], dtype=torch.float64)
        sig = (u * w) @ v.T
        out[off:off + size] = (sig + 0.01 * torch.randn(n, m, generator=gs,
                                                       dtype=torch.float64)).reshape(-1)
    return out.float()


def _batched_bucket(numel, step, seed, rank):
    """The first numel entries of an s x s low-rank-plus-noise matrix."""
    s = oracle.batched_side(numel)
    return _bucket([(0, (s, s))], step, seed, rank)[:numel].contiguous()


def _classify(hp):
    ohp = oracle_hparams(hp)

    def cls(shp):
        nm = oracle.matrix_view(shp)
        if nm is None:
            return None
        n, m = nm
        k = oracle.effective_rank(n, m, ohp.matrix_approximation_rank)
        return (n, m, k) if oracle.should_compress(n, m, k, ohp.min_compression_rate) else None
    return cls


def _run_both(hp, views, steps, seed, gpu=None, orc=None):
    """`steps` calls of bucket 1 (per layer) and bucket 4 (batched) on both sides."""
    r = hp["matrix_approximation_rank"]
    gpu = gpu or PowerSGDState(**hp)
    orc = orc or oracle.OracleState(oracle_hparams(hp))
    s = oracle.batched_side(BATCHED_NUMEL)
    buf = torch.zeros(s * s, device="cuda")
    last = {}
    for t in range(steps):
        b = _bucket(views, t, seed, r)
        dev = b.cuda()
        gpu.compress_bucket(dev, views, bucket_index=1)
        last[1] = orc.compress_bucket(b.numpy(), views, bucket_index=1)
        bb = _batched_bucket(BATCHED_NUMEL, t, seed + 1, r)
        buf[:BATCHED_NUMEL].copy_(bb.cuda())
        gpu.compress_bucket_batched(buf, numel=BATCHED_NUMEL, bucket_index=4)
        last[4] = orc.compress_bucket_batched(bb.numpy(), bucket_index=4)
    torch.cuda.synchronize()
    return gpu, orc, last


CASES = [
    ("r2 ef warm", VIEWS_SMALL_R, dict()),
    ("r2 ef, no warm start", VIEWS_SMALL_R, dict(warm_start=False)),
    ("r2 warm, no ef", VIEWS_SMALL_R, dict(use_error_feedback=False)),
    ("r8", VIEWS_SMALL_R, dict(matrix_approximation_rank=8)),
    ("r32 matrix cores", VIEWS_LARGE_R, dict(matrix_approximation_rank=32,
                                             orthogonalization_epsilon=1e-8)),
]


@pytest.mark.parametrize("name,views,kw", CASES, ids=[c[0] for c in CASES])
def test_export_matches_the_oracle(name, views, kw):
    log(f"case: export after 3 steps, {name}")
    hp = _hp(**kw)
    gpu, orc, last = _run_both(hp, views, 3, seed=5)
    head_g, bk_g = parse(gpu.export_state(), _classify(hp))
    head_o, bk_o = parse(orc.export_state(), _classify(hp))
    assert head_g == head_o
    assert len(bk_g) == len(bk_o) == 2
    for bg, bo in zip(bk_g, bk_o):
        for key in ("index", "numel", "variant", "has_q", "views"):
            assert bg[key] == bo[key], key
        assert sorted(bg["E"]) == sorted(bo["E"]) and sorted(bg["Q"]) == sorted(bo["Q"])
        res = last[bg["index"]]
        for vi, e in bg["E"].items():
            vr = res.views[vi]
            ne, nm = np.linalg.norm(vr.error), np.linalg.norm(vr.m_prime)
            err = rel_fro(e, bo["E"][vi], nm if ne < 1e-3 * nm else None)
            assert err <= TOL["f32"], (bg["index"], vi, "E", err)
        for vi, q in bg["Q"].items():
            err = rel_fro(q, bo["Q"][vi])
            assert err <= TOL["f32"], (bg["index"], vi, "Q", err)
        log(f"  bucket {bg['index']}: {len(bg['E'])} E, {len(bg['Q'])} Q within {TOL['f32']}")


@pytest.mark.parametrize("name,views,kw", [CASES[0], CASES[1], CASES[4]],
                         ids=[CASES[i][0] for i in (0, 1, 4)])
def test_resume_from_an_oracle_snapshot(name, views, kw):
    log(f"case: library resumed from the oracle's snapshot, {name}")
    hp = _hp(**kw)
    r = hp["matrix_approximation_rank"]
    first = oracle.OracleState(oracle_hparams(hp))
    for t in range(3):
        first.compress_bucket(_bucket(views, t, 9, r).numpy(), views, bucket_index=1)
    blob = first.export_state()
    par = BucketParity(hp, views, bucket_index=1)
    par.oracle.import_state(blob)
    par.gpu.import_state(blob)
    assert par.gpu.stats() == (first.iteration, first.numel_in, first.numel_comm)
    for t in range(3, 6):
        rep = par.step(_bucket(views, t, 9, r), t)
        log(f"  step {t}: " + ", ".join(f"{k}={v:.2e}" for k, v in rep.worst.items()))
    assert par.gpu.stats() == (par.oracle.iteration, par.oracle.numel_in,
                               par.oracle.numel_comm)


@pytest.mark.parametrize("name,views,kw", [CASES[0], CASES[2], CASES[4]],
                         ids=[CASES[i][0] for i in (0, 2, 4)])
def test_resume_from_an_own_snapshot_is_bitwise(name, views, kw):
    log(f"case: library resumed from its own snapshot, {name}")
    hp = _hp(**kw)
    r = hp["matrix_approximation_rank"]
    a, _, _ = _run_both(hp, views, 2, seed=21)
    blob = a.export_state()
    b = PowerSGDState(**hp)
    b.import_state(blob)
    assert b.export_state() == blob
    s = oracle.batched_side(BATCHED_NUMEL)
    bufs = [torch.zeros(s * s, device="cuda") for _ in range(2)]
    for t in range(2, 5):
        g = _bucket(views, t, 21, r).cuda()
        ga, gb = g.clone(), g.clone()
        a.compress_bucket(ga, views, bucket_index=1)
        b.compress_bucket(gb, views, bucket_index=1)
        bb = _batched_bucket(BATCHED_NUMEL, t, 22, r).cuda()
        for buf, st in zip(bufs, (a, b)):
            buf[:BATCHED_NUMEL].copy_(bb)
            st.compress_bucket_batched(buf, numel=BATCHED_NUMEL, bucket_index=4)
        torch.cuda.synchronize()
        assert torch.equal(ga.view(torch.int32), gb.view(torch.int32)), t
        assert torch.equal(bufs[0][:BATCHED_NUMEL].view(torch.int32),
                           bufs[1][:BATCHED_NUMEL].view(torch.int32)), t
    assert a.export_state() == b.export_state()
    log("  3 more steps bitwise identical, snapshots identical")


def test_malformed_snapshots_leave_the_state_unchanged():
    log("case: malformed snapshots are rejected")
    hp = _hp()
    a, _, _ = _run_both(hp, VIEWS_SMALL_R, 1, seed=3)
    blob = bytes(a.export_state())
    b, _, _ = _run_both(hp, VIEWS_SMALL_R, 2, seed=4)
    before = bytes(b.export_state())

    def put(pos, fmt, value):
        x = bytearray(blob)
        struct.pack_into(fmt, x, pos, value)
        return bytes(x)

    bad = [b"XSGDSNAP" + blob[8:], put(8, "<I", 2), put(12, "<I", 1), put(16, "<i", 3),
           put(20, "<I", 1), put(24, "<d", 2.5), put(32, "<Q", 12), put(40, "<q", -1),
           put(72, "<q", 3), put(80 + 8, "<q", 10), put(80 + 16, "<I", 2), blob[:-1],
           blob + b"\0", blob[:79]]
    for i, data in enumerate(bad):
        with pytest.raises(PowerSGDError) as ei:
            b.import_state(data)
        assert ei.value.status == api.POWERSGD_ERR_INVALID_ARG, i
        assert bytes(b.export_state()) == before, i
    # other hyperparameters
    c = PowerSGDState(**_hp(matrix_approximation_rank=4))
    with pytest.raises(PowerSGDError):
        c.import_state(blob)
    # an empty state exports a bare header that imports everywhere alike
    e = PowerSGDState(**hp)
    empty = bytes(e.export_state())
    assert len(empty) == 80 and empty[:8] == b"PSGDSNAP"
    b.import_state(empty)
    assert b.stats() == (0, 0, 0)
    with pytest.raises(PowerSGDError) as ei:
        b.error(1, 0)
    assert ei.value.status == api.POWERSGD_ERR_NOT_FOUND


def test_skipped_fp16_calls_count_in_the_statistics():
    log("case: statistics of skipped fp16 calls")
    hp = _hp(start_powerSGD_iter=1)
    par = BucketParity(hp, VIEWS_SMALL_R, dtype="f16", bucket_index=1)
    base = _bucket(VIEWS_SMALL_R, 0, 2, 2) * (2.0 ** -10) * 1024.0
    for t, inf in enumerate([True, True, False, True, False]):
        b = (base * 1.0).half()
        if inf:
            b[1800] = float("inf")
        par.step(b, t, inv_loss_scale=1.0 / 1024.0)
        assert par.gpu.stats() == (par.oracle.iteration, par.oracle.numel_in,
                                   par.oracle.numel_comm), t
    log(f"  stats {par.gpu.stats()}")
