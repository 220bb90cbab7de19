"""GPU parity of the wrapped hook (fp16_compress_wrapper / bf16_compress_wrapper around
powerSGD_hook) against the oracle, through the C ABI, element by element.

Tolerance: both sides round every materialized tensor to 16 bits; they differ only in
how the value before each rounding was accumulated (fp32 in the kernels, fp64 in the
oracle), which moves a small fraction of results by one 16-bit ulp. The relative
Frobenius difference of each quantity is held to 4u (u = 2^-11 for binary16, 2^-8 for
bfloat16), E's relative to ||M'|| (it carries M_hat's rounding error, which does not
shrink with E); the cast of uncompressed views is bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL_WRAPPED as TOL
from parity import log, oracle_hparams, rel_fro
from rank_gradient_compression_amd import PowerSGDError, PowerSGDState
from rank_gradient_compression_amd import powersgd as api
from snapshot_format import parse

pytestmark = pytest.mark.gpu

# aligned rows (300 x 260), a conv view, rows of 77 floats (unaligned access), rows of
# 3 floats (scalar access), vectors and a matrix the rate test keeps whole; rows of
# multiples of 8 floats take 8 columns per lane: 97 x 264 (two column blocks, the
# second partial), 400 x 256 (several pass-2 row blocks) and 20 x 40 (narrow)
VIEWS = [(0, (64, 3, 3, 3)), (1728, (64,)), (1792, (4, 4)), (1808, (300, 260)),
         (79808, (130, 77)), (89818, (400, 3)), (91018, (7,)), (91025, (97, 264)),
         (116633, (400, 256)), (219033, (20, 40))]


def _numel(views):
    return max(off + int(np.prod(shp)) for off, shp in views)


def _hp(**kw):
    base = dict(matrix_approximation_rank=2, start_powerSGD_iter=0, min_compression_rate=2.0,
                use_error_feedback=True, warm_start=True, orthogonalization_epsilon=0.0,
                random_seed=3, compression_stats_logging_frequency=0)
    base.update(kw)
    return base


def _bucket(views, step, seed, rank, scale=1.0, decay=None):
    """Per matrix view: a fixed rank-k part (k = max(16, 2r)) with singular-value
    weights 1/j, or decay^j when given, plus fresh N(0, 0.01^2) noise; vectors N(0, 1)."""
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
        w = torch.tensor([1.0 / (j + 1) if decay is None else decay ** j for j in range(k)],
                         dtype=torch.float64)
        out[off:off + size] = ((u * w) @ v.T + 0.01 * torch.randn(
            n, m, generator=gs, dtype=torch.float64)).reshape(-1)
    return (out * scale).float()


def _run(hp, dt, views, steps, seed=0, bucket_index=0, check_factors=True, decay=None,
         factor_scale=1.0):
    """factor_scale widens the bound of the factors P and Q (not of M_hat and E)."""
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    tol = TOL[dt]
    r = hp["matrix_approximation_rank"]
    for t in range(steps):
        x = _bucket(views, t, seed, r, decay=decay)
        dev = x.cuda()
        st.compress_bucket_wrapped(dev, views, dt, bucket_index=bucket_index)
        res = orc.compress_bucket_wrapped(x.numpy(), views, dt, bucket_index=bucket_index)
        torch.cuda.synchronize()
        out = dev.cpu().numpy()
        worst = {}
        if res.passthrough:
            np.testing.assert_array_equal(out, res.output)
            log(f"  step {t}: pass-through cast, bit-exact")
            continue
        dec = st.decisions(bucket_index, len(views))
        assert dec == [int(v.compressed) for v in res.views]
        for vi, ((off, shp), vr) in enumerate(zip(views, res.views)):
            size = int(np.prod(shp))
            if not vr.compressed:
                np.testing.assert_array_equal(out[off:off + size], res.output[off:off + size])
                continue
            n, m, k = st.view_info(bucket_index, vi)
            assert (n, m, k) == (vr.n, vr.m, vr.rank)
            errs = {"Mhat": rel_fro(out[off:off + size].reshape(n, m), vr.m_hat)}
            if check_factors:
                p, q = st.factors(bucket_index, vi)
                p, q = p.double().cpu().numpy(), q.double().cpu().numpy()
                errs["P"] = rel_fro(p, vr.p)
                errs["Q"] = rel_fro(q, vr.q)
                # the factors the library keeps are 16-bit values
                rnd = oracle.round_f16 if dt == "f16" else oracle.round_bf16
                assert np.all(rnd(p) == p) and np.all(rnd(q) == q)
            if vr.error is not None:
                # E = rnd(M' - M_hat) inherits M_hat's rounding error, about u ||M'||
                # whatever ||E|| is, so its difference is measured against ||M'||
                e = st.error(bucket_index, vi).double().cpu().numpy()
                errs["E"] = rel_fro(e, vr.error, np.linalg.norm(vr.m_prime))
            for key, v in errs.items():
                worst[key] = max(worst.get(key, 0.0), v)
                bound = tol * factor_scale if key in ("P", "Q") else tol
                assert v <= bound, (t, vi, key, v, (n, m, k))
        log(f"  step {t}: " + ", ".join(f"{k}={v:.2e}" for k, v in worst.items())
            + f" (tol {tol:.1e})")
    return st, orc


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("rank", [1, 2, 4, 8, 16, 32])
def test_wrapped_parity(dt, rank):
    """Ranks 16 and 32 run the matrix-core passes: at 16 the 300 x 260 view (rows
    16-byte aligned) and the 130 x 77 view (not aligned) are compressed, at 32 the
    300 x 260 view.

    At these ranks the trailing columns of P and Q are ill-conditioned in 16 bits: their
    rounding error is amplified by the gaps between neighbouring singular values, while
    M_hat = P Q^T (the hook's output) is not. The inputs there decay geometrically
    (0.85^j at rank 16, 0.92^j at rank 32: gaps and dynamic range both moderate) and P
    and Q are held to 12u, M_hat and E to 4u. For scale: the same 16-bit steps with
    float32 instead of fp64 products differ from the oracle by up to 2.7u (rank 16)
    and 5.2u (rank 32) in P on these inputs, and by up to 8.2u at rank 16 with 1/j."""
    log(f"case: wrapped hook {dt}, rank {rank}")
    decay = {16: 0.85, 32: 0.92}.get(rank)
    _run(_hp(matrix_approximation_rank=rank), dt, VIEWS, steps=4, seed=rank, decay=decay,
         factor_scale=3.0 if rank >= 16 else 1.0)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("ef,warm", [(False, True), (True, False), (False, False)])
def test_wrapped_parity_without_feedback_or_warm_start(dt, ef, warm):
    log(f"case: wrapped hook {dt}, error feedback {ef}, warm start {warm}")
    _run(_hp(use_error_feedback=ef, warm_start=warm), dt, VIEWS, steps=3, seed=7)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_wrapped_pass_through_and_statistics(dt):
    log(f"case: wrapped hook {dt}, start_powerSGD_iter 2")
    hp = _hp(start_powerSGD_iter=2)
    st, orc = _run(hp, dt, VIEWS, steps=4, seed=11)
    assert st.stats() == (orc.iteration, orc.numel_in, orc.numel_comm)


def test_wrapped_layout_and_argument_errors():
    log("case: wrapped hook errors")
    views = VIEWS
    x = _bucket(views, 0, 1, 2).cuda()
    st = PowerSGDState(**_hp())
    st.compress_bucket_wrapped(x.clone(), views, "f16", bucket_index=0)
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket_wrapped(x.clone(), views, "bf16", bucket_index=0)
    assert ei.value.status == api.POWERSGD_ERR_LAYOUT_CHANGED
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket(x.clone(), views, bucket_index=0)
    assert ei.value.status == api.POWERSGD_ERR_LAYOUT_CHANGED
    lib = api.load_library()
    arr = api.make_views(views)
    assert lib.powersgd_compress_bucket_wrapped(st._state, 5, 1, x.data_ptr(), 0, x.numel(), arr,
                                                len(views), None) == api.POWERSGD_ERR_INVALID_ARG
    with pytest.raises(TypeError):
        st.compress_bucket_wrapped(x.double(), views, "f16")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_wrapped_overflow_propagates_like_the_oracle(dt):
    """Values beyond the 16-bit range become inf in the cast; the compressed view then
    holds non-finite values exactly where the oracle's does."""
    log(f"case: wrapped hook {dt}, overflow in the cast")
    views = [(0, (64, 48)), (3072, (9,))]
    hp = _hp(matrix_approximation_rank=1)
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    x = _bucket(views, 0, 5, 1)
    big = 1e5 if dt == "f16" else 3.4e38  # finite in fp32, beyond the 16-bit range
    x[100] = big
    x[3075] = -big
    dev = x.cuda()
    st.compress_bucket_wrapped(dev, views, dt)
    res = orc.compress_bucket_wrapped(x.numpy(), views, dt)
    out = dev.cpu().numpy()
    np.testing.assert_array_equal(np.isfinite(out), np.isfinite(res.output))
    assert not np.isfinite(out[3075]) and not np.all(np.isfinite(out[:3072]))


@pytest.mark.parametrize("dt,code", [("f16", 1), ("bf16", 2)])
def test_wrapped_snapshot_matches_the_oracle_and_resumes(dt, code):
    log(f"case: snapshot of a wrapped {dt} bucket")
    hp = _hp()
    st, orc = _run(hp, dt, VIEWS, steps=2, seed=13, bucket_index=3, check_factors=False)
    cls_hp = oracle_hparams(hp)

    def cls(shp):
        nm = oracle.matrix_view(shp)
        if nm is None:
            return None
        n, m = nm
        k = oracle.effective_rank(n, m, cls_hp.matrix_approximation_rank)
        return (n, m, k) if oracle.should_compress(n, m, k, cls_hp.min_compression_rate) else None

    blob = bytes(st.export_state())
    head_g, bg = parse(blob, cls)
    head_o, bo = parse(orc.export_state(), cls)
    assert head_g == head_o
    assert bg[0]["variant"] == bo[0]["variant"] == code << 8
    for vi in bg[0]["E"]:
        assert rel_fro(bg[0]["E"][vi], bo[0]["E"][vi]) <= TOL[dt] * 10
        assert rel_fro(bg[0]["Q"][vi], bo[0]["Q"][vi]) <= TOL[dt]
    # resuming from the library's own snapshot is bitwise identical
    b = PowerSGDState(**hp)
    b.import_state(blob)
    assert bytes(b.export_state()) == blob
    x = _bucket(VIEWS, 2, 13, 2).cuda()
    xa, xb = x.clone(), x.clone()
    st.compress_bucket_wrapped(xa, VIEWS, dt, bucket_index=3)
    b.compress_bucket_wrapped(xb, VIEWS, dt, bucket_index=3)
    torch.cuda.synchronize()
    assert torch.equal(xa.view(torch.int32), xb.view(torch.int32))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("rank", [2, 8, 16, 32])
def test_wrapped_error_rebuild_is_bitwise(dt, rank):
    """With error feedback the 16-bit state keeps M' in the error's place and the next
    call rebuilds E = rnd(M' - rnd(P Q^T)) from it. A state that is exported and
    imported after every call holds the error itself and never rebuilds; both must
    produce the same bits: outputs, errors and snapshots (the rows of 260, 77 and 3
    floats take the aligned, unaligned and scalar paths; ranks 16 and 32 the matrix
    cores)."""
    log(f"case: wrapped {dt} rank {rank}, rebuilt error against the imported error")
    hp = _hp(matrix_approximation_rank=rank)
    decay = {16: 0.85, 32: 0.92}.get(rank)
    a = PowerSGDState(**hp)
    b = PowerSGDState(**hp)
    for t in range(4):
        x = _bucket(VIEWS, t, 40 + rank, rank, decay=decay).cuda()
        xa, xb = x.clone(), x.clone()
        a.compress_bucket_wrapped(xa, VIEWS, dt, bucket_index=2)
        b.compress_bucket_wrapped(xb, VIEWS, dt, bucket_index=2)
        torch.cuda.synchronize()
        assert torch.equal(xa.view(torch.int32), xb.view(torch.int32)), t
        blob = bytes(b.export_state())
        b = PowerSGDState(**hp)
        b.import_state(blob)
        # a materializes its error from M'; b widens the 16-bit error it imported
        for vi in range(len(VIEWS)):
            try:
                ea = a.error(2, vi)
            except PowerSGDError:
                continue  # not compressed
            assert torch.equal(ea.view(torch.int32), b.error(2, vi).view(torch.int32)), (t, vi)
        assert bytes(a.export_state()) == blob, t
    log("  4 calls: outputs, errors and snapshots bitwise identical")


# ------------------------------------------ the wrappers around batched_powerSGD_hook

@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("numel,rank", [(5000, 2), (16284, 4), (22400, 16), (22500, 32)])
def test_batched_wrapped_parity_and_resume(dt, numel, rank):
    """The bucket cast to 16 bits and viewed as one zero-padded s x s matrix. The
    padding is NaN before every call (the library must zero it); ranks 16 and 32 use
    the geometric inputs and the factor bound of test_wrapped_parity."""
    s = oracle.batched_side(numel)
    log(f"case: batched wrapped hook {dt}, numel {numel} -> {s} x {s}, rank {rank}")
    hp = _hp(matrix_approximation_rank=rank)
    st = PowerSGDState(**hp)
    orc = oracle.OracleState(oracle_hparams(hp))
    tol = TOL[dt]
    fscale = 3.0 if rank >= 16 else 1.0
    decay = {16: 0.85, 32: 0.92}.get(rank)
    rnd = oracle.round_f16 if dt == "f16" else oracle.round_bf16
    buf = torch.empty(s * s, device="cuda")
    for t in range(3):
        x = _bucket([(0, (s, s))], t, numel, rank, decay=decay)[:numel].contiguous()
        buf[numel:].fill_(float("nan"))
        buf[:numel].copy_(x.cuda())
        st.compress_bucket_batched_wrapped(buf, dt, numel=numel)
        res = orc.compress_bucket_batched_wrapped(x.numpy(), dt)
        torch.cuda.synchronize()
        vr = res.views[0]
        assert st.view_info(0, 0) == (s, s, vr.rank)
        out = buf[:numel].double().cpu().numpy()
        assert np.all(rnd(out) == out)
        p, q = st.factors(0, 0)
        e = st.error(0, 0).double().cpu().numpy()
        errs = {"out": rel_fro(out, res.output64),
                "P": rel_fro(p.double().cpu().numpy(), vr.p),
                "Q": rel_fro(q.double().cpu().numpy(), vr.q),
                "E": rel_fro(e, vr.error, np.linalg.norm(vr.m_prime))}
        for k, v in errs.items():
            assert v <= (tol * fscale if k in ("P", "Q") else tol), (t, k, v)
        log(f"  step {t}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert st.stats() == (orc.iteration, orc.numel_in, orc.numel_comm)
    # resume from the library's own snapshot: bitwise
    blob = bytes(st.export_state())
    b = PowerSGDState(**hp)
    b.import_state(blob)
    assert bytes(b.export_state()) == blob
    x = _bucket([(0, (s, s))], 3, numel, rank, decay=decay)[:numel].contiguous().cuda()
    bufs = [torch.zeros(s * s, device="cuda") for _ in range(2)]
    for bb, state in zip(bufs, (st, b)):
        bb[:numel].copy_(x)
        state.compress_bucket_batched_wrapped(bb, dt, numel=numel)
    torch.cuda.synchronize()
    assert torch.equal(bufs[0][:numel].view(torch.int32), bufs[1][:numel].view(torch.int32))


def test_batched_wrapped_errors():
    log("case: batched wrapped hook errors")
    st = PowerSGDState(**_hp())
    x = torch.zeros(100, device="cuda")
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket_batched_wrapped(x, "f16", numel=101)   # 11 x 11 > 100
    assert ei.value.status == api.POWERSGD_ERR_INVALID_ARG
    st.compress_bucket_batched_wrapped(x, "f16", numel=90)
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket_batched_wrapped(x, "bf16", numel=90)
    assert ei.value.status == api.POWERSGD_ERR_LAYOUT_CHANGED
    with pytest.raises(PowerSGDError) as ei:
        st.compress_bucket_batched(x, numel=90)
    assert ei.value.status == api.POWERSGD_ERR_LAYOUT_CHANGED
    with pytest.raises(TypeError):
        st.compress_bucket_batched_wrapped(x.half(), "f16")
