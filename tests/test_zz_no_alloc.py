"""powersgd_compress_matrix_noalloc through the C ABI against powersgd_compress_bucket
on a bucket that holds only the same matrix (rate test off with a rate <= 0): the
same kernels and work items, so P, Q, M_hat and E must be bitwise equal. Two calls in a
row, the second on a smaller matrix (the working array keeps the first call's
contents), then a warm-started step of the second; vector and matrix-core ranks."""
import ctypes

import pytest
import torch

from parity import log
from rank_gradient_compression_amd import PowerSGDState
from rank_gradient_compression_amd import powersgd as api

pytestmark = pytest.mark.gpu


def _hp(rank, eps):
    return dict(matrix_approximation_rank=rank, start_powerSGD_iter=0, min_compression_rate=-1.0,
                use_error_feedback=True, warm_start=True, orthogonalization_epsilon=eps,
                random_seed=9, compression_stats_logging_frequency=0)


def _c_hp(hp):
    c = api.powersgd_hparams_init()
    for k, v in hp.items():
        setattr(c, k, type(getattr(c, k))(v))
    return c


def _noalloc(chp, g, e, q, q_valid, p, bucket_index=3):
    n, m = g.shape
    api.powersgd_compress_matrix_noalloc(chp, bucket_index, 0, 0, g.data_ptr(), n, m,
                                         e.data_ptr(), q.data_ptr(), q_valid, p.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)


def _same(name, a, b):
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)), \
        (name, float((a - b).abs().max()))


@pytest.mark.parametrize("rank,eps,shapes", [
    (4, 0.0, [(700, 900), (300, 130)]),
    (3, 1e-8, [(513, 257), (64, 200)]),
    (32, 1e-8, [(1024, 600), (256, 300)]),
    # matrix-core column groups: three (4616 columns), then two on rows that are not
    # 16-byte multiples (2051 columns)
    (32, 0.0, [(200, 4616), (96, 2051)]),
])
def test_noalloc_matches_the_allocating_entry_point(rank, eps, shapes):
    hp = _hp(rank, eps)
    chp = _c_hp(hp)
    gen = torch.Generator(device="cuda").manual_seed(rank)
    for (n, m) in shapes:
        log(f"case: noalloc vs compress_bucket, {n} x {m}, rank {rank}, eps {eps}")
        r = min(rank, n, m)
        st = PowerSGDState(**hp)
        e = torch.zeros(n, m, device="cuda")
        q = torch.empty(m, r, device="cuda")
        p = torch.empty(n, r, device="cuda")
        for step in range(2):
            g = torch.randn(n, m, device="cuda", generator=gen)
            ref = g.clone().reshape(-1)
            st.compress_bucket(ref, [(0, (n, m))], bucket_index=3)
            _noalloc(chp, g, e, q, step > 0, p)
            torch.cuda.synchronize()
            pr, qr = st.factors(3, 0)
            _same("M_hat", g.reshape(-1), ref)
            _same("E", e, st.error(3, 0))
            _same("P", p, pr)
            _same("Q", q, qr)
            log(f"  step {step}: bitwise equal")
        st.close()


def test_noalloc_without_error_feedback_and_errors():
    hp = _hp(2, 0.0)
    hp["use_error_feedback"] = False
    chp = _c_hp(hp)
    n, m = 200, 300
    g = torch.randn(n, m, device="cuda")
    ref = g.clone().reshape(-1)
    st = PowerSGDState(**hp)
    st.compress_bucket(ref, [(0, (n, m))], bucket_index=0)
    q = torch.empty(m, 2, device="cuda")
    api.powersgd_compress_matrix_noalloc(chp, 0, 0, 0, g.data_ptr(), n, m, None, q.data_ptr(),
                                         False, None, None)
    torch.cuda.synchronize()
    _same("M_hat", g.reshape(-1), ref)
    _same("Q", q, st.factors(0, 0)[1])
    # a matrix beyond the working array is refused before anything is enqueued
    big = _c_hp(_hp(32, 0.0))
    with pytest.raises(api.PowerSGDError) as ei:
        api.powersgd_compress_matrix_noalloc(big, 0, 0, 0, g.data_ptr(), 1 << 21, 1 << 14,
                                             None, q.data_ptr(), False, None, None)
    assert ei.value.status == api.POWERSGD_ERR_UNSUPPORTED
    assert "64 MiB" in api.powersgd_last_error()
    lib = api.load_library()
    assert lib.powersgd_compress_matrix_noalloc(ctypes.byref(big), 0, 0, 0, None, 4, 4, None,
                                                ctypes.c_void_p(q.data_ptr()), 0, None,
                                                None) == api.POWERSGD_ERR_INVALID_ARG
    assert lib.powersgd_compress_matrix_noalloc(
        ctypes.byref(big), 0, 0, 0, ctypes.c_void_p(g.data_ptr() + 2), 4, 4, None,
        ctypes.c_void_p(q.data_ptr()), 0, None, None) == api.POWERSGD_ERR_INVALID_ARG
