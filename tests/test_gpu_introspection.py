"""The boundary's introspection calls through the C ABI on the GPU: the raw initial Q
draw against the oracle's generator bit for bit, and powersgd_get_factors /
powersgd_get_error (state-owned device pointers) against the copies the other
introspection calls make and against the layout the header states."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity import device_to_tensor, log, numel
from rank_gradient_compression_amd import PowerSGDState
from rank_gradient_compression_amd import powersgd as api
from synthetic import packed_views

pytestmark = pytest.mark.gpu

# (m, rank, random_seed, bucket_index, view, epoch): ragged counts (m * rank not a
# multiple of 4), all-ones and top-bit keys and counters, the ranks the workloads use
DRAWS = [
    (1, 1, 0, 0, 0, 0),
    (3, 3, 0, 0, 0, 0),
    (512, 1, 0, 0, 0, 0),
    (2048, 2, 0, 3, 17, 0),
    (1024, 4, 1234567, 7, 95, 0),
    (4096, 32, 0, 0, 39, 0),
    (16384, 32, 2 ** 64 - 1, 2 ** 63 - 1, 2 ** 31 - 1, 2 ** 64 - 1),
    (777, 5, 2 ** 63, 1, 2, 41),
]


@pytest.mark.parametrize("m,rank,seed,bucket,view,epoch", DRAWS)
def test_initial_q_draw_is_bit_exact_with_the_oracle(m, rank, seed, bucket, view, epoch):
    log(f"case: raw Q draw m={m} rank={rank} seed={seed} bucket={bucket} view={view} "
        f"epoch={epoch}")
    count = m * rank
    nwords = 4 * ((count + 3) // 4)
    out = torch.empty(count, dtype=torch.float32, device="cuda")
    words = torch.empty(nwords, dtype=torch.int64, device="cuda")
    api.powersgd_draw_q0(seed, bucket, view, epoch, m, rank, out.data_ptr(), words.data_ptr(),
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # the integer stream: Philox4x64-10 words of counters (b, view, epoch, 0)
    nb = nwords // 4
    mask = 0xFFFFFFFFFFFFFFFF
    w = oracle.philox4x64_10(np.arange(nb, dtype=np.uint64), np.uint64(view & mask),
                             np.uint64(epoch & mask), np.uint64(0), np.uint64(seed & mask),
                             np.uint64(bucket & mask))
    want_words = np.stack(w, axis=1).reshape(-1)
    got_words = words.cpu().numpy().view(np.uint64)
    assert np.array_equal(got_words, want_words)
    # the binary32 values, bit for bit
    want = oracle.standard_normal_q0(m, rank, seed, bucket, view, epoch).astype(np.float32)
    got = out.cpu().numpy().reshape(m, rank)
    diff = np.count_nonzero(got.view(np.uint32) != want.view(np.uint32))
    assert diff == 0, f"{diff} of {count} values differ"


def test_initial_q_draw_without_words_and_empty():
    out = torch.full((12,), -1.0, device="cuda")
    api.powersgd_draw_q0(5, 1, 2, 0, 4, 3, out.data_ptr(), None, None)
    torch.cuda.synchronize()
    want = oracle.standard_normal_q0(4, 3, 5, 1, 2, 0).astype(np.float32).reshape(-1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
    api.powersgd_draw_q0(5, 1, 2, 0, 0, 3, 0, None, None)  # m = 0: nothing to draw


def _hp(**kw):
    base = dict(matrix_approximation_rank=3, start_powerSGD_iter=0, min_compression_rate=0.5,
                use_error_feedback=True, warm_start=True, orthogonalization_epsilon=0.0,
                random_seed=0, compression_stats_logging_frequency=0)
    base.update(kw)
    return base


def _raw_factors(st, bucket_index, view):
    lib = api.load_library()
    p, q = ctypes.c_void_p(), ctypes.c_void_p()
    n, m, r = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    rc = lib.powersgd_get_factors(st._state, bucket_index, view, ctypes.byref(p), ctypes.byref(q),
                                  ctypes.byref(n), ctypes.byref(m), ctypes.byref(r))
    assert rc == api.POWERSGD_OK, api.powersgd_last_error()
    return (device_to_tensor(p.value, (n.value, r.value), torch.float32),
            device_to_tensor(q.value, (m.value, r.value), torch.float32), n.value, m.value,
            r.value)


def _raw_error(st, bucket_index, length):
    lib = api.load_library()
    e = ctypes.c_void_p()
    rc = lib.powersgd_get_error(st._state, bucket_index, ctypes.byref(e))
    assert rc == api.POWERSGD_OK, api.powersgd_last_error()
    return device_to_tensor(e.value, (length,), torch.float32)


def test_get_factors_and_get_error_per_layer():
    log("case: get_factors / get_error through the C ABI (rank 3 padded to 4, views "
        "with fewer columns than the rank, vectors in between)")
    shapes = [(40, 30), (7,), (64, 2), (33, 17, 2), (5,), (90, 120)]
    views = packed_views(shapes)
    total = sum(numel(s) for s in shapes)
    st = PowerSGDState(**_hp())
    g = torch.Generator().manual_seed(3)
    for step in range(2):
        b = torch.randn(total, generator=g).cuda()
        st.compress_bucket(b, views, bucket_index=5)
    torch.cuda.synchronize()
    dec = st.decisions(5, len(views))
    e_all = _raw_error(st, 5, total)
    for vi, (off, shp) in enumerate(views):
        size = numel(shp)
        if not dec[vi]:
            assert torch.count_nonzero(e_all[off:off + size]).item() == 0, vi
            with pytest.raises(api.PowerSGDError):
                api.powersgd_get_factors(st._state, 5, vi)
            continue
        p, q, n, m, r = _raw_factors(st, 5, vi)
        assert (n, m, r) == st.view_info(5, vi)
        pc, qc = st.factors(5, vi)
        assert torch.equal(p, pc) and torch.equal(q, qc), vi
        assert torch.equal(e_all[off:off + size].reshape(n, m), st.error(5, vi)), vi
    # a second get_factors of the same view refreshes the same memory
    p1 = api.powersgd_get_factors(st._state, 5, 0)
    p2 = api.powersgd_get_factors(st._state, 5, 0)
    assert p1 == p2
    with pytest.raises(api.PowerSGDError) as ei:
        api.powersgd_get_error(st._state, 99)
    assert ei.value.status == api.POWERSGD_ERR_NOT_FOUND


def test_get_error_batched_and_wrapped_and_without_error_feedback():
    log("case: get_error of the batched variant (s x s), of a 16-bit state, and without "
        "error feedback")
    numel_b = 1000
    side = api.powersgd_batched_side(numel_b)
    st = PowerSGDState(**_hp(matrix_approximation_rank=2))
    buf = torch.zeros(side * side, device="cuda")
    buf[:numel_b] = torch.randn(numel_b, generator=torch.Generator().manual_seed(4)).cuda()
    st.compress_bucket_batched(buf, numel=numel_b, bucket_index=1)
    e = _raw_error(st, 1, side * side)
    assert torch.equal(e.reshape(side, side), st.error(1, 0))
    p, q, n, m, r = _raw_factors(st, 1, 0)
    assert (n, m, r) == (side, side, 2)

    shapes = [(64, 48), (16,), (32, 80)]
    views = packed_views(shapes)
    total = sum(numel(s) for s in shapes)
    st2 = PowerSGDState(**_hp(matrix_approximation_rank=2))
    b = torch.randn(total, generator=torch.Generator().manual_seed(5)).cuda()
    st2.compress_bucket_wrapped(b, views, "bf16", bucket_index=2)
    e2 = _raw_error(st2, 2, total)
    for vi, (off, shp) in enumerate(views):
        size = numel(shp)
        if len(shp) < 2:
            assert torch.count_nonzero(e2[off:off + size]).item() == 0
            continue
        got = e2[off:off + size].reshape(shp)
        assert torch.equal(got, st2.error(2, vi))
        assert torch.equal(got.to(torch.bfloat16).float(), got)  # 16-bit values, widened

    st3 = PowerSGDState(**_hp(use_error_feedback=False))
    b3 = torch.randn(total, generator=torch.Generator().manual_seed(6)).cuda()
    st3.compress_bucket(b3, views, bucket_index=0)
    with pytest.raises(api.PowerSGDError) as ei:
        api.powersgd_get_error(st3._state, 0)
    assert ei.value.status == api.POWERSGD_ERR_NOT_FOUND
    p, q, n, m, r = _raw_factors(st3, 0, 0)  # factors exist without error feedback
    assert (n, m, r) == (64, 48, 3)
