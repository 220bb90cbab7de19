"""Steady-state calls replayed from a HIP graph.

After a bucket's first call (which allocates its memory and uploads its work tables),
a call enqueues only kernel launches on the caller's stream, so it can be captured
and replayed. A replay runs the kernels with the arguments of the capture: with warm
start (no per-iteration draw) every replay is one more step; the host's iteration and
statistics counters advance only when the host calls. Each replay is compared
bitwise with the same steps run eagerly on a second state, with eager work and
synchronizations between the replays."""
import numpy as np
import pytest
import torch

from parity import log
from rank_gradient_compression_amd import PowerSGDState

pytestmark = pytest.mark.gpu

VIEWS = [(0, (64, 3, 3, 3)), (1728, (64,)), (1792, (300, 260)), (79792, (130, 77)),
         (89802, (97, 264))]
NUMEL = 89802 + 97 * 264


def _inputs(steps, seed):
    g = torch.Generator().manual_seed(seed)
    base = torch.randn(NUMEL, generator=g)
    return [(base + 0.05 * torch.randn(NUMEL, generator=g)).cuda() for _ in range(steps)]


CASES = [("rank 2", 2, None), ("rank 32 (matrix cores)", 32, None), ("rank 4, bf16 wrapper", 4, "bf16")]


@pytest.mark.parametrize("name,rank,wrap", CASES, ids=[c[0] for c in CASES])
def test_steady_state_call_replays_bitwise(name, rank, wrap):
    log(f"case: graph replay, {name}")
    hp = dict(matrix_approximation_rank=rank, start_powerSGD_iter=0, warm_start=True,
              use_error_feedback=True, orthogonalization_epsilon=1e-8 if rank > 8 else 0.0,
              compression_stats_logging_frequency=0)
    a, b = PowerSGDState(**hp), PowerSGDState(**hp)
    xs = _inputs(6, rank)
    buf_a = torch.empty(NUMEL, device="cuda")
    buf_b = torch.empty(NUMEL, device="cuda")

    def call(st, buf, stream=None):
        if wrap:
            st.compress_bucket_wrapped(buf, VIEWS, wrap, stream=stream)
        else:
            st.compress_bucket(buf, VIEWS, stream=stream)

    for st, buf in ((a, buf_a), (b, buf_b)):  # first call: allocation and tables
        buf.copy_(xs[0])
        call(st, buf)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    buf_a.copy_(xs[1])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        call(a, buf_a, stream=s)
    for t in range(1, 6):
        buf_a.copy_(xs[t])
        graph.replay()
        buf_b.copy_(xs[t])
        call(b, buf_b)
        torch.cuda.synchronize()
        assert torch.equal(buf_a.view(torch.int32), buf_b.view(torch.int32)), t
        for vi in (2, 4):
            ea, eb = a.error(0, vi), b.error(0, vi)
            _, qa = a.factors(0, vi)
            _, qb = b.factors(0, vi)
            torch.cuda.synchronize()
            assert torch.equal(ea.view(torch.int32), eb.view(torch.int32)), (t, vi)
            assert torch.equal(qa.view(torch.int32), qb.view(torch.int32)), (t, vi)
        log(f"  replay {t}: bucket, E and Q bitwise equal to the eager step")
    assert np.isfinite(buf_a.cpu().numpy()).all()


def test_amp_call_replays_bitwise_with_an_inf_step():
    """The fp16 AMP call (fused unscale and inf check) replayed from a graph, the caller
    clearing found_inf with a fill kernel before each replay; replay 3 carries an inf,
    so that step is skipped on both sides and found_inf reads 1 only there."""
    log("case: graph replay, AMP fp16 rank 2 with an inf step")
    hp = dict(matrix_approximation_rank=2, start_powerSGD_iter=0, warm_start=True,
              use_error_feedback=True, orthogonalization_epsilon=0.0,
              compression_stats_logging_frequency=0)
    a, b = PowerSGDState(**hp), PowerSGDState(**hp)
    scale = 1024.0
    xs = [(x * scale).half() for x in _inputs(6, 11)]
    xs[3][5000] = float("inf")
    buf_a = torch.empty(NUMEL, dtype=torch.float16, device="cuda")
    buf_b = torch.empty(NUMEL, dtype=torch.float16, device="cuda")
    fa = torch.zeros(1, dtype=torch.int32, device="cuda")
    fb = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call(st, buf, found, stream=None):
        st.compress_bucket(buf, VIEWS, inv_loss_scale=1.0 / scale, found_inf=found, stream=stream)

    for st, buf, found in ((a, buf_a, fa), (b, buf_b, fb)):  # allocation and tables
        buf.copy_(xs[0])
        call(st, buf, found)
    torch.cuda.synchronize()
    assert int(fa.item()) == 0 and int(fb.item()) == 0
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    buf_a.copy_(xs[1])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        call(a, buf_a, fa, stream=s)
    for t in range(1, 6):
        buf_a.copy_(xs[t])
        fa.zero_()
        graph.replay()
        buf_b.copy_(xs[t])
        fb.zero_()
        call(b, buf_b, fb)
        torch.cuda.synchronize()
        assert int(fa.item()) == int(fb.item()) == int(t == 3), t
        assert torch.equal(buf_a.view(torch.int16), buf_b.view(torch.int16)), t
        for vi in (2, 4):
            ea, eb = a.error(0, vi), b.error(0, vi)
            _, qa = a.factors(0, vi)
            _, qb = b.factors(0, vi)
            torch.cuda.synchronize()
            assert torch.equal(ea.view(torch.int32), eb.view(torch.int32)), (t, vi)
            assert torch.equal(qa.view(torch.int32), qb.view(torch.int32)), (t, vi)
        log(f"  replay {t}: found_inf {int(fa.item())}; bucket, E and Q bitwise equal")


def test_batched_call_replays_bitwise():
    """batched_powerSGD_hook replayed from a graph: the zero padding of the square matrix
    is written by a kernel on every call, so the captured call redoes it; the first
    numel elements (the result) and the padding both match the eager steps bitwise."""
    log("case: graph replay, batched rank 1")
    hp = dict(matrix_approximation_rank=1, start_powerSGD_iter=0, warm_start=True,
              use_error_feedback=True, orthogonalization_epsilon=0.0,
              compression_stats_logging_frequency=0)
    a, b = PowerSGDState(**hp), PowerSGDState(**hp)
    xs = _inputs(6, 13)
    side = 1
    while side * side < NUMEL:
        side += 1
    buf_a = torch.full((side * side,), 7.0, device="cuda")
    buf_b = torch.full((side * side,), 7.0, device="cuda")
    for st, buf in ((a, buf_a), (b, buf_b)):
        buf[:NUMEL].copy_(xs[0])
        st.compress_bucket_batched(buf, numel=NUMEL)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    buf_a[:NUMEL].copy_(xs[1])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        a.compress_bucket_batched(buf_a, numel=NUMEL, stream=s)
    for t in range(1, 6):
        buf_a[:NUMEL].copy_(xs[t])
        buf_a[NUMEL:].fill_(3.0)  # the call must clear the padding itself
        graph.replay()
        buf_b[:NUMEL].copy_(xs[t])
        buf_b[NUMEL:].fill_(5.0)
        b.compress_bucket_batched(buf_b, numel=NUMEL)
        torch.cuda.synchronize()
        assert torch.equal(buf_a.view(torch.int32), buf_b.view(torch.int32)), t
        ea, eb = a.error(0, 0), b.error(0, 0)
        _, qa = a.factors(0, 0)
        _, qb = b.factors(0, 0)
        torch.cuda.synchronize()
        assert torch.equal(ea.view(torch.int32), eb.view(torch.int32)), t
        assert torch.equal(qa.view(torch.int32), qb.view(torch.int32)), t
        log(f"  replay {t}: buffer, E and Q bitwise equal to the eager step")
