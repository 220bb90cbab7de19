"""Plain fp64 CPU oracle for PowerSGD compression of one rank's gradient bucket.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does, and this
module imports nothing from the product package.

Sources (titles and sections of the pages this follows):

* "DDP Communication Hooks -- PyTorch 1.11.0", section "PowerSGD State": the
  hyperparameters, their defaults, the `min_compression_rate` inequality and the
  role of `orthogonalization_epsilon`; section "PowerSGD Hooks": the error-feedback
  memory (first warning) and powerSGD_hook's numbered steps 1 to 3.7.
* The spec-zone.ru translation of the same page ("Связки связи DDP"), section
  "Состояние PowerSGD", item 5: `batch_tensors_with_same_shape`, which batches
  same-shape tensors and leaves the arithmetic unchanged.
* "torch.cuda.amp -- PyTorch 1.5.0", section "Gradient Scaling", GradScaler's
  `unscale_` (divide by the scale, look for inf/NaN) and `step` (skip the update
  when any inf/NaN was found).

Readings taken where the pages are silent (each is marked READING below):
error feedback is M' = G + E, E <- M' - M_hat with E starting at zero; warm start
reuses the previous step's Q = M'^T P and draws Q only once (epoch 0), while without
warm start a fresh Q is drawn each step with epoch = iteration; epsilon is added to
the column norm in the denominator; Gram-Schmidt is the modified variant; the draw
is orthogonalized, a warm Q is not; a tensor with ndim >= 2 is viewed as
shape[0] x prod(shape[1:]); the rank used for a tensor is min(r, n, m); the rate
test is evaluated exactly on the given binary64 rate; fp16 buckets are unscaled
by an exact power-of-two factor and written back unscaled in fp16 with
round-to-nearest-even, and on inf/NaN the bucket and all state stay untouched while
the iteration still advances.

Everything is float64 on the host, except Gram-Schmidt, which runs in double-double
arithmetic (oracle.ddarith) and rounds its result to float64; the only library
routine used as a step is the matrix product (numpy's `@`).
"""
from __future__ import annotations

import math
import struct
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .rng import standard_normal_q0


@dataclass
class HParams:
    """PowerSGDState's hyperparameters and defaults ("PowerSGD State" section).

    `process_group` is absent: one rank, so every allreduce is the identity.
    `batch_tensors_with_same_shape` comes from the translated page's signature.
    """
    matrix_approximation_rank: int = 1
    start_powerSGD_iter: int = 1000
    min_compression_rate: float = 2.0
    use_error_feedback: bool = True
    warm_start: bool = True
    orthogonalization_epsilon: float = 0.0
    random_seed: int = 0
    compression_stats_logging_frequency: int = 10000
    batch_tensors_with_same_shape: bool = False


View = Tuple[int, Tuple[int, ...]]  # (element offset into the flat bucket, shape)


def matrix_view(shape: Sequence[int]) -> Optional[Tuple[int, int]]:
    """(n, m) of the matrix a parameter tensor is compressed as, or None.

    powerSGD_hook step 1.2 leaves "all the vector tensors" uncompressed; READING:
    a tensor of ndim >= 2 is the row-major matrix shape[0] x prod(shape[1:]).
    """
    if len(shape) < 2:
        return None
    n = int(shape[0])
    m = 1
    for d in shape[1:]:
        m *= int(d)
    return n, m


def should_compress(n: int, m: int, rank: int, min_compression_rate: float) -> bool:
    """The "PowerSGD State" rate test: (n + m) * rank * rate < n * m, strictly.

    READING: evaluated exactly on the rate's binary64 value (a Fraction), so the
    decision is an exact integer/rational comparison. Empty matrices are never
    compressed.
    """
    if n * m == 0:
        return False
    return (n + m) * rank * Fraction(min_compression_rate) < n * m


def batched_side(numel: int) -> int:
    """batched_powerSGD_hook step 1 ("PowerSGD Hooks"): the flat bucket is viewed as a
    square matrix with zero padding; its side is the smallest s with s * s >= numel."""
    if numel <= 0:
        return 0
    s = math.isqrt(numel)
    return s if s * s == numel else s + 1


def effective_rank(n: int, m: int, rank: int) -> int:
    """READING: a factor cannot have more columns than the matrix has rows or columns."""
    return min(rank, n, m)


def gram_schmidt(x: np.ndarray, epsilon: float) -> np.ndarray:
    """Orthogonalize the columns of x, in order (powerSGD_hook step 3.4).

    Modified Gram-Schmidt. READING of the "PowerSGD State" note on
    `orthogonalization_epsilon`: each column is divided by (its 2-norm + epsilon),
    which is what keeps an all-zero column from dividing by zero. After column i is
    normalized, its projection is removed from every later column.

    READING of "orthogonalizes" (the method's exact Gram-Schmidt): the steps run in
    double-double arithmetic (oracle.ddarith) on the binary64 input, and the result is
    rounded to binary64. Modified Gram-Schmidt in a precision u loses orthogonality in
    proportion to u times the condition number of x; warm-started steps on a matrix of
    rank below r drive that condition number of P past 1e12, where binary64 steps no
    longer give orthonormal columns while about 106-bit steps still do to 1e-18.
    """
    from . import ddarith as dd
    xh = np.array(x, dtype=np.float64, copy=True)
    r = xh.shape[1] if xh.ndim == 2 else 0
    hi = [xh[:, j].copy() for j in range(r)]
    lo = [np.zeros_like(xh[:, 0]) for _ in range(r)] if r else []
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for i in range(r):
            nh, nl = dd.dd_dot(hi[i], lo[i], hi[i], lo[i])
            ih, il = dd.inverse_norm_plus(nh, nl, float(epsilon))
            hi[i], lo[i] = dd.dd_mul(hi[i], lo[i], ih, il)
            for j in range(i + 1, r):
                ch, cl = dd.dd_dot(hi[i], lo[i], hi[j], lo[j])
                ph, pl = dd.dd_mul(hi[i], lo[i], -ch, -cl)
                hi[j], lo[j] = dd.dd_add(hi[j], lo[j], ph, pl)
    out = np.empty_like(xh)
    for j in range(r):
        out[:, j] = hi[j] + lo[j]
    return out


@dataclass
class ViewResult:
    """Per-view record of one call, for comparison with the device results."""
    compressed: bool
    n: int = 0
    m: int = 0
    rank: int = 0
    m_prime: Optional[np.ndarray] = None   # M' = G + E_prev
    p: Optional[np.ndarray] = None         # orthogonalized P (n x rank)
    q: Optional[np.ndarray] = None         # Q = M'^T P (m x rank)
    m_hat: Optional[np.ndarray] = None     # P Q^T
    error: Optional[np.ndarray] = None     # new E = M' - M_hat (None without error feedback)


@dataclass
class StepResult:
    output: np.ndarray                     # the bucket after the call (input dtype)
    output64: np.ndarray                   # the same before any cast (float64)
    found_inf: bool
    skipped: bool                          # inf/NaN found: nothing was changed
    passthrough: bool                      # iteration < start_powerSGD_iter
    views: List[ViewResult] = field(default_factory=list)


@dataclass
class _BucketMemory:
    layout: Tuple
    numel: int = 0                                               # bucket length
    error: Dict[int, np.ndarray] = field(default_factory=dict)   # view -> E (fp64)
    q: Dict[int, np.ndarray] = field(default_factory=dict)       # view -> warm Q


def any_nonfinite(bucket: np.ndarray, views: Sequence[View]) -> bool:
    """GradScaler's check ("Gradient Scaling", unscale_/step): is any gradient value
    in any view inf or NaN?"""
    for off, shp in views:
        size = int(np.prod(shp, dtype=np.int64))
        if not np.all(np.isfinite(bucket[off:off + size])):
            return True
    return False


class LayoutChanged(Exception):
    """A bucket's views changed after its E or Q was memorized ("PowerSGD State"
    warning on rebuilt buckets)."""


class OracleState:
    """The internal state PowerSGDState keeps "for all the gradients during the
    training": per-bucket error memory and warm-start Q, the iteration counter and
    the compression statistics."""

    def __init__(self, hp: HParams):
        if hp.matrix_approximation_rank < 1:
            raise ValueError("matrix_approximation_rank must be >= 1")
        if not (hp.orthogonalization_epsilon >= 0.0):
            raise ValueError("orthogonalization_epsilon must be >= 0")
        self.hp = hp
        self.iteration = 0
        self.numel_in = 0
        self.numel_comm = 0
        # iteration at or after which the next statistics line is due
        self.next_log_iteration = hp.start_powerSGD_iter
        self.buckets: Dict[int, _BucketMemory] = {}

    def _end_call(self, is_last: bool, compressing: bool) -> None:
        """Iteration bookkeeping at the end of a call: the last bucket of an iteration
        advances the counter; past start_powerSGD_iter it also moves the statistics
        schedule on by compression_stats_logging_frequency when a line was due
        ("PowerSGD State", compression_stats_logging_frequency)."""
        if not is_last:
            return
        freq = self.hp.compression_stats_logging_frequency
        if compressing and freq > 0 and self.iteration >= self.next_log_iteration:
            self.next_log_iteration = self.iteration + freq
        self.iteration += 1

    def _view_counts(self, views: Sequence[View]) -> Tuple[int, int]:
        """Elements in, and elements an allreduce would carry, for one per-layer call:
        (n + m) * rank per compressed view, numel per other view."""
        hp = self.hp
        numel_in = comm = 0
        for _, shp in views:
            size = int(np.prod(shp, dtype=np.int64))
            numel_in += size
            nm = matrix_view(shp)
            if nm is not None:
                n, m = nm
                rank = effective_rank(n, m, hp.matrix_approximation_rank)
                if should_compress(n, m, rank, hp.min_compression_rate):
                    comm += (n + m) * rank
                    continue
            comm += size
        return numel_in, comm

    def compress_bucket(self, bucket: np.ndarray, views: Sequence[View],
                        bucket_index: int = 0, is_last: bool = True,
                        inv_loss_scale: float = 1.0) -> StepResult:
        """One powerSGD_hook call on a single rank's flat bucket.

        `bucket` is float32 or float16 (the latter holds loss-scaled gradients).
        Returns the new bucket contents; the input array is not modified.
        """
        hp = self.hp
        bucket = np.asarray(bucket)
        if bucket.dtype not in (np.float32, np.float16):
            raise TypeError("bucket must be float32 or float16")
        is_fp16 = bucket.dtype == np.float16
        views = [(int(off), tuple(int(d) for d in shp)) for off, shp in views]
        x64 = bucket.astype(np.float64)

        # GradScaler.unscale_/step: look for inf/NaN, skip everything if found.
        # READING: past start_powerSGD_iter the call still counts in the compression
        # statistics: the hook compresses and communicates before GradScaler.step
        # decides to skip the update, and the statistics describe that communication.
        found_inf = is_fp16 and any_nonfinite(bucket, views)
        if found_inf:
            compressing = self.iteration >= hp.start_powerSGD_iter
            if compressing:
                n_in, n_comm = self._view_counts(views)
                self.numel_in += n_in
                self.numel_comm += n_comm
            self._end_call(is_last, compressing)
            return StepResult(output=bucket.copy(), output64=x64, found_inf=True,
                              skipped=True, passthrough=False)

        g_all = x64 * float(inv_loss_scale) if is_fp16 else x64
        out64 = x64.copy()
        result = StepResult(output=bucket, output64=out64, found_inf=False,
                            skipped=False, passthrough=False)

        # Before start_powerSGD_iter the hook does a vanilla allreduce: on one rank,
        # the identity on the (unscaled) gradients.
        if self.iteration < hp.start_powerSGD_iter:
            result.passthrough = True
            for off, shp in views:
                size = int(np.prod(shp, dtype=np.int64))
                out64[off:off + size] = g_all[off:off + size]
                result.views.append(ViewResult(compressed=False))
            result.output = out64.astype(bucket.dtype) if is_fp16 else bucket.copy()
            self._end_call(is_last, False)
            return result

        layout = tuple(views)
        mem = self.buckets.get(bucket_index)
        if mem is not None and mem.layout != layout:
            if hp.use_error_feedback or hp.warm_start:
                raise LayoutChanged(f"bucket {bucket_index} changed its layout")
            mem = None
        if mem is None:
            mem = _BucketMemory(layout=layout, numel=int(bucket.size))
            self.buckets[bucket_index] = mem

        comm = 0
        numel_in = 0
        for vi, (off, shp) in enumerate(views):
            size = int(np.prod(shp, dtype=np.int64))
            numel_in += size
            g = g_all[off:off + size]
            nm = matrix_view(shp)
            rank = 0
            compress = False
            if nm is not None:
                n, m = nm
                rank = effective_rank(n, m, hp.matrix_approximation_rank)
                compress = should_compress(n, m, rank, hp.min_compression_rate)
            if not compress:
                # Step 2: uncompressed tensors are allreduced as they are.
                out64[off:off + size] = g
                comm += size
                result.views.append(ViewResult(compressed=False))
                continue
            vr = self._compress_matrix(g.reshape(n, m), mem, vi, bucket_index, rank)
            out64[off:off + size] = vr.m_hat.reshape(-1)
            comm += (n + m) * rank
            result.views.append(vr)

        self.numel_in += numel_in
        self.numel_comm += comm
        if is_fp16:
            result.output = out64.astype(np.float16)
        else:
            result.output = out64.astype(np.float32)
        self._end_call(is_last, True)
        return result

    def compress_bucket_batched(self, bucket: np.ndarray, bucket_index: int = 0,
                                is_last: bool = True,
                                inv_loss_scale: float = 1.0) -> StepResult:
        """One batched_powerSGD_hook call ("PowerSGD Hooks", batched_powerSGD_hook,
        steps 1 to 9) on a single rank's flat bucket of numel elements.

        The bucket, followed by s * s - numel zeros, is the s x s row-major matrix M
        (step 1); then P = M Q, Gram-Schmidt, Q = M^T P, M_hat = P Q^T as in
        powerSGD_hook (steps 2 to 8, both allreduces the identity), and the result is
        M_hat's first numel elements (step 9).
        READING: the state's error feedback and warm start apply as for powerSGD_hook,
        with E covering all s * s entries (the padding of G is zero at every call, so
        E's padded entries carry over); there is no rate test; the rank is
        min(r, s); the Q draw uses view index 0; the memorized layout of the bucket is
        ("batched", numel). The returned views list holds the one matrix; stats count
        numel in and 2 s r communicated.
        """
        hp = self.hp
        bucket = np.asarray(bucket)
        if bucket.dtype not in (np.float32, np.float16):
            raise TypeError("bucket must be float32 or float16")
        is_fp16 = bucket.dtype == np.float16
        numel = int(bucket.size)
        x64 = bucket.astype(np.float64)
        found_inf = is_fp16 and not bool(np.all(np.isfinite(bucket)))
        s = batched_side(numel)
        if found_inf:
            # statistics count the skipped call, as in compress_bucket
            compressing = self.iteration >= hp.start_powerSGD_iter
            if compressing:
                self.numel_in += numel
                if s > 0:
                    self.numel_comm += 2 * s * effective_rank(s, s, hp.matrix_approximation_rank)
            self._end_call(is_last, compressing)
            return StepResult(output=bucket.copy(), output64=x64, found_inf=True,
                              skipped=True, passthrough=False)
        g_all = x64 * float(inv_loss_scale) if is_fp16 else x64
        result = StepResult(output=bucket, output64=g_all.copy(), found_inf=False,
                            skipped=False, passthrough=False)
        if self.iteration < hp.start_powerSGD_iter:
            result.passthrough = True
            result.output = g_all.astype(bucket.dtype) if is_fp16 else bucket.copy()
            self._end_call(is_last, False)
            return result
        layout = ("batched", numel)
        mem = self.buckets.get(bucket_index)
        if mem is not None and mem.layout != layout:
            if hp.use_error_feedback or hp.warm_start:
                raise LayoutChanged(f"bucket {bucket_index} changed its layout")
            mem = None
        if mem is None:
            mem = _BucketMemory(layout=layout, numel=numel)
            self.buckets[bucket_index] = mem
        if s > 0:
            padded = np.zeros(s * s, dtype=np.float64)
            padded[:numel] = g_all
            rank = effective_rank(s, s, hp.matrix_approximation_rank)
            vr = self._compress_matrix(padded.reshape(s, s), mem, 0, bucket_index, rank)
            result.output64 = vr.m_hat.reshape(-1)[:numel].copy()
            result.views.append(vr)
            self.numel_comm += 2 * s * rank
        self.numel_in += numel
        result.output = result.output64.astype(bucket.dtype)
        self._end_call(is_last, True)
        return result

    def compress_bucket_wrapped(self, bucket: np.ndarray, views: Sequence[View],
                                compute_dtype: str = "f16", bucket_index: int = 0,
                                is_last: bool = True) -> StepResult:
        """fp16_compress_wrapper(powerSGD_hook) or bf16_compress_wrapper(powerSGD_hook)
        ("Default Communication Hooks") on one rank's fp32 bucket: the bucket is cast
        to 16 bits, the hook runs on that tensor with every tensor it materializes held
        in 16 bits (oracle.lowp), and the result is cast back to fp32.

        READING: elements outside every view are left as they are (a DDP bucket has
        none); the Q draw is the binary32 draw of powerSGD_hook cast to 16 bits, then
        orthogonalized and rounded; the memorized layout is ("wrapped", dtype, views),
        so E and Q of another variant are never reused. No loss scaling is involved:
        values beyond the 16-bit range become inf and propagate.
        """
        from .lowp import ROUNDERS, compress_matrix_step_lowp

        hp = self.hp
        rnd = ROUNDERS[compute_dtype]
        bucket = np.asarray(bucket)
        if bucket.dtype != np.float32:
            raise TypeError("the wrapped hook takes a float32 bucket")
        views = [(int(off), tuple(int(d) for d in shp)) for off, shp in views]
        x64 = bucket.astype(np.float64)
        out64 = x64.copy()
        result = StepResult(output=bucket, output64=out64, found_inf=False, skipped=False,
                            passthrough=False)
        # the wrapper's cast of the gradients
        b16 = x64.copy()
        for off, shp in views:
            size = int(np.prod(shp, dtype=np.int64))
            b16[off:off + size] = rnd(x64[off:off + size])
        if self.iteration < hp.start_powerSGD_iter:
            result.passthrough = True
            for off, shp in views:
                size = int(np.prod(shp, dtype=np.int64))
                out64[off:off + size] = b16[off:off + size]
                result.views.append(ViewResult(compressed=False))
            result.output = out64.astype(np.float32)
            self._end_call(is_last, False)
            return result

        layout = ("wrapped", compute_dtype, tuple(views))
        mem = self.buckets.get(bucket_index)
        if mem is not None and mem.layout != layout:
            if hp.use_error_feedback or hp.warm_start:
                raise LayoutChanged(f"bucket {bucket_index} changed its layout")
            mem = None
        if mem is None:
            mem = _BucketMemory(layout=layout, numel=int(bucket.size))
            self.buckets[bucket_index] = mem

        eps = float(hp.orthogonalization_epsilon)
        comm = numel_in = 0
        for vi, (off, shp) in enumerate(views):
            size = int(np.prod(shp, dtype=np.int64))
            numel_in += size
            g16 = b16[off:off + size]
            nm = matrix_view(shp)
            compress = False
            if nm is not None:
                n, m = nm
                rank = effective_rank(n, m, hp.matrix_approximation_rank)
                compress = should_compress(n, m, rank, hp.min_compression_rate)
            if not compress:
                out64[off:off + size] = g16
                comm += size
                result.views.append(ViewResult(compressed=False))
                continue
            if hp.warm_start and vi in mem.q:
                q = mem.q[vi]
            else:
                epoch = 0 if hp.warm_start else self.iteration
                draw = standard_normal_q0(m, rank, hp.random_seed, bucket_index, vi, epoch)
                q = rnd(gram_schmidt(rnd(draw), eps))
            e_prev = mem.error.get(vi) if hp.use_error_feedback else None
            m_prime, p, q_new, m_hat, err = compress_matrix_step_lowp(
                g16.reshape(n, m), e_prev, q, eps, hp.use_error_feedback, rnd)
            if hp.use_error_feedback:
                mem.error[vi] = err
            if hp.warm_start:
                mem.q[vi] = q_new
            out64[off:off + size] = m_hat.reshape(-1)
            comm += (n + m) * rank
            result.views.append(ViewResult(compressed=True, n=n, m=m, rank=rank,
                                           m_prime=m_prime, p=p, q=q_new, m_hat=m_hat,
                                           error=err))
        self.numel_in += numel_in
        self.numel_comm += comm
        result.output = out64.astype(np.float32)
        self._end_call(is_last, True)
        return result

    def compress_bucket_batched_wrapped(self, bucket: np.ndarray, compute_dtype: str = "f16",
                                        bucket_index: int = 0,
                                        is_last: bool = True) -> StepResult:
        """fp16_compress_wrapper or bf16_compress_wrapper around batched_powerSGD_hook
        ("Default Communication Hooks"; "PowerSGD Hooks", batched_powerSGD_hook steps 1
        to 9): the fp32 bucket is cast to 16 bits, zero-padded to the s x s matrix, the
        hook's steps run with every formed tensor in 16 bits (oracle.lowp), and the
        first numel entries of M_hat are cast back to fp32.

        READING: as compress_bucket_batched (E over all s * s entries, no rate test,
        rank min(r, s), view index 0 for the draw) and compress_bucket_wrapped (the
        binary32 draw cast to 16 bits, no loss scaling); the memorized layout is
        ("batched", numel, dtype).
        """
        from .lowp import ROUNDERS, compress_matrix_step_lowp

        hp = self.hp
        rnd = ROUNDERS[compute_dtype]
        bucket = np.asarray(bucket)
        if bucket.dtype != np.float32:
            raise TypeError("the wrapped hook takes a float32 bucket")
        numel = int(bucket.size)
        g16 = rnd(bucket.astype(np.float64))          # the wrapper's cast
        result = StepResult(output=bucket, output64=g16.copy(), found_inf=False,
                            skipped=False, passthrough=False)
        if self.iteration < hp.start_powerSGD_iter:
            result.passthrough = True
            result.output = g16.astype(np.float32)
            self._end_call(is_last, False)
            return result
        layout = ("batched", numel, compute_dtype)
        mem = self.buckets.get(bucket_index)
        if mem is not None and mem.layout != layout:
            if hp.use_error_feedback or hp.warm_start:
                raise LayoutChanged(f"bucket {bucket_index} changed its layout")
            mem = None
        if mem is None:
            mem = _BucketMemory(layout=layout, numel=numel)
            self.buckets[bucket_index] = mem
        s = batched_side(numel)
        if s > 0:
            eps = float(hp.orthogonalization_epsilon)
            padded = np.zeros(s * s, dtype=np.float64)
            padded[:numel] = g16
            rank = effective_rank(s, s, hp.matrix_approximation_rank)
            if hp.warm_start and 0 in mem.q:
                q = mem.q[0]
            else:
                epoch = 0 if hp.warm_start else self.iteration
                q = rnd(gram_schmidt(rnd(standard_normal_q0(s, rank, hp.random_seed,
                                                            bucket_index, 0, epoch)), eps))
            e_prev = mem.error.get(0) if hp.use_error_feedback else None
            m_prime, p, q_new, m_hat, err = compress_matrix_step_lowp(
                padded.reshape(s, s), e_prev, q, eps, hp.use_error_feedback, rnd)
            if hp.use_error_feedback:
                mem.error[0] = err
            if hp.warm_start:
                mem.q[0] = q_new
            result.output64 = m_hat.reshape(-1)[:numel].copy()
            result.views.append(ViewResult(compressed=True, n=s, m=s, rank=rank,
                                           m_prime=m_prime, p=p, q=q_new, m_hat=m_hat,
                                           error=err))
            self.numel_comm += 2 * s * rank
        self.numel_in += numel
        result.output = result.output64.astype(np.float32)
        self._end_call(is_last, True)
        return result

    # ---- snapshot (checkpoint / resume) -------------------------------------------
    # The pages describe no PowerSGDState checkpoint (GradScaler.state_dict in
    # "Gradient Scaling" is the analogue). The byte format is the library's documented
    # version-1 snapshot, written here independently: a little-endian 80-byte header,
    # then per bucket (ascending index) its record (the variant word: bit 0 batched,
    # bits 8-9 the precision of a wrapped bucket's state, 1 binary16, 2 bfloat16), its
    # views, and per compressed view E (n*m binary32, with error feedback) and the
    # warm-start Q (m*k binary32).

    _SNAP_MAGIC = b"PSGDSNAP"
    _SNAP_HEADER = struct.Struct("<8sIIiIdQqqqqq")   # 80 bytes
    _SNAP_BUCKET = struct.Struct("<qqIIq")           # 32 bytes

    _SNAP_PRECISION = {None: 0, "f16": 1, "bf16": 2}

    def _snapshot_views(self, mem: _BucketMemory):
        """(batched, 16-bit precision or None, views, compressed view indices with their
        (n, m, rank))."""
        hp = self.hp
        if mem.layout[:1] == ("batched",):
            prec = mem.layout[2] if len(mem.layout) > 2 else None
            s = batched_side(mem.numel)
            if s == 0:
                return True, prec, [], []
            return True, prec, [(0, (s, s))], [(0, s, s, effective_rank(
                s, s, hp.matrix_approximation_rank))]
        prec = None
        views = list(mem.layout)
        if mem.layout[:1] == ("wrapped",):
            prec, views = mem.layout[1], list(mem.layout[2])
        comp = []
        for vi, (_, shp) in enumerate(views):
            nm = matrix_view(shp)
            if nm is None:
                continue
            n, m = nm
            rank = effective_rank(n, m, hp.matrix_approximation_rank)
            if should_compress(n, m, rank, hp.min_compression_rate):
                comp.append((vi, n, m, rank))
        return False, prec, views, comp

    def export_state(self) -> bytes:
        """The state as a version-1 snapshot. E and Q are rounded to binary32, the
        precision the snapshot stores."""
        hp = self.hp
        flags = (1 if hp.use_error_feedback else 0) | (2 if hp.warm_start else 0)
        parts = [self._SNAP_HEADER.pack(
            self._SNAP_MAGIC, 1, flags, hp.matrix_approximation_rank, 0,
            float(hp.min_compression_rate), hp.random_seed, self.iteration, self.numel_in,
            self.numel_comm, self.next_log_iteration, len(self.buckets))]
        for idx in sorted(self.buckets):
            mem = self.buckets[idx]
            batched, prec, views, comp = self._snapshot_views(mem)
            has_q = bool(hp.warm_start and comp and all(vi in mem.q for vi, *_ in comp))
            variant = int(batched) | (self._SNAP_PRECISION[prec] << 8)
            parts.append(self._SNAP_BUCKET.pack(idx, mem.numel, variant, int(has_q),
                                                len(views)))
            for off, shp in views:
                parts.append(struct.pack(f"<qq{len(shp)}q", off, len(shp), *shp))
            for vi, n, m, rank in comp:
                if hp.use_error_feedback:
                    e = mem.error.get(vi)
                    if e is None:
                        e = np.zeros((n, m))
                    parts.append(np.ascontiguousarray(e, dtype="<f4").tobytes())
                if has_q:
                    parts.append(np.ascontiguousarray(mem.q[vi], dtype="<f4").tobytes())
        return b"".join(parts)

    def import_state(self, data: bytes) -> None:
        """Replaces the state with a version-1 snapshot taken under the same error
        feedback, warm start, rank, min_compression_rate and random_seed. Raises
        ValueError (state unchanged) on anything malformed."""
        hp = self.hp
        data = bytes(data)
        pos = 0

        def take(fmt_or_len):
            nonlocal pos
            if isinstance(fmt_or_len, int):
                if fmt_or_len < 0 or pos + fmt_or_len > len(data):
                    raise ValueError("snapshot truncated")
                out = data[pos:pos + fmt_or_len]
                pos += fmt_or_len
                return out
            st = fmt_or_len if isinstance(fmt_or_len, struct.Struct) else struct.Struct(fmt_or_len)
            if pos + st.size > len(data):
                raise ValueError("snapshot truncated")
            out = st.unpack_from(data, pos)
            pos += st.size
            return out

        (magic, version, flags, rank, reserved, rate, seed, iteration, numel_in, numel_comm,
         next_log, nbuckets) = take(self._SNAP_HEADER)
        if magic != self._SNAP_MAGIC:
            raise ValueError("bad magic")
        if version != 1:
            raise ValueError(f"unknown version {version}")
        if reserved != 0 or flags & ~3:
            raise ValueError("bad flags")
        want = (1 if hp.use_error_feedback else 0) | (2 if hp.warm_start else 0)
        if (flags != want or rank != hp.matrix_approximation_rank or seed != hp.random_seed
                or struct.pack("<d", rate) != struct.pack("<d", float(hp.min_compression_rate))):
            raise ValueError("snapshot taken under other hyperparameters")
        if min(iteration, numel_in, numel_comm, next_log, nbuckets) < 0:
            raise ValueError("negative counter")
        buckets: Dict[int, _BucketMemory] = {}
        prev = None
        for _ in range(nbuckets):
            idx, numel, variant, has_q, nviews = take(self._SNAP_BUCKET)
            if prev is not None and idx <= prev:
                raise ValueError("bucket indices not strictly ascending")
            prev = idx
            batched, pcode = variant & 1, (variant >> 8) & 3
            if numel < 0 or nviews < 0 or variant & ~0x301 or pcode == 3 or has_q > 1:
                raise ValueError("bad bucket record")
            prec = {0: None, 1: "f16", 2: "bf16"}[pcode]
            if has_q and not hp.warm_start:
                raise ValueError("warm-start Q without warm start")
            views = []
            for _ in range(nviews):
                off, ndim = take("<qq")
                if not 0 <= ndim <= 8:
                    raise ValueError("view ndim out of range")
                shp = take(f"<{ndim}q") if ndim else ()
                views.append((off, tuple(shp)))
            if batched:
                s = batched_side(numel)
                if views != ([(0, (s, s))] if numel > 0 else []):
                    raise ValueError("batched bucket is not one s x s view")
                layout = ("batched", numel) if prec is None else ("batched", numel, prec)
                mem = _BucketMemory(layout=layout, numel=numel)
            else:
                spans = []
                for off, shp in views:
                    size = int(np.prod(shp, dtype=np.int64)) if shp else 1
                    if min(shp, default=0) < 0 or off < 0 or off + size > numel:
                        raise ValueError("view outside the bucket")
                    if size > 0:
                        spans.append((off, off + size))
                spans.sort()
                if any(b[0] < a[1] for a, b in zip(spans, spans[1:])):
                    raise ValueError("views overlap")
                layout = tuple(views) if prec is None else ("wrapped", prec, tuple(views))
                mem = _BucketMemory(layout=layout, numel=numel)
            _, _, _, comp = self._snapshot_views(mem)
            # a 16-bit state holds 16-bit values: what the snapshot gives is rounded
            from .lowp import ROUNDERS
            fix = (lambda a: a) if prec is None else ROUNDERS[prec]
            if has_q and not comp:
                raise ValueError("warm-start Q on a bucket with no compressed view")
            for vi, n, m, k in comp:
                if hp.use_error_feedback:
                    raw = take(4 * n * m)
                    mem.error[vi] = fix(np.frombuffer(raw, dtype="<f4").astype(np.float64)
                                        ).reshape(n, m)
                if has_q:
                    raw = take(4 * m * k)
                    mem.q[vi] = fix(np.frombuffer(raw, dtype="<f4").astype(np.float64)
                                    ).reshape(m, k)
            buckets[idx] = mem
        if pos != len(data):
            raise ValueError(f"{len(data) - pos} trailing bytes")
        self.buckets = buckets
        self.iteration = iteration
        self.numel_in = numel_in
        self.numel_comm = numel_comm
        self.next_log_iteration = next_log

    def _compress_matrix(self, g: np.ndarray, mem: _BucketMemory, view: int,
                         bucket_index: int, rank: int) -> ViewResult:
        """Pick E and Q for one matrix, run the step, memorize the new E and Q."""
        hp = self.hp
        n, m = g.shape
        eps = float(hp.orthogonalization_epsilon)
        e_prev = mem.error.get(view) if hp.use_error_feedback else None
        if hp.warm_start and view in mem.q:
            q = mem.q[view]
        else:
            epoch = 0 if hp.warm_start else self.iteration
            q = gram_schmidt(standard_normal_q0(m, rank, hp.random_seed, bucket_index,
                                                view, epoch), eps)
        vr = compress_matrix_step(g, e_prev, q, eps, hp.use_error_feedback)
        if hp.use_error_feedback:
            mem.error[view] = vr.error
        if hp.warm_start:
            mem.q[view] = vr.q
        return vr


def compress_matrix_step(g: np.ndarray, e_prev: Optional[np.ndarray], q: np.ndarray,
                         epsilon: float, use_error_feedback: bool = True) -> ViewResult:
    """Steps 3.2 to 3.7 of powerSGD_hook for one n x m matrix on one rank.

    g: the gradient; e_prev: the error memory (None = zero); q: the m x r starting Q
    (a warm Q, or an orthogonalized draw). Both allreduces are the identity.
    """
    g = np.asarray(g, dtype=np.float64)
    n, m = g.shape
    m_prime = g + e_prev if (use_error_feedback and e_prev is not None) else g.copy()
    p = m_prime @ q                          # 3.2  P = M Q
    p = gram_schmidt(p, epsilon)             # 3.4
    q_new = m_prime.T @ p                    # 3.5  Q = M^T P
    m_hat = p @ q_new.T                      # 3.7  M ~ P Q^T
    err = m_prime - m_hat if use_error_feedback else None
    return ViewResult(compressed=True, n=n, m=m, rank=q.shape[1], m_prime=m_prime, p=p,
                      q=q_new, m_hat=m_hat, error=err)
