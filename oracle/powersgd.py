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

Everything is float64 on the host; the only library routine used as a step is the
matrix product (numpy's `@`).
"""
from __future__ import annotations

import math
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
    """
    q = np.array(x, dtype=np.float64, copy=True)
    r = q.shape[1]
    for i in range(r):
        col = q[:, i]
        q[:, i] = col / (math.sqrt(float(col @ col)) + epsilon)
        for j in range(i + 1, r):
            q[:, j] = q[:, j] - float(q[:, i] @ q[:, j]) * q[:, i]
    return q


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
        self.buckets: Dict[int, _BucketMemory] = {}

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
        found_inf = is_fp16 and any_nonfinite(bucket, views)
        if found_inf:
            if is_last:
                self.iteration += 1
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
            if is_last:
                self.iteration += 1
            return result

        layout = tuple(views)
        mem = self.buckets.get(bucket_index)
        if mem is not None and mem.layout != layout:
            if hp.use_error_feedback or hp.warm_start:
                raise LayoutChanged(f"bucket {bucket_index} changed its layout")
            mem = None
        if mem is None:
            mem = _BucketMemory(layout=layout)
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
        if is_last:
            self.iteration += 1
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
        if found_inf:
            if is_last:
                self.iteration += 1
            return StepResult(output=bucket.copy(), output64=x64, found_inf=True,
                              skipped=True, passthrough=False)
        g_all = x64 * float(inv_loss_scale) if is_fp16 else x64
        result = StepResult(output=bucket, output64=g_all.copy(), found_inf=False,
                            skipped=False, passthrough=False)
        if self.iteration < hp.start_powerSGD_iter:
            result.passthrough = True
            result.output = g_all.astype(bucket.dtype) if is_fp16 else bucket.copy()
            if is_last:
                self.iteration += 1
            return result
        layout = ("batched", numel)
        mem = self.buckets.get(bucket_index)
        if mem is not None and mem.layout != layout:
            if hp.use_error_feedback or hp.warm_start:
                raise LayoutChanged(f"bucket {bucket_index} changed its layout")
            mem = None
        if mem is None:
            mem = _BucketMemory(layout=layout)
            self.buckets[bucket_index] = mem
        s = batched_side(numel)
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
        if is_last:
            self.iteration += 1
        return result

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
