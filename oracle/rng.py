"""Counter-based normal draws for the oracle's initial Q.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg do.

The pages fix only that Q starts from "a standard normal distribution" and that a
`random_seed` hyperparameter exists (DDP Communication Hooks, PyTorch 1.11, section
"PowerSGD Hooks", powerSGD_hook step 3.1; section "PowerSGD State", constructor
signature). They name no generator. Both sides of the parity check therefore
implement, independently, the same published counter-based generator:

* Philox4x64-10 from Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
  easy as 1, 2, 3" (SC 2011): a 4-word counter, a 2-word key, ten rounds of two
  64x64->128-bit multiplies, with a Weyl-sequence key bump between rounds.
* Box-Muller (Box and Muller, 1958) in binary64, rounded to binary32.

The mapping of Q entries to counters is this repository's own convention:
entry e of the row-major (m x r) Q of view `view` in bucket `bucket_index` is
output word (e mod 4) of Philox4x64-10 with
    counter = (e div 4, view, epoch, 0),  key = (random_seed, bucket_index),
and the four words (w0, w1, w2, w3) of one block give two Box-Muller pairs,
(w0, w1) -> (z0, z1) and (w2, w3) -> (z2, z3), with
    u = ((w_even >> 11) + 1) * 2**-53   in (0, 1]
    v = (w_odd >> 11) * 2**-53          in [0, 1)
    z_even = sqrt(-2 ln u) cos(2 pi v),  z_odd = sqrt(-2 ln u) sin(2 pi v).
"""
from __future__ import annotations

import numpy as np

_U64 = np.uint64
_MASK32 = _U64(0xFFFFFFFF)

# Philox4x64 round multipliers and key-schedule (Weyl) increments, as published.
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
PHILOX_ROUNDS = 10


def mulhilo64(a, b):
    """Full 128-bit product of two uint64 arrays, returned as (high, low) words.

    Schoolbook multiplication on 32-bit halves; every partial sum stays below 2**64.
    """
    a = np.asarray(a, dtype=_U64)
    b = np.asarray(b, dtype=_U64)
    a0, a1 = a & _MASK32, a >> _U64(32)
    b0, b1 = b & _MASK32, b >> _U64(32)
    p00 = a0 * b0
    p01 = a0 * b1
    p10 = a1 * b0
    p11 = a1 * b1
    mid = (p00 >> _U64(32)) + (p01 & _MASK32) + (p10 & _MASK32)
    lo = (p00 & _MASK32) | ((mid & _MASK32) << _U64(32))
    hi = p11 + (p01 >> _U64(32)) + (p10 >> _U64(32)) + (mid >> _U64(32))
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Philox4x64 with ten rounds on broadcastable uint64 arrays.

    Returns the four output words. Round i uses key (k0 + i*W0, k1 + i*W1) mod 2**64;
    one round maps (x0, x1, x2, x3) to
        (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0)).
    """
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=_U64) for c in (c0, c1, c2, c3))
        k0 = np.asarray(k0, dtype=_U64)
        k1 = np.asarray(k1, dtype=_U64)
        m0, m1 = _U64(PHILOX_M0), _U64(PHILOX_M1)
        for rnd in range(PHILOX_ROUNDS):
            if rnd:
                k0 = k0 + _U64(PHILOX_W0)
                k1 = k1 + _U64(PHILOX_W1)
            hi0, lo0 = mulhilo64(m0, x0)
            hi1, lo1 = mulhilo64(m1, x2)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def box_muller(w_even, w_odd):
    """Two standard normals (binary64) from two uint64 words, as described above."""
    w_even = np.asarray(w_even, dtype=_U64)
    w_odd = np.asarray(w_odd, dtype=_U64)
    u = ((w_even >> _U64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    v = (w_odd >> _U64(11)).astype(np.float64) * 2.0 ** -53
    radius = np.sqrt(-2.0 * np.log(u))
    angle = 2.0 * np.pi * v
    return radius * np.cos(angle), radius * np.sin(angle)


def _as_u64(x: int) -> np.uint64:
    return _U64(int(x) & 0xFFFFFFFFFFFFFFFF)


def standard_normal_q0(m: int, r: int, random_seed: int, bucket_index: int,
                       view: int, epoch: int) -> np.ndarray:
    """The (m x r) initial Q of one view, as binary32 values held in float64."""
    count = m * r
    if count == 0:
        return np.zeros((m, r), dtype=np.float64)
    nblocks = (count + 3) // 4
    block = np.arange(nblocks, dtype=_U64)
    w = philox4x64_10(block, _as_u64(view), _as_u64(epoch), _U64(0),
                      _as_u64(random_seed), _as_u64(bucket_index))
    z0, z1 = box_muller(w[0], w[1])
    z2, z3 = box_muller(w[2], w[3])
    z = np.stack([z0, z1, z2, z3], axis=1).reshape(-1)[:count]
    return z.astype(np.float32).astype(np.float64).reshape(m, r)
