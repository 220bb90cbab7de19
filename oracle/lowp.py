"""Half-precision rounding and the PowerSGD matrix step in 16-bit storage (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "DDP Communication Hooks -- PyTorch 1.11.0", section "Default Communication
Hooks": fp16_compress_wrapper / bf16_compress_wrapper cast the gradient handed to a
hook to torch.float16 / torch.bfloat16 and cast the hook's result back to the input
dtype; wrapped around powerSGD_hook ("PowerSGD Hooks", steps 1 to 3.7) the hook then
works on a 16-bit tensor.

READING: every tensor the hook materializes is 16-bit (the bucket, M' = G + E, P
after the product and after Gram-Schmidt, Q, M_hat = P Q^T, E = M' - M_hat, the
initial draw of Q): each is the correctly rounded (nearest, ties to even) 16-bit value
of the exact result of its step on 16-bit operands. The oracle evaluates every step
in fp64 and rounds once; the cast back to fp32 is exact.
"""
from __future__ import annotations

import numpy as np

from .powersgd import gram_schmidt

# bfloat16: 8 significant bits, the exponent range of binary32
_BF16_MAX = float.fromhex("0x1.fep127")          # (2 - 2^-7) * 2^127
_BF16_OVERFLOW = float.fromhex("0x1.ffp127")     # max + half an ulp: rounds to inf
_BF16_MIN_EXP = -133                             # spacing of the subnormals, 2^-133


def round_f16(x) -> np.ndarray:
    """Nearest binary16 value (ties to even), as float64; overflow gives +-inf.

    numpy converts binary64 to binary16 directly (one rounding); the pins check that
    against hand-worked ties where rounding through binary32 first would differ."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even), as float64, from the definition: keep 8
    significant bits of a normal number (a fixed spacing of 2^-133 below 2^-126),
    round half to even, and give +-inf from (2 - 2^-8) * 2^127 up. NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    xf = x[fin]
    _, e = np.frexp(xf)                          # |xf| = f * 2^e, f in [0.5, 1)
    step = np.maximum(e - 8, _BF16_MIN_EXP)      # exponent of the ulp
    q = np.rint(np.ldexp(xf, -step))             # exact scaling; rint: half to even
    r = np.ldexp(q, step)
    r = np.where(np.abs(xf) >= _BF16_OVERFLOW, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out


ROUNDERS = {"f16": round_f16, "bf16": round_bf16}


def compress_matrix_step_lowp(g16: np.ndarray, e_prev: np.ndarray | None, q16: np.ndarray,
                              epsilon: float, use_error_feedback: bool, rnd):
    """Steps 3.2 to 3.7 of powerSGD_hook for one n x m matrix held in 16 bits.

    g16: the 16-bit gradient; e_prev: the 16-bit error memory (None = zero); q16: the
    16-bit starting Q (warm, or an orthogonalized draw); rnd: round_f16 or round_bf16.
    Returns (m_prime, p, q_new, m_hat, err), every one 16-bit valued (err None
    without error feedback).
    """
    m_prime = rnd(g16 + e_prev) if (use_error_feedback and e_prev is not None) else g16
    p = rnd(m_prime @ q16)                       # 3.2  P = M Q
    p = rnd(gram_schmidt(p, epsilon))            # 3.4
    q_new = rnd(m_prime.T @ p)                   # 3.5  Q = M^T P
    m_hat = rnd(p @ q_new.T)                     # 3.7  M ~ P Q^T
    err = rnd(m_prime - m_hat) if use_error_feedback else None
    return m_prime, p, q_new, m_hat, err
