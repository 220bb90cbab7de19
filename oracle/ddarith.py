"""Double-double arithmetic on numpy float64 arrays, for the oracle's Gram-Schmidt.

TEST INFRASTRUCTURE ONLY (imported by oracle.powersgd; never by the product path).

A double-double value is an unevaluated sum hi + lo of two binary64 numbers with
|lo| <= ulp(hi) / 2, which carries about 106 significant bits. The building blocks are
the classical error-free transformations:

* TwoSum (Knuth, The Art of Computer Programming vol. 2, 4.2.2, Theorem B): s + e =
  a + b exactly, s = fl(a + b);
* Dekker's splitting and TwoProduct (Dekker, "A floating-point technique for extending
  the available precision", Numer. Math. 18, 1971): a = hi + lo with 26-bit halves, and
  p + e = a * b exactly, p = fl(a * b).

numpy never contracts a * b + c into a fused multiply-add, so the splitting formulas
hold as written. Sums of many terms use a pairwise tree of TwoSums whose rounding
errors are kept and added at the end, which gives the sum as if computed with twice
the working precision (Ogita, Rump and Oishi, "Accurate sum and dot product", SIAM J.
Sci. Comput. 26, 2005, algorithm Sum2, arranged as a tree). Scalars (a norm, its
reciprocal) go through Python's decimal module at 60 digits.
"""
from __future__ import annotations

import decimal
import math

import numpy as np

_SPLITTER = 134217729.0  # 2**27 + 1
_CTX = decimal.Context(prec=60)


def two_sum(a, b):
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    return s, e


def fast_two_sum(a, b):
    """Requires |a| >= |b| (or a == 0)."""
    s = a + b
    return s, b - (s - a)


def split(a):
    c = _SPLITTER * a
    hi = c - (c - a)
    return hi, a - hi


def two_prod(a, b):
    p = a * b
    ah, al = split(a)
    bh, bl = split(b)
    e = ((ah * bh - p) + ah * bl + al * bh) + al * bl
    return p, e


def dd_add(ah, al, bh, bl):
    s, e = two_sum(ah, bh)
    t, f = two_sum(al, bl)
    e = e + t
    s, e = fast_two_sum(s, e)
    e = e + f
    return fast_two_sum(s, e)


def dd_mul(ah, al, bh, bl):
    p, e = two_prod(ah, bh)
    e = e + (ah * bl + al * bh)
    return fast_two_sum(p, e)


def dd_sum(h, l):
    """The sum of the double-double vector (h, l) as a double-double scalar."""
    h = np.asarray(h, dtype=np.float64).ravel()
    l = np.asarray(l, dtype=np.float64).ravel()
    errs = [l]
    while h.size > 1:
        if h.size % 2:
            h = np.append(h, 0.0)
        s, e = two_sum(h[0::2], h[1::2])
        errs.append(e)
        h = s
    head = float(h[0]) if h.size else 0.0
    tail = float(sum(float(np.sum(e)) for e in errs))
    if not (math.isfinite(head) and math.isfinite(tail)):
        return head + tail, 0.0
    s, e = fast_two_sum(head, tail) if abs(head) >= abs(tail) else fast_two_sum(tail, head)
    return float(s), float(e)


def dd_dot(xh, xl, yh, yl):
    """sum_i (xh_i + xl_i)(yh_i + yl_i) as a double-double scalar: the products of the
    high parts exactly, the cross terms in binary64 (they are 2^-53 smaller)."""
    p, e = two_prod(xh, yh)
    e = e + (xh * yl + xl * yh)
    return dd_sum(p, e)


def to_decimal(hi: float, lo: float) -> decimal.Decimal:
    return _CTX.add(decimal.Decimal(hi), decimal.Decimal(lo))


def from_decimal(d: decimal.Decimal):
    hi = float(d)
    lo = float(_CTX.subtract(d, decimal.Decimal(hi))) if math.isfinite(hi) else 0.0
    return hi, lo


def inverse_norm_plus(hh: float, hl: float, epsilon: float):
    """1 / (sqrt(hh + hl) + epsilon) as a double-double: the reciprocal of a column norm
    plus epsilon. A zero denominator gives inf (so a zero column becomes 0 * inf =
    NaN, as in binary64); non-finite input gives NaN."""
    if not (math.isfinite(hh) and math.isfinite(hl)):
        return math.nan, 0.0
    nn = to_decimal(hh, hl)
    if nn < 0:
        nn = decimal.Decimal(0)
    den = _CTX.add(_CTX.sqrt(nn), decimal.Decimal(epsilon))
    if den == 0:
        return math.inf, 0.0
    return from_decimal(_CTX.divide(decimal.Decimal(1), den))
