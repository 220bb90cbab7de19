"""Pins for the oracle's counter-based normal generator (oracle/rng.py).

Philox4x64-10 is checked against numpy's own, independently written Philox bit
generator; the 128-bit multiply against Python's exact integers; Box-Muller at
points where it has a closed form and in distribution.
"""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import box_muller, mulhilo64, philox4x64_10, standard_normal_q0

MASK64 = (1 << 64) - 1


def _numpy_philox_block(counter, key):
    """numpy's Philox returns the block of (its counter + 1) first."""
    c = list(counter)
    # subtract one from the 256-bit counter, with borrow
    for i in range(4):
        if c[i] > 0:
            c[i] -= 1
            break
        c[i] = MASK64
    bg = np.random.Philox(counter=np.array(c, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("counter,key", [
    ((1, 0, 0, 0), (0, 0)),
    ((0, 0, 0, 0), (0, 0)),                    # exercises the borrow across words
    ((12345, 7, 3, 0), (0xDEADBEEF, 42)),
    ((MASK64, MASK64, MASK64, 5), (MASK64, MASK64)),
    ((2 ** 40 + 17, 2 ** 63, 1, 2), (2 ** 62 + 3, 9)),
])
def test_philox_matches_numpy(counter, key):
    ours = [int(x) for x in philox4x64_10(*counter, *key)]
    assert ours == _numpy_philox_block(counter, key)


def test_philox_vectorized_matches_numpy_many():
    rng = np.random.default_rng(5)
    c = rng.integers(1, 2 ** 63, size=(64, 4), dtype=np.uint64)
    k = rng.integers(0, 2 ** 63, size=(64, 2), dtype=np.uint64)
    out = philox4x64_10(c[:, 0], c[:, 1], c[:, 2], c[:, 3], k[:, 0], k[:, 1])
    for i in range(64):
        expect = _numpy_philox_block([int(v) for v in c[i]], [int(v) for v in k[i]])
        assert [int(o[i]) for o in out] == expect


def test_mulhilo_matches_python_integers():
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.integers(0, 2 ** 64 - 1, size=1000, dtype=np.uint64,
                                     endpoint=True),
                        np.array([0, 1, MASK64, 2 ** 32, 2 ** 32 - 1], dtype=np.uint64)])
    b = np.concatenate([rng.integers(0, 2 ** 64 - 1, size=1000, dtype=np.uint64,
                                     endpoint=True),
                        np.array([MASK64, MASK64, MASK64, 2 ** 32, 2 ** 32 + 1],
                                 dtype=np.uint64)])
    hi, lo = mulhilo64(a, b)
    for x, y, h, l in zip(a, b, hi, lo):
        prod = int(x) * int(y)
        assert int(h) == prod >> 64 and int(l) == prod & MASK64


def test_box_muller_closed_form_points():
    # u = 0.5 (top 53 bits = 2**52 - 1), v = 0: z0 = sqrt(2 ln 2), z1 = 0
    z0, z1 = box_muller(np.uint64((2 ** 52 - 1) << 11), np.uint64(0))
    assert z0 == pytest.approx(math.sqrt(2 * math.log(2)), rel=1e-15)
    assert z1 == 0.0
    # v = 1/4: the angle is pi/2, so z0 ~ 0 and z1 = radius
    z0, z1 = box_muller(np.uint64((2 ** 52 - 1) << 11), np.uint64(2 ** 51 << 11))
    assert abs(z0) < 1e-15
    assert z1 == pytest.approx(math.sqrt(2 * math.log(2)), rel=1e-15)
    # u = 1 exactly (top bits all ones): radius 0
    z0, z1 = box_muller(np.uint64(MASK64), np.uint64(12345 << 11))
    assert z0 == 0.0 and z1 == 0.0
    # the low 11 bits are discarded
    a = box_muller(np.uint64((77 << 11) | 0x7FF), np.uint64((99 << 11) | 0x3))
    b = box_muller(np.uint64(77 << 11), np.uint64(99 << 11))
    assert a == b


def test_q0_distribution_is_standard_normal():
    q = standard_normal_q0(50000, 4, random_seed=3, bucket_index=1, view=2, epoch=0)
    flat = q.reshape(-1)
    assert abs(flat.mean()) < 0.01
    assert abs(flat.var() - 1.0) < 0.01
    assert stats.kstest(flat, "norm").pvalue > 1e-3
    # each of the four output words feeds a normal: check each lane separately
    for lane in range(4):
        assert stats.kstest(flat[lane::4], "norm").pvalue > 1e-4


def test_q0_values_are_binary32():
    q = standard_normal_q0(333, 3, 0, 0, 0, 0)
    assert np.array_equal(q, q.astype(np.float32).astype(np.float64))


def test_q0_counter_layout_prefix_property():
    # entry e of the row-major Q depends only on e, not on m: a taller Q with the
    # same rank starts with the shorter one
    a = standard_normal_q0(37, 4, 9, 2, 5, 0)
    b = standard_normal_q0(80, 4, 9, 2, 5, 0)
    assert np.array_equal(a, b[:37])
    # and a different rank reflows the same stream
    c = standard_normal_q0(74, 2, 9, 2, 5, 0)
    assert np.array_equal(a.reshape(-1)[:148], c.reshape(-1)[:148])


def test_q0_keys_separate_streams():
    base = standard_normal_q0(64, 2, 0, 0, 0, 0)
    for kw in (dict(random_seed=1), dict(bucket_index=1), dict(view=1), dict(epoch=1)):
        args = dict(m=64, r=2, random_seed=0, bucket_index=0, view=0, epoch=0)
        args.update(kw)
        other = standard_normal_q0(**args)
        assert not np.array_equal(base, other)
        # independent streams: essentially uncorrelated
        assert abs(np.corrcoef(base.reshape(-1), other.reshape(-1))[0, 1]) < 0.3
    assert np.array_equal(base, standard_normal_q0(64, 2, 0, 0, 0, 0))


def test_q0_negative_bucket_index_is_twos_complement():
    a = standard_normal_q0(8, 1, 0, -1, 0, 0)
    b = standard_normal_q0(8, 1, 0, 2 ** 64 - 1, 0, 0)
    assert np.array_equal(a, b)
