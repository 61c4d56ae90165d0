"""Pins of the oracle's Philox4x64-10 against NumPy's independent implementation."""

import numpy as np
import pytest

from oracle import philox

MASK = (1 << 64) - 1


def numpy_philox_block(counter, key):
    """Output block of NumPy's Philox for exactly this counter.

    NumPy's generator increments its 256-bit counter before each block, so it
    is started one below the wanted counter (with borrow across words).
    """
    c = counter[0] | (counter[1] << 64) | (counter[2] << 128) | (counter[3] << 192)
    c = (c - 1) % (1 << 256)
    start = np.array([(c >> (64 * i)) & MASK for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=start)
    return [int(x) for x in g.random_raw(4)]


def test_philox_matches_numpy_library():
    rng = np.random.default_rng(1234)
    cases = [((0, 0, 0, 0), (0, 0)), ((MASK, MASK, MASK, MASK), (MASK, MASK)),
             ((1, 2, 3, 4), (5, 6))]
    for _ in range(300):
        c = tuple(int(x) for x in rng.integers(0, 2 ** 64, 4, dtype=np.uint64))
        k = tuple(int(x) for x in rng.integers(0, 2 ** 64, 2, dtype=np.uint64))
        cases.append((c, k))
    # counters the thinning path actually uses: small words
    for i in range(50):
        cases.append(((i, (3 << 20) | 7, 31, 2), (0, 0)))
    for c, k in cases:
        assert philox.philox4x64_10(c, k) == numpy_philox_block(c, k), (c, k)


def test_uniform_range_and_exactness():
    us = [philox.uniform(i, 5, 3, 1, seed=42) for i in range(2000)]
    assert min(us) >= 0.0 and max(us) < 1.0
    for u in us:
        assert float(u * 2 ** 53).is_integer()


def test_uniform_offset_is_floor_of_scaled_uniform():
    for r in (1, 2, 8, 128, 1024):
        for i in range(200):
            u = philox.uniform(i, 3, 0, philox.TAG_SUBSAMPLE, seed=9)
            off = philox.uniform_offset(i, 3, 0, philox.TAG_SUBSAMPLE, 9, r)
            assert 0 <= off < r and off == int(np.floor(u * r))


def test_uniform_chi_square():
    n, bins = 20000, 20
    us = np.array([philox.uniform(i, 1, 2, 3, seed=7) for i in range(n)])
    counts = np.histogram(us, bins=bins, range=(0, 1))[0]
    chi2 = ((counts - n / bins) ** 2 / (n / bins)).sum()
    # 19 degrees of freedom: the 0.9999 quantile is about 49
    assert chi2 < 49.0, chi2


@pytest.mark.parametrize("seed", [0, 1, 2 ** 40 + 3])
def test_streams_differ_by_tag_and_unit(seed):
    a = [philox.uniform(i, 0, 0, 0, seed) for i in range(64)]
    b = [philox.uniform(i, 0, 0, 1, seed) for i in range(64)]
    c = [philox.uniform(i, 0, 1, 0, seed) for i in range(64)]
    assert a != b and a != c and b != c
