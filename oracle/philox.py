"""Philox4x64-10 counter-based generator, pure-Python integers (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3" (SC'11), the Philox-4x64 bijection with 10 rounds.  One round maps
counter words (x0, x1, x2, x3) with key (k0, k1) to

    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))

and the key is then bumped by the Weyl constants (W0, W1) modulo 2^64.

Pin: ``tests/test_oracle_philox.py`` compares this function with NumPy's
``numpy.random.Philox`` (a separate library implementation of the same
bijection) on many counters and keys.

Stream layout used by the thinning path (the pages fix none; this is the
reading recorded for the random choices, keyed by seed, unit and bin):
    counter = (c0, c1, c2, c3), key = (seed, 0)
    c0 = pair index (halving) or group index (subsampling)
    c1 = bin id  (Compress: level << 20 | bin-in-level; Express: batch or
                  HALVE ordinal; subsampling: log2 of the group size)
    c2 = unit = b * H_kv + h_kv
    c3 = tag  (0 Compress halving, 1 Express batch halving, 2 / 3 first /
               second halving of a HALVE, 4 subsampling)
A uniform is u = (word0 >> 11) * 2^-53, exact in float64, in [0, 1).
"""

MASK64 = (1 << 64) - 1

# Philox-4x64 multipliers and Weyl key increments (SC'11 paper).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B

TAG_COMPRESS = 0
TAG_BATCH = 1
TAG_HALVE_FIRST = 2
TAG_HALVE_SECOND = 3
TAG_SUBSAMPLE = 4
TAG_BASE_SAMPLE = 5


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for a 4-word counter and 2-word key."""
    x = [int(c) & MASK64 for c in counter]
    k0, k1 = int(key[0]) & MASK64, int(key[1]) & MASK64
    for _ in range(10):
        p0 = PHILOX_M0 * x[0]
        p1 = PHILOX_M1 * x[2]
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        x = [hi1 ^ x[1] ^ k0, lo1, hi0 ^ x[3] ^ k1, lo0]
        k0 = (k0 + PHILOX_W0) & MASK64
        k1 = (k1 + PHILOX_W1) & MASK64
    return x


def uniform(c0, c1, c2, c3, seed):
    """u in [0, 1): the top 53 bits of word 0, scaled by 2^-53 (exact)."""
    w0 = philox4x64_10((c0, c1, c2, c3), (seed, 0))[0]
    return float(w0 >> 11) * (2.0 ** -53)


def uniform_offset(c0, c1, c2, c3, seed, r):
    """floor(u * r) for a power-of-two r (exact: u * r is a float64 scaling)."""
    assert r >= 1 and (r & (r - 1)) == 0
    return int(uniform(c0, c1, c2, c3, seed) * r)
