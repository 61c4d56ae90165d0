"""Unmasked Thinformer coreset by recursive four-way Compress, float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "Thinformer" README (introduction) and "Express Language Modeling"
(section "Problem Statement") name Thinformer as the thinning approximation
of unmasked attention but give no schedule.  The reading taken is the
KT-Compress-style recursion:

* depth j = max{ j : 4^j divides S and S / 4^j >= 4^g }  (g = oversampling,
  0 by default); base blocks of s0 = S / 4^j consecutive tokens;
* Compress(block of 4^l * s0 tokens) = the block itself for l = 0; otherwise
  Compress each of its four contiguous quarters, concatenate the four results
  in order and apply one kernel halving to the concatenation;
* the coreset has n_out = S / 2^j points, each of weight 2^j, so the weights
  sum to S.

Bin id of the halving of the block starting at token t on level l:
(l << 20) | (t / (4^l * s0)); tag 0.  Decision logs are ordered by level
(ascending), then bin (ascending), then pair.

Pins: the size rule (n_out 16 / 392 / 64 for S = 256 / 3136 / 4096), weights
summing to S, indices ascending and unique with one point of every pair,
and exact attention when thinning is disabled (4^g >= S gives j = 0).
"""

import numpy as np

from . import kernel_halving as khm
from . import philox


def compress_depth(S, g=0):
    """Return (j, s0) of the recursion for S tokens and oversampling g."""
    j = 0
    while S % (4 ** (j + 1)) == 0 and S // (4 ** (j + 1)) >= 4 ** g:
        j += 1
    return j, S // (4 ** j)


def coreset_size(S, g=0):
    j, _ = compress_depth(S, g)
    return S >> j


def decisions_per_unit(S, g=0):
    """Number of halving decisions of one unit (sum over levels)."""
    j, s0 = compress_depth(S, g)
    total = 0
    for level in range(1, j + 1):
        bins = S // (4 ** level * s0)
        pairs = (4 * s0 * 2 ** (level - 1)) // 2
        total += bins * pairs
    return total


def thin_unmasked(K, V, scale, delta, seed, unit, g=0, override=None,
                  stats=None, greedy=False):
    """Coreset of one unit: (idx ascending int64 [n_out], weight, log).

    K [S, E], V [S, D] float64.  ``log`` maps (level, bin) to the kept-first
    booleans of that halving; ``override`` has the same layout and forces
    another implementation's decisions (replay).
    """
    S = K.shape[0]
    j, s0 = compress_depth(S, g)
    log = {}

    def compress(start, level):
        if level == 0:
            return np.arange(start, start + s0, dtype=np.int64)
        quarter = (4 ** (level - 1)) * s0
        children = [compress(start + c * quarter, level - 1) for c in range(4)]
        pts = np.concatenate(children)
        bin_id = (level << 20) | (start // (4 ** level * s0))
        ov = None if override is None else override[(level, start // (4 ** level * s0))]
        keep_first, _ = khm.kernel_halving(K[pts], V[pts], scale, delta, seed,
                                           unit, bin_id, philox.TAG_COMPRESS,
                                           override=ov, stats=stats, greedy=greedy)
        log[(level, start // (4 ** level * s0))] = keep_first
        return pts[khm.kept_positions(keep_first)]

    idx = compress(0, j)
    return idx, float(2 ** j), log


def log_to_flat(log, S, g=0):
    """Flatten a Compress decision log into the library's order (uint8, 1 = first kept)."""
    j, s0 = compress_depth(S, g)
    parts = []
    for level in range(1, j + 1):
        for b in range(S // (4 ** level * s0)):
            parts.append(np.asarray(log[(level, b)], dtype=np.uint8))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.uint8)


def flat_to_log(flat, S, g=0):
    """Inverse of log_to_flat: split a flat decision array into per-bin arrays."""
    j, s0 = compress_depth(S, g)
    out = {}
    pos = 0
    for level in range(1, j + 1):
        pairs = (4 * s0 * 2 ** (level - 1)) // 2
        for b in range(S // (4 ** level * s0)):
            out[(level, b)] = np.asarray(flat[pos:pos + pairs]).astype(bool)
            pos += pairs
    assert pos == len(flat)
    return out
