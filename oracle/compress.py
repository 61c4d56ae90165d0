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

Base subsampling (``subsample_base=True``), the alternative size rule: the
pages quote coresets of about sqrt(S) points, which the recursion above gives
for S a power of four but not for S = 3136 = 4^3 * 49 (392 = 7 sqrt(S)).
Reading taken: before the Compress, every base block is stratified: each run
of r consecutive points keeps one uniformly drawn point, r the largest
divisor of s0 with r^2 <= s0 and s0 / r >= 4^g (r = 1 leaves the list
alone; so does j = 0).  Stratum t keeps point t r + min(floor(u r), r - 1),
u = uniform(t, 0, unit, TAG_BASE_SAMPLE, seed).  The Compress then runs on
the L = S / r kept points by the rule above (depth and decision log those of
L), and each coreset point carries weight r 2^j, so the weights still sum to
S; with s0 = r^2 the coreset has sqrt(S) points (56 for S = 3136).  Pins:
sizes (56 / 14 / 12 for S = 3136 / 196 / 144), weights summing to S, one
point per stratum inside it, uniform offsets, r = 1 equal to the plain rule.
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


def base_stride(S, g=0, subsample_base=False):
    """Stratum length r of base subsampling (1 when it is off or changes nothing)."""
    if not subsample_base:
        return 1
    j, s0 = compress_depth(S, g)
    if j == 0:
        return 1
    return max(r for r in range(1, s0 + 1) if s0 % r == 0 and r * r <= s0 and s0 // r >= 4 ** g)


def thinned_length(S, g=0, subsample_base=False):
    """Length of the list the Compress runs on (S, or S / r after base subsampling)."""
    return S // base_stride(S, g, subsample_base)


def base_sample(S, r, seed, unit):
    """Positions kept by base subsampling: one per stratum of r, ascending."""
    out = np.empty(S // r, dtype=np.int64)
    for t in range(S // r):
        u = philox.uniform(t, 0, unit, philox.TAG_BASE_SAMPLE, seed)
        out[t] = t * r + min(int(np.floor(u * r)), r - 1)
    return out


def coreset_size(S, g=0, subsample_base=False):
    L = thinned_length(S, g, subsample_base)
    j, _ = compress_depth(L, g)
    return L >> j


def decisions_per_unit(S, g=0, subsample_base=False):
    """Number of halving decisions of one unit (sum over levels)."""
    S = thinned_length(S, g, subsample_base)
    j, s0 = compress_depth(S, g)
    total = 0
    for level in range(1, j + 1):
        bins = S // (4 ** level * s0)
        pairs = (4 * s0 * 2 ** (level - 1)) // 2
        total += bins * pairs
    return total


def thin_unmasked(K, V, scale, delta, seed, unit, g=0, override=None,
                  stats=None, greedy=False, subsample_base=False):
    """Coreset of one unit: (idx ascending int64 [n_out], weight, log).

    K [S, E], V [S, D] float64.  ``log`` maps (level, bin) to the kept-first
    booleans of that halving; ``override`` has the same layout and forces
    another implementation's decisions (replay).
    """
    S = K.shape[0]
    r = base_stride(S, g, subsample_base)
    if r > 1:
        pos = base_sample(S, r, seed, unit)
        idx, w, log = thin_unmasked(K[pos], V[pos], scale, delta, seed, unit, g, override=override,
                                    stats=stats, greedy=greedy)
        return pos[idx], w * r, log
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
