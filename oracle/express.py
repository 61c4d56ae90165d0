"""EXPRESS weighted cache and Thinformer Express, float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "Express Language Modeling", section "Methodology / The EXPRESS
Meta-Procedure" (cache object with target size n_out, inflation factor m
and a base halving; exact, thin and HALVE phases; size bound 6 n_out) and
section "Thinformer Express" (base halving = kernel halving under
kappa_att).  Where the pages leave a step open the reading is:

* n_out defaults to the smallest power of two p >= 2 with p^2 >= S; tokens
  are ingested in blocks of n_out consecutive tokens.
* m starts at 1.  While m = 1 each block is appended to the cache unchanged
  (weight 1): the exact phase.
* While m >= 4 the thin phase runs: with r = m / 2, every aligned group of r
  tokens completed by the block contributes one representative, the token at
  offset floor(u * r) (u from the Philox stream, counter (group, log2 r,
  unit, 4)), with weight r (uniform subsampling).  When the buffer holds
  2 n_out representatives, one kernel halving (tag 1, bin = batch ordinal)
  thins it to n_out points of weight m, which are appended to the cache
  (COMPRESS2 read as one halving).
* Whenever the cache holds 4 n_out points it is halved twice (tags 2 then 3,
  bin = HALVE ordinal) back to n_out points, and m becomes 4 m.
* A query at token t in block beta = t // n_out sees the cache and buffer as
  they stood after blocks 0 .. beta-1, plus the raw tokens beta*n_out .. t
  with weight 1.
* Groups longer than a block (r = m / 2 > n_out, reached once t passes about
  2 n_out^2): a group contributes its representative when the block that
  completes the group is ingested (the representative itself may lie in an
  earlier block of the group).  The tokens of a group still in progress are
  then in no weight until it completes, so the weights a query sees sum to
  t + 1 - ((beta n_out) mod r) (exactly t + 1 whenever r divides n_out); the
  cache keeps its size bound regardless of the length, as EXPRESS states.
* A trailing partial block is never thinned.
* Lists are kept in token order; the decision log is ordered by the halvings'
  chronological order.

Pins: the HALVE positions (after 4, 16, 64, ... blocks) and the values of m;
exact causal attention for t < 4 n_out and for n_out >= S; visible set
below 6 n_out; weights summing to t + 1 (less the tokens of a group in
progress); streaming == prefill.
"""

import math

import numpy as np

from . import kernel_halving as khm
from . import philox


def default_cache_size(S):
    p = 2
    while p * p < S:
        p *= 2
    return p


class ExpressCache:
    """The EXPRESS weighted cache of one unit (one batch entry and KV head)."""

    def __init__(self, n_out, K, V, scale, delta, seed, unit,
                 override=None, stats=None, greedy=False):
        assert n_out >= 2 and (n_out & (n_out - 1)) == 0
        self.n_out = n_out
        self.K, self.V = K, V
        self.scale, self.delta, self.seed, self.unit = scale, delta, seed, unit
        self.override = override
        self.greedy = greedy
        self.stats = stats
        self.m = 1
        self.cache = np.zeros(0, dtype=np.int64)
        self.buffer = []
        self.blocks = 0
        self.n_batch = 0
        self.n_halve = 0
        self.log = []          # [((tag, bin), keep_first)] in chronological order

    # --- the base halving under kappa_att --------------------------------
    def _halve(self, pts, tag, bin_id):
        ov = None if self.override is None else self.override[(tag, bin_id)]
        keep_first, _ = khm.kernel_halving(self.K[pts], self.V[pts], self.scale,
                                           self.delta, self.seed, self.unit,
                                           bin_id, tag, override=ov,
                                           stats=self.stats, greedy=self.greedy)
        self.log.append(((tag, bin_id), keep_first))
        return pts[khm.kept_positions(keep_first)]

    # --- one block of n_out raw tokens -----------------------------------
    def ingest_block(self, start):
        n = self.n_out
        assert start == self.blocks * n
        if self.m == 1:
            self.cache = np.concatenate([self.cache, np.arange(start, start + n)])
        else:
            r = self.m // 2
            log2r = r.bit_length() - 1
            # the groups this block completes (r > n: at most one, possibly begun blocks ago)
            for g in range(start // r, (start + n) // r):
                off = philox.uniform_offset(g, log2r, self.unit,
                                            philox.TAG_SUBSAMPLE, self.seed, r)
                self.buffer.append(g * r + off)
                if len(self.buffer) == 2 * n:
                    kept = self._halve(np.array(self.buffer, dtype=np.int64),
                                       philox.TAG_BATCH, self.n_batch)
                    self.n_batch += 1
                    self.cache = np.concatenate([self.cache, kept])
                    self.buffer = []
        if len(self.cache) == 4 * n:
            once = self._halve(self.cache, philox.TAG_HALVE_FIRST, self.n_halve)
            self.cache = self._halve(once, philox.TAG_HALVE_SECOND, self.n_halve)
            self.m *= 4
            self.n_halve += 1
        self.blocks += 1

    # --- what a query sees -----------------------------------------------
    def summary(self):
        """(idx, w) of the cache and buffer as they stand now."""
        idx = np.concatenate([self.cache, np.array(self.buffer, dtype=np.int64)])
        w = np.concatenate([np.full(len(self.cache), float(self.m)),
                            np.full(len(self.buffer), float(self.m // 2))])
        return idx, w

    def visible(self, t):
        """Visible (idx, w) of query t, which must lie in the next block."""
        start = self.blocks * self.n_out
        assert start <= t < start + self.n_out
        idx, w = self.summary()
        raw = np.arange(start, t + 1, dtype=np.int64)
        return (np.concatenate([idx, raw]),
                np.concatenate([w, np.ones(len(raw))]))


def schedule(S, n_out):
    """Static halving schedule: list of (tag, bin, pairs) in chronological order.

    Depends only on S and n_out (representatives and halvings are placed by
    token counts, never by data).
    """
    events = []
    m, cache, buf, nb, nh = 1, 0, 0, 0, 0
    for blk in range(S // n_out):
        if m == 1:
            cache += n_out
        else:
            r = m // 2
            start = blk * n_out
            for _ in range((start + n_out) // r - start // r):   # groups completed by this block
                buf += 1
                if buf == 2 * n_out:
                    events.append((philox.TAG_BATCH, nb, n_out))
                    nb += 1
                    cache += n_out
                    buf = 0
        if cache == 4 * n_out:
            events.append((philox.TAG_HALVE_FIRST, nh, 2 * n_out))
            events.append((philox.TAG_HALVE_SECOND, nh, n_out))
            cache = n_out
            m *= 4
            nh += 1
    return events


def log_to_flat(log):
    parts = [np.asarray(kf, dtype=np.uint8) for _, kf in log]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.uint8)


def flat_to_log(flat, S, n_out):
    """Split a flat decision array into {(tag, bin): keep_first} by the schedule."""
    out = {}
    pos = 0
    for tag, b, pairs in schedule(S, n_out):
        out[(tag, b)] = np.asarray(flat[pos:pos + pairs]).astype(bool)
        pos += pairs
    assert pos == len(flat), (pos, len(flat))
    return out


def run_unit(K, V, n_out, scale, delta, seed, unit, query_positions=None,
             override=None, stats=None, greedy=False):
    """Thinformer Express over one unit's S tokens.

    Returns (visible, final, log):
    * visible: {t: (idx, w)} for each t in query_positions (all t if None);
    * final: (idx, w) of cache, buffer and the trailing partial block;
    * log: the chronological decision log.
    """
    S = K.shape[0]
    cache = ExpressCache(n_out, K, V, scale, delta, seed, unit,
                         override=override, stats=stats, greedy=greedy)
    wanted = None if query_positions is None else set(int(t) for t in query_positions)
    visible = {}
    n_blocks = math.ceil(S / n_out)
    for beta in range(n_blocks):
        lo, hi = beta * n_out, min((beta + 1) * n_out, S)
        for t in range(lo, hi):
            if wanted is None or t in wanted:
                visible[t] = cache.visible(t)
        if hi - lo == n_out:
            cache.ingest_block(lo)
    idx, w = cache.summary()
    tail = np.arange(cache.blocks * n_out, S, dtype=np.int64)
    final = (np.concatenate([idx, tail]), np.concatenate([w, np.ones(len(tail))]))
    return visible, final, cache.log


def run_unit_blocks(K, V, n_out, scale, delta, seed, unit, override=None, stats=None, greedy=False):
    """Thinformer Express over one unit's S tokens, reporting per block instead of per query.

    Returns (blocks, final, log): blocks is a list of (lo, hi, idx, w), the
    state (cache and buffer) that the queries at tokens lo .. hi-1 of one
    block see besides the raw tokens of their block; final and log as in
    run_unit.
    """
    S = K.shape[0]
    cache = ExpressCache(n_out, K, V, scale, delta, seed, unit,
                         override=override, stats=stats, greedy=greedy)
    blocks = []
    for beta in range(math.ceil(S / n_out)):
        lo, hi = beta * n_out, min((beta + 1) * n_out, S)
        idx, w = cache.summary()
        blocks.append((lo, hi, idx, w))
        if hi - lo == n_out:
            cache.ingest_block(lo)
    idx, w = cache.summary()
    tail = np.arange(cache.blocks * n_out, S, dtype=np.int64)
    final = (np.concatenate([idx, tail]), np.concatenate([w, np.ones(len(tail))]))
    return blocks, final, cache.log
