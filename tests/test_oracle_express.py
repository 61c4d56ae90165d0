"""Pins of the causal (Thinformer Express) oracle: schedule, exact phases, bounds, streaming."""

import math

import numpy as np
import pytest

from oracle import attention as att
from oracle import express as exp
from oracle import forward as fwd
from oracle import philox


def test_default_cache_size():
    assert exp.default_cache_size(32768) == 256
    assert exp.default_cache_size(131072) == 512
    assert exp.default_cache_size(256) == 16
    assert exp.default_cache_size(3) == 2


def _count(events, tag):
    return sum(1 for e in events if e[0] == tag)


def test_schedule_prefill_32k():
    """n_out = 256: HALVE after blocks 4, 16, 64 (tokens 1024, 4096, 16384), 7 batch halvings."""
    ev = exp.schedule(32768, 256)
    assert _count(ev, philox.TAG_HALVE_FIRST) == 3
    assert _count(ev, philox.TAG_BATCH) == 7
    assert sum(p for _, _, p in ev) == 3 * (512 + 256) + 7 * 256     # 4096 per unit (x32 = 131072)


def test_schedule_kv_131k():
    ev = exp.schedule(131072, 512)
    assert _count(ev, philox.TAG_HALVE_FIRST) == 4
    assert _count(ev, philox.TAG_BATCH) == 9
    assert sum(p for _, _, p in ev) == 4 * (1024 + 512) + 9 * 512    # 10752 per unit (x8 = 86016)


def _tiny(seed, S, E=4, D=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((S, E)) * 0.6, rng.standard_normal((S, D))


def test_cache_phases_and_weights():
    n = 8
    S = n * 64
    K, V = _tiny(0, S)
    c = exp.ExpressCache(n, K, V, 0.5, 0.5, 0, 0)
    halves = []
    for blk in range(S // n):
        c.ingest_block(blk * n)
        if c.n_halve and (not halves or halves[-1][1] != c.n_halve):
            halves.append((blk + 1, c.n_halve))
        idx, w = c.summary()
        # weights sum to the tokens ingested; cache never reaches 4 n_out after an ingest
        assert w.sum() == (blk + 1) * n
        assert len(c.cache) < 4 * n and len(c.buffer) < 2 * n
        assert len(idx) + n < 6 * n                      # what a query can see, below 6 n_out
        assert np.all(np.diff(idx) > 0)
    assert [b for b, _ in halves] == [4, 16, 64]
    assert c.m == 64


def test_exact_phase_gives_exact_causal_attention():
    """Queries before token 4 n_out see every earlier token with weight 1."""
    rng = np.random.default_rng(1)
    S, n = 64, 16
    q = rng.standard_normal((1, S, 2, 8)); k = rng.standard_normal((1, S, 2, 8)); v = rng.standard_normal((1, S, 2, 8))
    out = fwd.forward(q, k, v, causal=True, n_out=n)["out"]
    ref = fwd.exact(q, k, v, causal=True)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_large_cache_disables_thinning():
    rng = np.random.default_rng(2)
    S = 50
    q = rng.standard_normal((1, S, 1, 8)); k = rng.standard_normal((1, S, 1, 8)); v = rng.standard_normal((1, S, 1, 4))
    for n in (64, 256):
        out = fwd.forward(q, k, v, causal=True, n_out=n)["out"]
        assert np.max(np.abs(out - fwd.exact(q, k, v, causal=True))) <= 1e-12


def _pending(t, n):
    """Tokens of a subsampling group still in progress when query t's block began: with
    beta = t // n and m = 4^floor(log4 beta) (m = 1 before block 4), r = m / 2 and the
    group in progress holds (beta n) mod r tokens of the earlier blocks (0 whenever r | n)."""
    beta = t // n
    if beta < 4:
        return 0
    m = 4
    while m * 4 <= beta:
        m *= 4
    return (beta * n) % (m // 2)


@pytest.mark.parametrize("S,n", [(512, 8), (500, 8), (67, 4), (2048 + 17, 32), (2000, 4), (4096 + 9, 16)])
def test_visible_sets(S, n):
    """Every token is in the weights a query sees, except those of a group longer than a
    block that is still in progress (n = 4 from token 64 on, n = 16 from token 1024 on)."""
    K, V = _tiny(3, S)
    vis, final, log = exp.run_unit(K, V, n, 0.5, 0.5, 7, 2)
    for t, (idx, w) in vis.items():
        assert w.sum() == t + 1 - _pending(t, n)
        assert len(idx) < 6 * n
        assert np.all(np.diff(idx) > 0) and idx[-1] == t
    idx, w = final
    assert w.sum() == S - _pending((S // n) * n, n) and np.all(np.diff(idx) > 0)
    assert len(idx) < 6 * n + n
    # the trailing partial block stays exact
    tail = S % n
    if tail:
        assert np.array_equal(idx[-tail:], np.arange(S - tail, S)) and np.all(w[-tail:] == 1)


def test_subsample_representatives():
    """In the thin phase each group of r tokens contributes its Philox-chosen member."""
    n = 4
    K, V = _tiny(4, 40 * n)
    c = exp.ExpressCache(n, K, V, 0.5, 0.5, 3, 5)
    for blk in range(4):
        c.ingest_block(blk * n)
    assert c.m == 4
    c.ingest_block(4 * n)                                  # r = 2: two reps
    for k, g in enumerate(range(4 * n // 2, 5 * n // 2)):
        off = philox.uniform_offset(g, 1, 5, philox.TAG_SUBSAMPLE, 3, 2)
        assert c.buffer[k] == 2 * g + off


def test_flat_log_round_trip():
    S = 8 * 64 + 5
    K, V = _tiny(5, S)
    _, _, log = exp.run_unit(K, V, 8, 0.5, 0.5, 1, 0)
    flat = exp.log_to_flat(log)
    back = exp.flat_to_log(flat, S, 8)
    assert [k for k, _ in log] == list(back.keys())
    assert len(flat) == sum(p for _, _, p in exp.schedule(S, 8))


def test_groups_longer_than_a_block_join_when_complete():
    """n = 4, epoch m = 16 (blocks 16 .. 63): groups of r = 8 tokens span two blocks.  After
    block b the buffer holds one representative per group completed so far, each the
    Philox-chosen member g r + floor(u r) of its group, in order."""
    n = 4
    K, V = _tiny(8, 64 * n)
    c = exp.ExpressCache(n, K, V, 0.5, 0.5, 3, 5)
    for blk in range(16):
        c.ingest_block(blk * n)
    assert c.m == 16 and c.buffer == []
    start_group = 16 * n // 8
    for blk in range(16, 24):
        c.ingest_block(blk * n)
        done = (blk + 1 - 16) * n // 8                     # groups of 8 completed since block 16
        expect = [8 * g + philox.uniform_offset(g, 3, 5, philox.TAG_SUBSAMPLE, 3, 8)
                  for g in range(start_group, start_group + done)]
        assert c.buffer == expect, blk


def test_schedule_counts_groups_longer_than_a_block():
    """The static schedule past the old 2 n_out^2 limit: n = 4 over 4096 tokens (1024 blocks):
    HALVEs after 4, 16, 64, 256 blocks (and at 1024), a batch every m n_out tokens."""
    ev = exp.schedule(4096, 4)
    halves = [b for t, b, _ in ev if t == philox.TAG_HALVE_FIRST]
    batches = [b for t, b, _ in ev if t == philox.TAG_BATCH]
    assert halves == [0, 1, 2, 3, 4]
    assert batches == list(range(12))                      # three per epoch m = 4, 16, 64, 256
    K, V = _tiny(9, 4096)
    _, _, log = exp.run_unit(K, V, 4, 0.5, 0.5, 1, 0, query_positions=[])
    assert [k for k, _ in log] == [(t, b) for t, b, _ in ev]


def test_streaming_decode_equals_prefill():
    """Token-by-token decode gives exactly the causal forward's outputs."""
    rng = np.random.default_rng(6)
    S0, steps, Hkv, H, n = 150, 90, 2, 4, 8
    total = S0 + steps
    k = rng.standard_normal((1, total, Hkv, 8)); v = rng.standard_normal((1, total, Hkv, 4))
    q = rng.standard_normal((1, total, H, 8))
    pre = fwd.forward(q, k, v, causal=True, n_out=n, seed=3)
    dec, _, _ = fwd.decode(k[:, :S0], v[:, :S0], q[:, S0:], k[:, S0:], v[:, S0:], n_out=n, seed=3)
    assert np.array_equal(dec, pre["out"][:, S0:])


def test_causal_gqa_heads_share_state():
    rng = np.random.default_rng(7)
    S, n = 300, 8
    q = rng.standard_normal((1, S, 4, 8)); k = rng.standard_normal((1, S, 1, 8)); v = rng.standard_normal((1, S, 1, 4))
    r = fwd.forward(q, k, v, causal=True, n_out=n, seed=1)
    K, V = k[0, :, 0], v[0, :, 0]
    vis, _, _ = exp.run_unit(K, V, n, 1 / math.sqrt(8), 0.5, 1, 0, query_positions=[299])
    idx, w = vis[299]
    for h in range(4):
        ref = att.weighted_attention(q[0, 299, h][None], K[idx], V[idx], w, 1 / math.sqrt(8))[0]
        assert np.max(np.abs(r["out"][0, 299, h] - ref)) <= 1e-13


def test_causal_error_shrinks_with_cache_size():
    rng = np.random.default_rng(8)
    S = 2048
    q = rng.standard_normal((1, S, 1, 8)) * 0.6; k = rng.standard_normal((1, S, 1, 8)) * 0.6
    v = rng.standard_normal((1, S, 1, 8))
    rows = np.array([[0, t, 0] for t in range(1500, 2048, 7)])
    ref = fwd.exact(q, k, v, causal=True, queries=rows)
    errs = [att.rel_frobenius_error(fwd.forward(q, k, v, causal=True, n_out=n, queries=rows)["out"], ref)
            for n in (32, 64, 128)]
    assert errs[0] > errs[1] > errs[2], errs


@pytest.mark.parametrize("S,n,H,Hkv", [(4096 + 77, 64, 2, 1), (500, 16, 4, 2), (67, 4, 1, 1), (300, 512, 2, 2)])
def test_block_outputs_match_per_query(S, n, H, Hkv):
    """Causal outputs formed a block at a time (one masked weighted attention per Express
    block) agree with the query-at-a-time visible sets, HALVEs included."""
    rng = np.random.default_rng(S + n)
    q = rng.standard_normal((1, S, H, 8)); k = rng.standard_normal((1, S, Hkv, 8)); v = rng.standard_normal((1, S, Hkv, 4))
    a = fwd.forward(q, k, v, causal=True, n_out=n, seed=2)
    b = fwd.forward(q, k, v, causal=True, n_out=n, seed=2, block_outputs=True)
    assert np.max(np.abs(a["out"] - b["out"])) <= 1e-12
    for u in a["coreset"]:
        assert np.array_equal(a["coreset"][u][0], b["coreset"][u][0])
        assert np.array_equal(a["log"][u], b["log"][u])


def test_block_outputs_exact_when_disabled():
    rng = np.random.default_rng(3)
    S = 200
    q = rng.standard_normal((1, S, 2, 8)); k = rng.standard_normal((1, S, 2, 8)); v = rng.standard_normal((1, S, 2, 4))
    out = fwd.forward(q, k, v, causal=True, n_out=256, block_outputs=True)["out"]
    assert np.max(np.abs(out - fwd.exact(q, k, v, causal=True))) <= 1e-12
