"""The whole Thinformer / Thinformer Express path, float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Shapes follow the "Thinformer" README, section "Getting Started": query
[B, T, H, E], key [B, S, H_kv, E], value [B, S, H_kv, D]; causal attention
requires S == T.  H_kv may divide H (grouped queries: query head h reads KV
head h // (H / H_kv)); thinning is done once per (b, KV head) "unit",
unit = b * H_kv + h_kv.  The call returns the attention output and, as the
second item (the README's attn_output_weights), the coreset of every unit
as (token indices, weights).

Replay: ``decisions`` may pass, per unit, another implementation's flat
decision array (uint8, 1 = first point of the pair kept, in the library's
order).  The oracle then follows those decisions, counting in ``stats``
where its own walk disagreed: near ties (margin < tie_margin) and failures.
"""

import math

import numpy as np

from . import attention as att
from . import compress as cmp
from . import express as exp
from . import kernel_halving as khm


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def forward(q, k, v, causal=False, seed=0, scale=None, g=0, n_out=None,
            delta=0.5, queries=None, decisions=None, tie_margin=1e-6, greedy=False,
            subsample_base=False, block_outputs=False):
    """Run the path.  ``queries``: None for the full output, or an int array of
    (b, t, h) rows for sampled outputs.  ``greedy``: every kernel halving
    takes greedy signs (see oracle.kernel_halving); ``subsample_base``: the
    unmasked Compress runs after base subsampling (see oracle.compress).
    ``block_outputs`` (full output only): every query of a unit (unmasked) or
    of an Express block (causal) shares one coreset / state, so their outputs
    are formed together, as one weighted attention of all those queries,
    instead of one query at a time; the result agrees to rounding.

    Returns a dict with
      out      [B, T, H, D] (or [n_queries, D]) float64
      coreset  {unit: (idx int64, w float64)}
      log      {unit: flat uint8 decisions}
      stats    HalvingStats over all units
      n_out    coreset size (unmasked) or cache size (causal)
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, T, H, E = q.shape
    _, S, Hkv, _ = k.shape
    D = v.shape[3]
    assert k.shape == (B, S, Hkv, E) and v.shape == (B, S, Hkv, D)
    assert H % Hkv == 0
    group = H // Hkv
    s = 1.0 / math.sqrt(E) if scale is None else float(scale)
    if causal:
        assert S == T, "causal attention needs key length T"
        size = exp.default_cache_size(S) if n_out is None else int(n_out)
    else:
        size = cmp.coreset_size(S, g, subsample_base)
    Lt = cmp.thinned_length(S, g, subsample_base)   # the unmasked decision log's list length

    if queries is None:
        want = [(b, t, h) for b in range(B) for t in range(T) for h in range(H)]
    else:
        want = [tuple(int(x) for x in row) for row in np.asarray(queries).reshape(-1, 3)]
    by_unit = {}
    for n, (b, t, h) in enumerate(want):
        by_unit.setdefault(b * Hkv + h // group, []).append((n, b, t, h))

    stats = khm.HalvingStats()
    coreset, logs = {}, {}
    results = np.zeros((len(want), D))
    blocked = block_outputs and queries is None
    full = np.zeros((B, T, H, D)) if blocked else None
    for b in range(B):
        for hk in range(Hkv):
            unit = b * Hkv + hk
            K, V = k[b, :, hk, :], v[b, :, hk, :]
            rows = [] if blocked else by_unit.get(unit, [])
            heads = range(hk * group, (hk + 1) * group)
            if blocked and causal:
                ov = None if decisions is None else exp.flat_to_log(decisions[unit], S, size)
                blocks, final, log = exp.run_unit_blocks(K, V, size, s, delta, seed, unit, override=ov,
                                                         stats=stats, greedy=greedy)
                coreset[unit] = final
                logs[unit] = exp.log_to_flat(log)
                for lo, hi, idx, w in blocks:
                    for h in heads:
                        full[b, lo:hi, h] = att.express_block_attention(q[b, lo:hi, h], K, V, idx, w, lo, s)
                continue
            if not causal:
                ov = None
                if decisions is not None:
                    ov = cmp.flat_to_log(decisions[unit], Lt, g)
                idx, w, log = cmp.thin_unmasked(K, V, s, delta, seed, unit, g,
                                                override=ov, stats=stats, greedy=greedy,
                                                subsample_base=subsample_base)
                coreset[unit] = (idx, np.full(len(idx), w))
                logs[unit] = cmp.log_to_flat(log, Lt, g)
                if blocked:
                    for h in heads:
                        full[b, :, h] = att.weighted_attention(q[b, :, h], K[idx], V[idx], coreset[unit][1], s)
                for n, bb, t, h in rows:
                    results[n] = att.weighted_attention(q[bb, t, h][None, :], K[idx], V[idx],
                                                        coreset[unit][1], s)[0]
            else:
                ov = None
                if decisions is not None:
                    ov = exp.flat_to_log(decisions[unit], S, size)
                visible, final, log = exp.run_unit(
                    K, V, size, s, delta, seed, unit,
                    query_positions=[t for _, _, t, _ in rows], override=ov, stats=stats, greedy=greedy)
                coreset[unit] = final
                logs[unit] = exp.log_to_flat(log)
                for n, bb, t, h in rows:
                    idx, w = visible[t]
                    results[n] = att.weighted_attention(q[bb, t, h][None, :], K[idx], V[idx], w, s)[0]
    out = full if blocked else (results.reshape(B, T, H, D) if queries is None else results)
    return {"out": out, "coreset": coreset, "log": logs, "stats": stats, "n_out": size}


def forward_subset(q, k, v, key_idx, seed=0, scale=None, g=0, delta=0.5, queries=None, decisions=None,
                   tie_margin=1e-6, greedy=False, subsample_base=False):
    """Unmasked Thinformer over a chosen key list per unit (thinning after a KV
    selector: the "Express Language Modeling" explainer on gist.science,
    "Experimental Results", accelerated KV cache compression, where the
    thinning step no longer depends on how the initial keys were picked).

    key_idx [B, H_kv, L] lists, per unit, token indices into k / v in the order
    to thin.  The list is the point sequence of an unmasked forward with
    S = L (the same recursion, size rule, decision layout and random streams);
    its coreset positions map back to tokens through the list.  Returns the
    same dict as ``forward``, coreset indices being tokens.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    key_idx = np.asarray(key_idx, dtype=np.int64)
    B, T, H, E = q.shape
    _, S, Hkv, _ = k.shape
    D = v.shape[3]
    L = key_idx.shape[2]
    assert key_idx.shape == (B, Hkv, L) and key_idx.min() >= 0 and key_idx.max() < S
    group = H // Hkv
    s = 1.0 / math.sqrt(E) if scale is None else float(scale)
    if queries is None:
        want = [(b, t, h) for b in range(B) for t in range(T) for h in range(H)]
    else:
        want = [tuple(int(x) for x in row) for row in np.asarray(queries).reshape(-1, 3)]
    Lt = cmp.thinned_length(L, g, subsample_base)
    stats = khm.HalvingStats()
    coreset, logs = {}, {}
    for b in range(B):
        for hk in range(Hkv):
            unit = b * Hkv + hk
            sel = key_idx[b, hk]
            ov = None if decisions is None else cmp.flat_to_log(decisions[unit], Lt, g)
            pos, w, log = cmp.thin_unmasked(k[b, sel, hk, :], v[b, sel, hk, :], s, delta, seed, unit, g,
                                            override=ov, stats=stats, greedy=greedy,
                                            subsample_base=subsample_base)
            coreset[unit] = (sel[pos], np.full(len(pos), w))
            logs[unit] = cmp.log_to_flat(log, Lt, g)
    results = np.zeros((len(want), D))
    for n, (b, t, h) in enumerate(want):
        tok, w = coreset[b * Hkv + h // group]
        results[n] = att.weighted_attention(q[b, t, h][None, :], k[b, tok, h // group, :], v[b, tok, h // group, :],
                                            w, s)[0]
    out = results.reshape(B, T, H, D) if queries is None else results
    return {"out": out, "coreset": coreset, "log": logs, "stats": stats,
            "n_out": cmp.coreset_size(L, g, subsample_base)}


def exact(q, k, v, causal=False, scale=None, queries=None):
    """Exact softmax attention with the same conventions (GQA, sampling)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, T, H, E = q.shape
    Hkv = k.shape[2]
    group = H // Hkv
    s = 1.0 / math.sqrt(E) if scale is None else float(scale)
    if queries is None:
        out = np.zeros((B, T, H, v.shape[3]))
        for b in range(B):
            for h in range(H):
                out[b, :, h, :] = att.exact_attention(q[b, :, h, :], k[b, :, h // group, :],
                                                      v[b, :, h // group, :], s, causal)
        return out
    rows = np.asarray(queries).reshape(-1, 3)
    out = np.zeros((len(rows), v.shape[3]))
    for n, (b, t, h) in enumerate(rows):
        kk = k[b, :, h // group, :]
        vv = v[b, :, h // group, :]
        if causal:
            kk, vv = kk[: t + 1], vv[: t + 1]
        out[n] = att.exact_attention(q[b, t, h][None, :], kk, vv, s)[0]
    return out


def decode(k_hist, v_hist, q_steps, k_steps, v_steps, n_out=None, seed=0,
           scale=None, delta=0.5, decisions=None, tie_margin=1e-6, greedy=False):
    """Token-by-token Express decode of one batch entry per unit.

    k_hist [B, S0, H_kv, E] is ingested first; then step i appends
    (k_steps[:, i], v_steps[:, i]) at token S0 + i and the queries
    q_steps[:, i] [B, H, E] attend to what that token's query sees.
    Written as its own driver loop (one token at a time) so that it checks the
    block bookkeeping of ``forward``.  Returns (out [B, steps, H, D], stats, logs).
    """
    kh, vh = _as64(k_hist), _as64(v_hist)
    qs, ks, vs = _as64(q_steps), _as64(k_steps), _as64(v_steps)
    B, S0, Hkv, E = kh.shape
    steps, H = qs.shape[1], qs.shape[2]
    D = vh.shape[3]
    group = H // Hkv
    total = S0 + steps
    size = exp.default_cache_size(S0) if n_out is None else int(n_out)
    s = 1.0 / math.sqrt(E) if scale is None else float(scale)
    stats = khm.HalvingStats()
    out = np.zeros((B, steps, H, D))
    logs = {}
    for b in range(B):
        for hk in range(Hkv):
            unit = b * Hkv + hk
            K = np.concatenate([kh[b, :, hk, :], ks[b, :, hk, :]])
            V = np.concatenate([vh[b, :, hk, :], vs[b, :, hk, :]])
            ov = None
            if decisions is not None:
                ov = exp.flat_to_log(decisions[unit], (total // size) * size, size)
            cache = exp.ExpressCache(size, K, V, s, delta, seed, unit, override=ov, stats=stats, greedy=greedy)
            for t in range(total):
                if t >= S0:
                    idx, w = cache.visible(t)
                    for h in range(hk * group, (hk + 1) * group):
                        out[b, t - S0, h] = att.weighted_attention(
                            qs[b, t - S0, h][None, :], K[idx], V[idx], w, s)[0]
                if (t + 1) % size == 0:
                    cache.ingest_block(t + 1 - size)
            logs[unit] = exp.log_to_flat(cache.log)
    return out, stats, logs
