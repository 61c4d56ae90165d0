"""Weighted-coreset attention, exact attention and error metrics, float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Weighted-coreset attention.  "Express Language Modeling" (lay section "The
Smart Summarizer", technical section "Thinformer Express") describes
attending to a small weighted summary of the keys and values instead of all
of them.  A point of weight w stands for w raw key-value pairs, so the
output of query q over the coreset C is

    out(q) = sum_{j in C} w_j exp(s<q,k_j>) v_j / sum_{j in C} w_j exp(s<q,k_j>).

The softmax scale s is 1/sqrt(E) unless given (the README's "drop-in
replacement for a standard attention layer").  The maximum logit is
subtracted before exponentiating; that leaves the ratio unchanged.

Exact attention is written out separately (no shared helper) so that it can
pin the weighted form: with w = 1 on all S keys the two must agree to 1e-12.
"""

import numpy as np


def weighted_attention(q, Kc, Vc, w, scale):
    """q [T, E]; Kc [n, E]; Vc [n, D]; w [n] > 0.  Returns [T, D] float64."""
    logits = scale * (q @ Kc.T)                          # [T, n]
    shift = logits.max(axis=1, keepdims=True)
    p = w[None, :] * np.exp(logits - shift)
    return (p @ Vc) / p.sum(axis=1, keepdims=True)


def express_block_attention(q, K, V, state_idx, state_w, lo, scale):
    """Outputs of the queries at tokens lo, lo + 1, ... of one Express block (q [T, E],
    T <= the block's length): each attends to the state its block sees (tokens
    state_idx with weights state_w) and to the raw tokens lo .. its own token
    with weight 1.  This is the weighted form above with the causal mask of the
    raw part written out: token lo + j is visible to the query at lo + i iff
    j <= i.  K, V hold every token's key and value."""
    T = q.shape[0]
    raw = np.arange(lo, lo + T)
    keys = np.concatenate([np.asarray(state_idx, dtype=np.int64), raw])
    w = np.concatenate([np.asarray(state_w, dtype=np.float64), np.ones(T)])
    logits = scale * (q @ K[keys].T)                                   # [T, |state| + T]
    hidden = np.zeros(logits.shape, dtype=bool)
    hidden[:, len(state_idx):] = np.arange(T)[None, :] > np.arange(T)[:, None]
    logits = np.where(hidden, -np.inf, logits)
    shift = logits.max(axis=1, keepdims=True)
    p = w[None, :] * np.exp(logits - shift)
    return (p @ V[keys]) / p.sum(axis=1, keepdims=True)


def exact_attention(q, k, v, scale, causal=False, q_positions=None):
    """Plain softmax attention of q [T, E] against k [S, E], v [S, D].

    With causal=True query row i sits at token q_positions[i] (default i) and
    sees keys 0 .. that token.
    """
    T = q.shape[0]
    S = k.shape[0]
    scores = scale * (q @ k.T)
    if causal:
        pos = np.arange(T) if q_positions is None else np.asarray(q_positions)
        mask = np.arange(S)[None, :] > pos[:, None]
        scores = np.where(mask, -np.inf, scores)
    top = np.max(scores, axis=1, keepdims=True)
    e = np.exp(scores - top)
    return (e / np.sum(e, axis=1, keepdims=True)) @ v


def max_abs_error(out, ref):
    return float(np.max(np.abs(np.asarray(out, np.float64) - ref))) if ref.size else 0.0


def rel_frobenius_error(out, ref):
    num = np.linalg.norm(np.asarray(out, np.float64) - ref)
    den = np.linalg.norm(ref)
    return float(num / den) if den > 0 else float(num)
