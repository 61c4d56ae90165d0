"""Key-value attention kernel and kernel halving, float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Attention kernel.  "Express Language Modeling", section "Thinformer Express",
names the key-value attention kernel kappa_att, chosen so that thinning keeps
the averages attention needs.  Those averages are sum_j exp(s<q,k_j>) v_j and
sum_j exp(s<q,k_j>); both are inner products in the product space of the
exponential dot-product kernel on keys and the linear kernel on (v, 1).  The
reading taken is therefore

    kappa((k, v), (k', v')) = exp(s * <k, k'>) * (<v, v'> + 1).

Kernel halving.  The same section names Kernel Halving as the base halving
of EXPRESS; the pages do not spell it out.  The steps below are the
self-balancing walk of the kernel-thinning papers (Dwivedi and Mackey,
"Kernel Thinning", the KT-SPLIT walk; Shetty, Dwivedi and Mackey,
"Distribution Compression in Near-linear Time", kernel halving), with the
failure parameter of one call spread over its N points:
delta_i = delta / N, so the walk constant is c_N = sqrt(2 ln(2 N / delta)).

For a list x_0 .. x_{N-1} (N = 2P) the pairs are (x_{2i}, x_{2i+1}).  With
h_i = kappa(x_{2i}, .) - kappa(x_{2i+1}, .) the pair Gram is
G_ij = <h_i, h_j>.  For i = 0 .. P-1:

    b_i^2   = G_ii                       (clamped at 0 against rounding)
    alpha_i = sum_{j<i} eta_j G_ij       (the walk evaluated at the pair)
    a_i     = max(b_i * sigma_{i-1} * c_N, b_i^2)
    p~_i    = (1 - alpha_i / a_i) / 2    (1/2 when a_i = 0)
    p_i     = clip(p~_i, 0, 1)
    eta_i   = +1 if u_i < p_i else -1    (u_i from the Philox stream)
    sigma_i^2 = sigma_{i-1}^2 + b_i^2 * max(0, 1 + (b_i^2 - 2 a_i) sigma_{i-1}^2 / a_i^2)
                                         (unchanged when a_i = 0)

eta_i = +1 keeps x_{2i}, -1 keeps x_{2i+1}; the kept points carry twice the
input weight.  The decision margin is |u_i - p~_i| (relative to a_i by
construction).

Greedy signs (``greedy=True``), the deterministic variant: eta_i = +1 exactly
when alpha_i < 0, else -1 (alpha_i = 0, so pair 0 of every bin, keeps
x_{2i+1}); a_i, sigma and u play no part.  It is written on alpha's sign, not
as the walk with u_i = 1/2: in 1 - alpha / a the sign of alpha is rounded away
once |alpha| < 2^-53 a, which keys with heavy outlier channels (kernel values
spread over tens of orders of magnitude) reach.  Its margin is
|alpha_i| / sum_{j<i} |G_ij|, alpha against the rounding scale of its own sum
(0 when that sum is 0).  The sub-Gaussian guarantee of the walk holds for the
randomised signs only.

Parity pins (tests/test_oracle_kh.py): brute-force recomputation of every
b_i, alpha_i, a_i, sigma_i and p_i from explicit kernel sums on tiny bins;
the MMD identity ||mean(kept) - mean(all)||^2 = eta^T G eta / (4 P^2) against
direct kernel sums; forced decisions when |alpha| >= a; invariance of every
decision under kappa -> 2^k kappa; the kernel Gram is symmetric PSD.
"""

import math

import numpy as np

from . import philox


def kappa_matrix(K1, V1, K2, V2, scale):
    """kappa between every row of (K1, V1) and every row of (K2, V2)."""
    return np.exp(scale * (K1 @ K2.T)) * (V1 @ V2.T + 1.0)


def pair_gram(Kpts, Vpts, scale):
    """G_ij = kappa(x2i,x2j) - kappa(x2i,x2j+1) - kappa(x2i+1,x2j) + kappa(x2i+1,x2j+1)."""
    kap = kappa_matrix(Kpts, Vpts, Kpts, Vpts, scale)
    return kap[0::2, 0::2] - kap[0::2, 1::2] - kap[1::2, 0::2] + kap[1::2, 1::2]


class HalvingStats:
    """Counts gathered while replaying another implementation's decisions."""

    def __init__(self):
        self.decisions = 0
        self.near_ties = 0      # differing decisions with margin < tie_margin
        self.fails = 0          # differing decisions with margin >= tie_margin
        self.min_margin = math.inf

    def merge(self, other):
        self.decisions += other.decisions
        self.near_ties += other.near_ties
        self.fails += other.fails
        self.min_margin = min(self.min_margin, other.min_margin)


def kernel_halving(Kpts, Vpts, scale, delta, seed, unit, bin_id, tag,
                   override=None, stats=None, tie_margin=1e-6, G=None, greedy=False):
    """One kernel halving pass over an ordered list of N = 2P points.

    Kpts [N, E], Vpts [N, D] are the points' keys and values (float64).
    Returns (keep_first, margins): keep_first[i] is True when x_{2i} is kept.

    ``override`` (optional, length P of bools): decisions of another
    implementation.  Where it differs from this walk's own decision the
    walk follows it and counts a near tie (margin < tie_margin) or a failure
    in ``stats``.  ``G`` may pass a precomputed pair Gram (used by the
    scale-invariance pin).
    """
    N = Kpts.shape[0]
    assert N % 2 == 0 and N >= 2
    P = N // 2
    if G is None:
        G = pair_gram(Kpts, Vpts, scale)
    c_N = math.sqrt(2.0 * math.log(2.0 * N / delta))
    eta = np.zeros(P)
    keep_first = np.zeros(P, dtype=bool)
    margins = np.zeros(P)
    sigma2 = 0.0
    for i in range(P):
        b2 = max(G[i, i], 0.0)
        b = math.sqrt(b2)
        alpha = float(np.dot(eta[:i], G[i, :i]))
        a = max(b * math.sqrt(sigma2) * c_N, b2)
        p_tilde = 0.5 * (1.0 - alpha / a) if a > 0.0 else 0.5
        p = min(max(p_tilde, 0.0), 1.0)
        if greedy:
            first = alpha < 0.0
            scale_i = float(np.abs(G[i, :i]).sum())
            margin = abs(alpha) / scale_i if scale_i > 0.0 else 0.0
        else:
            u = philox.uniform(i, bin_id, unit, tag, seed)
            first = u < p
            margin = abs(u - p_tilde)
        margins[i] = margin
        if stats is not None:
            stats.decisions += 1
            stats.min_margin = min(stats.min_margin, margin)
        if override is not None and bool(override[i]) != first:
            if stats is not None:
                if margin < tie_margin:
                    stats.near_ties += 1
                else:
                    stats.fails += 1
            first = bool(override[i])
        eta[i] = 1.0 if first else -1.0
        keep_first[i] = first
        if a > 0.0:
            sigma2 = sigma2 + b2 * max(0.0, 1.0 + (b2 - 2.0 * a) * sigma2 / (a * a))
    return keep_first, margins


def kept_positions(keep_first):
    """Positions (into the input list) of the kept points, in pair order."""
    return np.array([2 * i if f else 2 * i + 1 for i, f in enumerate(keep_first)],
                    dtype=np.int64)
