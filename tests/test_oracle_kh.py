"""Pins of the oracle's kernel halving (brute force, closed forms, invariants)."""

import itertools
import math

import numpy as np
import pytest

from oracle import kernel_halving as khm
from oracle import philox


def _points(rng, N, E=4, D=3, scale_k=0.7):
    return rng.standard_normal((N, E)) * scale_k, rng.standard_normal((N, D))


def _kap_scalar(kx, vx, ky, vy, s):
    """kappa by explicit loops over the coordinates (no matrix products)."""
    dk = 0.0
    for a, b in zip(kx, ky):
        dk += a * b
    dv = 0.0
    for a, b in zip(vx, vy):
        dv += a * b
    return math.exp(s * dk) * (dv + 1.0)


@pytest.mark.parametrize("N,seed", [(2, 0), (4, 1), (8, 2), (12, 3), (16, 4), (16, 5)])
def test_every_step_by_brute_force(N, seed):
    """Recompute b, alpha, a, sigma, p of every pair from pointwise kernel sums."""
    rng = np.random.default_rng(seed)
    K, V = _points(rng, N)
    s, delta, unit, bin_id, tag = 0.9, 0.5, 3, 17, philox.TAG_COMPRESS
    keep, margins = khm.kernel_halving(K, V, s, delta, seed, unit, bin_id, tag)
    P = N // 2
    c = math.sqrt(2 * math.log(2 * N / delta))
    kap = lambda i, j: _kap_scalar(K[i], V[i], K[j], V[j], s)
    eta = []
    sigma2 = 0.0
    for i in range(P):
        x, xp = 2 * i, 2 * i + 1
        b2 = kap(x, x) + kap(xp, xp) - 2 * kap(x, xp)
        # psi_{i-1}(x) - psi_{i-1}(x'), psi = sum_j eta_j (kappa(x_2j, .) - kappa(x_2j+1, .))
        alpha = 0.0
        for j in range(i):
            alpha += eta[j] * (kap(2 * j, x) - kap(2 * j + 1, x) - kap(2 * j, xp) + kap(2 * j + 1, xp))
        b = math.sqrt(max(b2, 0.0))
        a = max(b * math.sqrt(sigma2) * c, b2)
        pt = 0.5 * (1 - alpha / a) if a > 0 else 0.5
        u = philox.uniform(i, bin_id, unit, tag, seed)
        assert abs(margins[i] - abs(u - pt)) <= 1e-9 * max(1.0, abs(pt))
        e = 1.0 if u < min(max(pt, 0.0), 1.0) else -1.0
        assert keep[i] == (e > 0)
        eta.append(e)
        if a > 0:
            sigma2 = sigma2 + b2 * max(0.0, 1 + (b2 - 2 * a) * sigma2 / a ** 2)


@pytest.mark.parametrize("N,seed", [(4, 0), (8, 1), (16, 2), (32, 3)])
def test_mmd_identity(N, seed):
    """||mean(kept) - mean(all)||^2 from direct kernel sums equals eta^T G eta / (4 P^2)."""
    rng = np.random.default_rng(100 + seed)
    K, V = _points(rng, N)
    s = 0.8
    keep, _ = khm.kernel_halving(K, V, s, 0.5, seed, 0, 0, 0)
    P = N // 2
    kept = khm.kept_positions(keep)
    kap = lambda i, j: _kap_scalar(K[i], V[i], K[j], V[j], s)
    allp = range(N)
    mmd2 = (sum(kap(i, j) for i in kept for j in kept) / P ** 2
            - 2 * sum(kap(i, j) for i in kept for j in allp) / (P * N)
            + sum(kap(i, j) for i in allp for j in allp) / N ** 2)
    G = khm.pair_gram(K, V, s)
    eta = np.where(keep, 1.0, -1.0)
    assert mmd2 == pytest.approx(eta @ G @ eta / (4 * P ** 2), rel=1e-9, abs=1e-12)


def test_enumerate_all_sign_vectors_report_rank():
    """All 2^P outcomes of a tiny bin: both MMD formulas agree for every one.

    The rank of the chosen outcome is reported, not asserted: the walk is
    randomised and is not a minimiser.
    """
    rng = np.random.default_rng(7)
    N = 12
    K, V = _points(rng, N)
    s = 1.0
    G = khm.pair_gram(K, V, s)
    P = N // 2
    kap = khm.kappa_matrix(K, V, K, V, s)
    vals = []
    for signs in itertools.product((1.0, -1.0), repeat=P):
        eta = np.array(signs)
        kept = [2 * i if e > 0 else 2 * i + 1 for i, e in enumerate(eta)]
        direct = (kap[np.ix_(kept, kept)].sum() / P ** 2
                  - 2 * kap[kept, :].sum() / (P * N) + kap.sum() / N ** 2)
        quad = eta @ G @ eta / (4 * P ** 2)
        assert direct == pytest.approx(quad, rel=1e-8, abs=1e-12)
        vals.append(quad)
    keep, _ = khm.kernel_halving(K, V, s, 0.5, 0, 0, 0, 0)
    chosen = np.where(keep, 1.0, -1.0) @ G @ np.where(keep, 1.0, -1.0) / (4 * P ** 2)
    rank = int((np.array(vals) < chosen - 1e-15).sum())
    print(f"kernel halving outcome rank {rank} of {len(vals)}")


def test_forced_decisions_follow_the_walk_sign():
    """|alpha| > a clips p to 0 or 1: the second pair must oppose the first."""
    G = np.array([[1.0, 5.0], [5.0, 1.0]])
    dummy = np.zeros((4, 1))
    for seed in range(200):
        keep, margins = khm.kernel_halving(dummy, dummy, 1.0, 0.5, seed, 0, 0, 0, G=G)
        assert keep[1] != keep[0]
        assert margins[1] > 0.5  # p~ lies outside [0, 1]


def test_degenerate_pair_is_a_fair_coin():
    """b = 0 (identical points) gives p = 1/2 exactly: keep first iff u < 1/2."""
    K = np.zeros((2, 3)); V = np.ones((2, 2))
    for seed in range(100):
        keep, margins = khm.kernel_halving(K, V, 1.0, 0.5, seed, 5, 9, 1)
        u = philox.uniform(0, 9, 5, 1, seed)
        assert keep[0] == (u < 0.5)
        assert margins[0] == abs(u - 0.5)


@pytest.mark.parametrize("k", [-6, -2, 2, 4, 10])
def test_scale_invariance_of_decisions(k):
    """kappa -> 4^k kappa changes no decision (bit-identical)."""
    rng = np.random.default_rng(11)
    K, V = _points(rng, 64)
    G = khm.pair_gram(K, V, 0.9)
    a, _ = khm.kernel_halving(K, V, 0.9, 0.5, 3, 1, 2, 0, G=G)
    b, _ = khm.kernel_halving(K, V, 0.9, 0.5, 3, 1, 2, 0, G=G * (4.0 ** k))
    assert np.array_equal(a, b)


def test_kernel_gram_symmetric_psd():
    rng = np.random.default_rng(5)
    K, V = _points(rng, 40, E=8, D=8)
    kap = khm.kappa_matrix(K, V, K, V, 0.5)
    assert np.allclose(kap, kap.T, rtol=0, atol=1e-12 * np.abs(kap).max())
    assert np.linalg.eigvalsh(kap).min() >= -1e-12 * np.trace(kap)
    G = khm.pair_gram(K, V, 0.5)
    assert np.all(np.diag(G) >= 0)
    assert np.linalg.eigvalsh(G).min() >= -1e-12 * np.trace(G)


def test_halving_beats_random_halving():
    """The walk keeps the kept half's mean close to the full mean.

    Keeping a uniformly random point of every pair gives E[eta^T G eta] =
    trace G.  On low-dimensional points (where the kernel's effective rank is
    small) the walk stays far below that; a sign error in alpha or p makes it
    grow far above it instead (about 60x trace G on this data).
    """
    rng = np.random.default_rng(21)
    ratios = []
    for seed in range(6):
        K, V = _points(rng, 512, E=1, D=1, scale_k=0.5)
        G = khm.pair_gram(K, V, 1.0)
        keep, _ = khm.kernel_halving(K, V, 1.0, 0.5, seed, 0, 0, 0, G=G)
        eta = np.where(keep, 1.0, -1.0)
        ratios.append((eta @ G @ eta) / np.trace(G))
    assert np.mean(ratios) < 0.5, ratios


def test_replay_counts_flips():
    rng = np.random.default_rng(2)
    K, V = _points(rng, 32)
    keep, margins = khm.kernel_halving(K, V, 1.0, 0.5, 0, 0, 0, 0)
    flipped = keep.copy()
    flipped[3] = not flipped[3]
    st = khm.HalvingStats()
    keep2, _ = khm.kernel_halving(K, V, 1.0, 0.5, 0, 0, 0, 0, override=flipped, stats=st)
    assert np.array_equal(keep2, flipped)
    assert st.decisions == 16
    if margins[3] < 1e-6:
        assert st.near_ties == 1 and st.fails == 0
    else:
        assert st.fails == 1 and st.near_ties == 0


@pytest.mark.parametrize("N,seed", [(2, 0), (4, 1), (8, 2), (16, 3), (16, 4)])
def test_greedy_signs_by_brute_force(N, seed):
    """Greedy signs: pair i keeps its first point exactly when the walk's value
    alpha_i (recomputed from pointwise kernel sums) is negative, whatever the seed."""
    rng = np.random.default_rng(100 + seed)
    K, V = _points(rng, N)
    s = 0.9
    kap = lambda i, j: _kap_scalar(K[i], V[i], K[j], V[j], s)
    keeps = [khm.kernel_halving(K, V, s, 0.5, sd, 3, 17, philox.TAG_COMPRESS, greedy=True)[0] for sd in (0, 7)]
    assert np.array_equal(keeps[0], keeps[1])
    keep = keeps[0]
    eta = []
    for i in range(N // 2):
        x, xp = 2 * i, 2 * i + 1
        alpha = 0.0
        for j in range(i):
            alpha += eta[j] * (kap(2 * j, x) - kap(2 * j + 1, x) - kap(2 * j, xp) + kap(2 * j + 1, xp))
        assert keep[i] == (alpha < 0)
        eta.append(1.0 if alpha < 0 else -1.0)


@pytest.mark.parametrize("N,seed", [(8, 0), (32, 1), (64, 2)])
def test_greedy_walk_norm_bound(N, seed):
    """Each greedy step adds b_i^2 + 2 eta_i alpha_i <= b_i^2 to ||psi||^2, so every
    prefix of the walk has ||psi_i||^2 <= sum_{j<=i} b_j^2 (checked on the pair
    Gram); the randomised walk has no such per-prefix bound."""
    rng = np.random.default_rng(200 + seed)
    K, V = _points(rng, N, E=6, D=4)
    s = 0.8
    keep, _ = khm.kernel_halving(K, V, s, 0.5, seed, 0, 0, 0, greedy=True)
    G = khm.pair_gram(K, V, s)
    eta = np.where(keep, 1.0, -1.0)
    for i in range(1, N // 2 + 1):
        e = eta[:i]
        assert e @ G[:i, :i] @ e <= np.trace(G[:i, :i]) * (1 + 1e-12) + 1e-300


def test_greedy_degenerate_pair_keeps_second():
    """b = 0 gives alpha_0 = 0 for the first pair: keep-first needs alpha < 0, so the second point is kept."""
    K = np.zeros((2, 3)); V = np.ones((2, 2))
    keep, margins = khm.kernel_halving(K, V, 1.0, 0.5, 4, 5, 9, 1, greedy=True)
    assert not keep[0] and margins[0] == 0.0


def test_greedy_sign_survives_wide_dynamic_range():
    """A pair whose alpha is far below a (|alpha| / a ~ 1e-40) still takes alpha's sign:
    pair 0 (alpha = 0) keeps its second point, so pair 1 has alpha = -G_01 and keeps its
    first point when G_01 > 0, its second when G_01 < 0."""
    dummy = np.zeros((6, 1))
    for g01 in (1.0, -1.0):
        G = np.array([[1e40, g01, 0.0], [g01, 1e20, 0.0], [0.0, 0.0, 1.0]])
        keep, margins = khm.kernel_halving(dummy, dummy, 1.0, 0.5, 0, 0, 0, 0, G=G, greedy=True)
        assert not keep[0]
        assert keep[1] == (g01 > 0)
        assert margins[1] == 1.0 and margins[2] == 0.0


# ---------------------------------------------------------------------------
# The threshold schedule a_i / sigma_i, pinned from the walk's observable
# outputs.  For a non-forced decision the oracle's margin |u_i - p~_i| and its
# decision give p~_i back (p~_i = u_i + margin when the first point is kept,
# u_i - margin otherwise), and a_i = alpha_i / (1 - 2 p~_i) with alpha_i
# summed here from the pair Gram and the kept signs.  The expected a_i are
# worked out by hand from the published recursion for a few simple Grams.
# ---------------------------------------------------------------------------
def _observed_thresholds(kh, G, seed, delta=0.5):
    P = G.shape[0]
    dummy = np.zeros((2 * P, 1))
    keep, margins = kh(dummy, dummy, 1.0, delta, seed, 0, 0, 0, G=G)
    eta = np.where(keep, 1.0, -1.0)
    a = [None]
    for i in range(1, P):
        u = philox.uniform(i, 0, 0, 0, seed)
        pt = u + margins[i] if keep[i] else u - margins[i]
        alpha = sum(eta[j] * G[i, j] for j in range(i))
        assert 0.0 < pt < 1.0, "the Grams below keep |alpha| far below a"
        a.append(alpha / (1.0 - 2.0 * pt))
    return a


def _gram(b):
    """Diagonal b_i^2; below it G_ij = 0.01 (1 + i / 10) 2^j (symmetric), so no signed sum
    of a row's entries vanishes and |alpha| stays far below every a_i."""
    P = len(b)
    G = np.zeros((P, P))
    for i in range(P):
        G[i, i] = b[i] ** 2
        for j in range(i):
            G[i, j] = G[j, i] = 0.01 * (1 + i / 10) * 2 ** j
    return G


def _expected_unit_b(c):
    """b = (1, 1, 1, 1).  sigma_1^2 = b_0^2 = 1 (pair 0 has a_0 = b_0^2 and sigma_0 = 0);
    a_1 = max(b_1 sigma_1 c, b_1^2) = c; sigma_2^2 = 1 + (1 + (1 - 2c)/c^2) = 1 + (1 - 1/c)^2;
    a_2 = c sigma_2 (> 1); sigma_3^2 = sigma_2^2 + (1 + sigma_2^2/a_2^2 - 2 sigma_2^2/a_2)
    = sigma_2^2 + 1 + 1/c^2 - 2 sigma_2/c (positive for these c); a_3 = c sigma_3."""
    s2 = 1.0 + (1.0 - 1.0 / c) ** 2
    s3 = s2 + 1.0 + 1.0 / c ** 2 - 2.0 * math.sqrt(s2) / c
    return [None, c, c * math.sqrt(s2), c * math.sqrt(s3)]


def _expected_mixed_b(c):
    """b = (0.1, 1, 2, 1) with c < 10: a_1 = max(0.1 c, 1) = 1 (the b^2 branch);
    sigma_2^2 = 0.01 + (1 + (1 - 2) 0.01 / 1) = 1 exactly; a_2 = max(2 c, 4) = 2 c (c > 2);
    sigma_3^2 = 1 + 4 (1 + (4 - 4c) / (4 c^2)) = 5 + 4/c^2 - 4/c; a_3 = max(c sigma_3, 1)."""
    s3 = 5.0 + 4.0 / c ** 2 - 4.0 / c
    return [None, 1.0, 2.0 * c, max(c * math.sqrt(s3), 1.0)]


def _check_threshold_schedule(kh):
    N = 8
    c = math.sqrt(2.0 * math.log(2.0 * N / 0.5))   # c_N with delta_i = delta / N
    assert 2.0 < c < 10.0
    for b, expect in (((1.0, 1.0, 1.0, 1.0), _expected_unit_b(c)), ((0.1, 1.0, 2.0, 1.0), _expected_mixed_b(c))):
        for seed in range(6):
            got = _observed_thresholds(kh, _gram(b), seed)
            for i in range(1, 4):
                assert got[i] == pytest.approx(expect[i], rel=1e-9), (b, seed, i, got[i], expect[i])


def _clip_count(kh, nbins=100, N=128):
    """Decisions whose p~ falls outside [0, 1] (|alpha_i| > a_i) over many random bins."""
    rng = np.random.default_rng(123)
    clips = 0
    for z in range(nbins):
        K = rng.standard_normal((N, 2)) * 0.5
        V = rng.standard_normal((N, 2))
        keep, margins = kh(K, V, 1.0, 0.5, z, 0, z, 0)
        for i in range(N // 2):
            u = philox.uniform(i, z, 0, 0, z)
            pt = u + margins[i] if keep[i] else u - margins[i]
            clips += not (0.0 <= pt <= 1.0)
    return clips, nbins * (N // 2)


def test_threshold_schedule_closed_forms():
    """a_1, a_2, a_3 of two hand-worked Grams (both branches of a = max(b sigma c, b^2))."""
    _check_threshold_schedule(khm.kernel_halving)


def test_clip_rate_within_delta():
    """The self-balancing walk forces a decision (|alpha_i| > a_i) with probability at most
    delta_i = delta / N at each step (kernel-thinning papers, self-balancing Hilbert walk);
    over 6400 decisions of N = 128 that bounds the expected count by 25."""
    clips, decisions = _clip_count(khm.kernel_halving)
    assert clips <= decisions * 0.5 / 128, (clips, decisions)


def _mutant(old, new):
    import inspect
    src = inspect.getsource(khm.kernel_halving)
    assert src.count(old) == 1, old
    ns = dict(khm.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["kernel_halving"]


SIGMA_UPDATE = "sigma2 = sigma2 + b2 * max(0.0, 1.0 + (b2 - 2.0 * a) * sigma2 / (a * a))"


@pytest.mark.parametrize("old,new", [
    (SIGMA_UPDATE, "sigma2 = 0.0"),                                                  # sigma never updated
    (SIGMA_UPDATE, SIGMA_UPDATE.replace("1.0 + (b2", "1.0 - (b2")),                 # update sign flipped
    (SIGMA_UPDATE, SIGMA_UPDATE.replace("b2 * max", "0.5 * b2 * max")),              # update halved
    ("a = max(b * math.sqrt(sigma2) * c_N, b2)", "a = b * math.sqrt(sigma2) * c_N"),  # b^2 branch dropped
    ("a = max(b * math.sqrt(sigma2) * c_N, b2)", "a = max(b * sigma2 * c_N, b2)"),    # sigma^2 for sigma
    ("2.0 * N / delta", "2.0 / delta"),                                              # delta not spread over N
])
def test_schedule_pins_catch_planted_mistakes(old, new):
    """A mistake planted in a copy of the oracle's walk fails the closed forms or the clip bound."""
    kh = _mutant(old, new)
    caught = False
    try:
        _check_threshold_schedule(kh)
    except (AssertionError, ZeroDivisionError, ValueError):
        caught = True
    if not caught:
        clips, decisions = _clip_count(kh, nbins=40)
        caught = clips > decisions * 0.5 / 128
    assert caught
