"""Kernel-level GPU parity: Philox stream, coreset attention, one halving."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import forward as fwd
from oracle import kernel_halving as khm
from oracle import philox
from sub_quadratic_attention_amd import inputs
from tests.parity import TOL, say, to_gpu, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


def test_philox_matches_oracle():
    from sub_quadratic_attention_amd.binding import philox as gpu_philox
    rng = np.random.default_rng(0)
    n = 20000
    ctr = rng.integers(0, 2 ** 63, (n, 4), dtype=np.int64)
    ctr[:100] = np.arange(400).reshape(100, 4)          # small words, as the path uses them
    seed = 0x1234_5678_9ABC
    say("[philox] GPU vs oracle on", n, "counters")
    out = gpu_philox(torch.from_numpy(ctr).cuda(), seed).cpu().numpy().view(np.uint64)
    for i in range(n):
        ref = philox.philox4x64_10([int(x) for x in ctr[i]], (seed, 0))
        assert [int(x) for x in out[i]] == ref, i


CASES = [
    # dtype, E, D, H, Hkv, B, T, S, n
    ("f32", 64, 64, 1, 1, 2, 100, 256, 16),
    ("f32", 128, 128, 2, 1, 1, 70, 300, 45),
    ("bf16", 128, 128, 4, 2, 1, 130, 512, 96),
    ("bf16", 64, 256, 1, 1, 2, 64, 4096, 64),
    ("bf16", 64, 64, 2, 2, 1, 33, 100, 33),
]


@pytest.mark.parametrize("dt,E,D,H,Hkv,B,T,S,n", CASES)
def test_coreset_attention_matches_oracle(dt, E, D, H, Hkv, B, T, S, n):
    """Attention alone on an oracle-chosen weighted coreset (all ragged sizes)."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    say(f"[coreset-attn] {dt} E{E} D{D} H{H}/{Hkv} B{B} T{T} S{S} n{n}")
    rng = np.random.default_rng(E + D + n)
    cast = inputs.bf16_round if dt == "bf16" else (lambda x: x.astype(np.float32))
    q = cast(rng.standard_normal((B, T, H, E)))
    k = cast(rng.standard_normal((B, S, Hkv, E)))
    v = cast(rng.standard_normal((B, S, Hkv, D)))
    units = B * Hkv
    idx = np.stack([np.sort(rng.choice(S, n, replace=False)) for _ in range(units)]).astype(np.int32)
    w = rng.uniform(0.5, 64.0, (units, n)).astype(np.float32)
    ta = ThinAttention(E, D, H, Hkv, torch_dtype(dt))
    out = ta.coreset_attention(to_gpu(q, dt), to_gpu(k, dt), to_gpu(v, dt),
                               torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda())
    o = out.float().cpu().numpy()
    s = 1 / math.sqrt(E)
    group = H // Hkv
    worst = 0.0
    for b in range(B):
        for h in range(H):
            u = b * Hkv + h // group
            ref = att.weighted_attention(q[b, :, h].astype(np.float64), k[b, idx[u], h // group].astype(np.float64),
                                         v[b, idx[u], h // group].astype(np.float64), w[u].astype(np.float64), s)
            worst = max(worst, att.max_abs_error(o[b, :, h], ref))
    say(f"[coreset-attn] max abs {worst:.3g}")
    assert worst <= TOL[dt]


@pytest.mark.parametrize("dt,E,D,S", [("f32", 64, 64, 200), ("bf16", 128, 128, 333)])
def test_exact_attention_path(dt, E, D, S):
    """idx = NULL: plain attention over all keys equals the oracle's exact attention."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    rng = np.random.default_rng(S)
    cast = inputs.bf16_round if dt == "bf16" else (lambda x: x.astype(np.float32))
    q = cast(rng.standard_normal((2, 77, 2, E)))
    k = cast(rng.standard_normal((2, S, 2, E)))
    v = cast(rng.standard_normal((2, S, 2, D)))
    ta = ThinAttention(E, D, 2, 2, torch_dtype(dt))
    o = ta.coreset_attention(to_gpu(q, dt), to_gpu(k, dt), to_gpu(v, dt)).float().cpu().numpy()
    ref = fwd.exact(q, k, v)
    assert att.max_abs_error(o, ref) <= TOL[dt]


@pytest.mark.parametrize("dt,E,D,N,scale", [
    ("f32", 64, 64, 16, 0.0), ("f32", 64, 64, 196, 0.0), ("bf16", 128, 128, 512, 0.0),
    ("bf16", 64, 256, 128, 0.0), ("bf16", 128, 128, 1024, 0.0), ("f32", 64, 64, 130, 1.0),
])
def test_single_halving_matches_oracle(dt, E, D, N, scale):
    """Pair Gram to 1e-12 relative; every decision equal except near ties."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    say(f"[halving] {dt} E{E} D{D} N{N} scale{scale}")
    rng = np.random.default_rng(N)
    S = 2 * N + 17
    if dt == "bf16":
        d = inputs.causal_prefill(seed=N, H=2, S=S, E=E, D=D) if E == D else inputs.biggan_self_attention(B=1)
        k, v = d["k"][:, :S], d["v"][:, :S]
        Hkv = k.shape[2]
    else:
        d = inputs.unmasked_small(seed=N, S=S, E=E, D=D)
        k, v = d["k"], d["v"]
        Hkv = 1
    S = k.shape[1]
    units = Hkv
    pts = np.stack([np.sort(rng.choice(S, N, replace=False)) for _ in range(units)]).astype(np.int32)
    ta = ThinAttention(E, D, Hkv, Hkv, torch_dtype(dt), scale=scale)
    seed, tag, bin_id = 77, philox.TAG_BATCH, 5
    kept, dec, gram = ta.halving(to_gpu(k, dt), to_gpu(v, dt), torch.from_numpy(pts).cuda(), seed, tag, bin_id)
    kept, dec, gram = kept.cpu().numpy(), dec.cpu().numpy(), gram.cpu().numpy()
    s = scale if scale else 1 / math.sqrt(E)
    for u in range(units):
        K = k[0, pts[u], u].astype(np.float64)
        V = v[0, pts[u], u].astype(np.float64)
        G = khm.pair_gram(K, V, s)
        up = np.triu(np.ones_like(G, dtype=bool))
        rel = np.abs(gram[u][up] - G[up]) / np.abs(G).max()
        say(f"[halving] unit {u}: max rel Gram diff {rel.max():.3g}")
        assert rel.max() <= 1e-12
        st = khm.HalvingStats()
        keep, _ = khm.kernel_halving(K, V, s, 0.5, seed, u, bin_id, tag, override=dec[u].astype(bool), stats=st)
        say(f"[halving] unit {u}: near ties {st.near_ties} fails {st.fails} of {st.decisions}")
        assert st.fails == 0
        assert np.array_equal(kept[u], pts[u][khm.kept_positions(keep)])
