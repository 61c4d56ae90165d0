"""Key streams longer than one staged window of the attention kernel (1536 gathered
tokens per window), and the handling of out-of-range token indices."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from sub_quadratic_attention_amd import inputs
from tests.parity import TOL, run_and_compare, sample_queries, say, to_gpu, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


@pytest.mark.parametrize("dt,E,D,H,Hkv,T,S,n", [
    ("f32", 64, 64, 1, 1, 200, 5000, 2000),        # two windows
    ("bf16", 128, 128, 4, 2, 150, 8000, 3100),     # three windows, GQA, ragged last chunk
    ("bf16", 64, 256, 1, 1, 70, 4096, 1537),       # one key past the first window
])
def test_coreset_attention_multi_window(dt, E, D, H, Hkv, T, S, n):
    """Weighted coresets of more than 1536 keys, every output against the oracle."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    say(f"[multi-window] {dt} E{E} D{D} H{H}/{Hkv} T{T} S{S} n{n}")
    rng = np.random.default_rng(n)
    cast = inputs.bf16_round if dt == "bf16" else (lambda x: x.astype(np.float32))
    B = 1
    q = cast(rng.standard_normal((B, T, H, E)))
    k = cast(rng.standard_normal((B, S, Hkv, E)))
    v = cast(rng.standard_normal((B, S, Hkv, D)))
    units = B * Hkv
    idx = np.stack([np.sort(rng.choice(S, n, replace=False)) for _ in range(units)]).astype(np.int32)
    w = rng.uniform(0.5, 64.0, (units, n)).astype(np.float32)
    ta = ThinAttention(E, D, H, Hkv, torch_dtype(dt))
    out = ta.coreset_attention(to_gpu(q, dt), to_gpu(k, dt), to_gpu(v, dt), torch.from_numpy(idx).cuda(),
                               torch.from_numpy(w).cuda())
    ta.status()
    o = out.float().cpu().numpy()
    s = 1 / math.sqrt(E)
    group = H // Hkv
    worst = 0.0
    for h in range(H):
        u = h // group
        ref = att.weighted_attention(q[0, :, h].astype(np.float64), k[0, idx[u], u].astype(np.float64),
                                     v[0, idx[u], u].astype(np.float64), w[u].astype(np.float64), s)
        worst = max(worst, att.max_abs_error(o[0, :, h], ref))
    say(f"[multi-window] max abs {worst:.3g}")
    assert worst <= TOL[dt]


def test_unmasked_forward_multi_window():
    """S = 10000 = 16 * 625: a 2500-point coreset (two Compress levels of 2500 and 5000
    points), attended over two windows; every output, decision and coreset entry."""
    d = inputs.unmasked_small(seed=3, S=10000, E=64, D=64)
    s = run_and_compare("unmasked S=10000", d, False, 1, 1, 64, 64, block_outputs=True)
    assert s["idx"].shape[1] == 2500


def test_causal_forward_multi_window():
    """n_out = 512, S = 8192 + 300, two heads: after the first HALVE the visible sets grow
    to 3 n_out + raw block (up to ~2000 keys), beyond one window; every output."""
    d = inputs.causal_prefill(seed=5, H=2, S=8192 + 300)
    s = run_and_compare("causal n_out=512 S=8492", d, True, 2, 2, 128, 128, n_out=512, block_outputs=True)
    assert s["decisions"] > 0


def test_causal_exact_long_raw_range():
    """Thinning disabled on a 5000-token causal stream (n_out >= S): the raw range runs over
    four windows; every output against exact causal attention."""
    d = inputs.causal_prefill(seed=6, H=2, S=5000)
    s = run_and_compare("causal exact S=5000", d, True, 2, 2, 128, 128, n_out=8192, block_outputs=True)
    assert s["decisions"] == 0


def test_causal_forward_groups_longer_than_a_block():
    """n_out = 16, S = 4105: past token 1024 the subsampling groups (32, then 128 tokens) span
    several blocks; every output, decision and coreset entry."""
    d = inputs.causal_prefill(seed=7, H=2, S=4096 + 9)
    s = run_and_compare("causal n_out=16 S=4105", d, True, 2, 2, 128, 128, n_out=16, block_outputs=True)
    assert s["decisions"] > 0


# ---- token indices outside [0, S): clamped, reported, never read out of bounds --------

def test_out_of_range_key_idx_is_reported():
    from sub_quadratic_attention_amd.binding import ThinAttention, ThinAttnError
    rng = np.random.default_rng(11)
    B, T, S, H, Hkv, L = 1, 64, 512, 4, 2, 256
    q = torch.from_numpy(inputs.bf16_round(rng.standard_normal((B, T, H, 128)))).to(torch.bfloat16).cuda()
    k = torch.from_numpy(inputs.bf16_round(rng.standard_normal((B, S, Hkv, 128)))).to(torch.bfloat16).cuda()
    v = torch.from_numpy(inputs.bf16_round(rng.standard_normal((B, S, Hkv, 128)))).to(torch.bfloat16).cuda()
    good = np.stack([np.sort(rng.choice(S, L, replace=False)) for _ in range(B * Hkv)]).reshape(B, Hkv, L)
    bad = good.copy()
    bad[0, 0, 5] = S + 1000
    bad[0, 1, 7] = -3
    clamped = np.clip(bad, 0, S - 1)
    ta = ThinAttention(128, 128, H, Hkv, torch.bfloat16)
    say("[bad-index] forward_subset with two entries outside [0, S)")
    out_bad = ta.forward_subset(q, k, v, torch.from_numpy(bad.astype(np.int32)).cuda())
    with pytest.raises(ThinAttnError) as e:
        ta.status()
    assert e.value.code == -1
    ta.status()   # reported once, then cleared
    out_clamped = ta.forward_subset(q, k, v, torch.from_numpy(clamped.astype(np.int32)).cuda())
    ta.status()
    assert torch.equal(out_bad, out_clamped)
    # reported by the next call when no status call intervenes
    ta.forward_subset(q, k, v, torch.from_numpy(bad.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    with pytest.raises(ThinAttnError):
        ta.forward_subset(q, k, v, torch.from_numpy(good.astype(np.int32)).cuda())
    ta.forward_subset(q, k, v, torch.from_numpy(good.astype(np.int32)).cuda())
    ta.status()


def test_out_of_range_coreset_and_points_are_reported():
    from sub_quadratic_attention_amd.binding import ThinAttention, ThinAttnError
    rng = np.random.default_rng(12)
    B, T, S, n = 1, 40, 300, 64
    q, k, v = (torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).cuda()
               for sh in ((B, T, 1, 64), (B, S, 1, 64), (B, S, 1, 64)))
    ta = ThinAttention(64, 64, 1, 1, torch.float32)
    idx = np.sort(rng.choice(S, n, replace=False)).astype(np.int32)[None]
    idx[0, -1] = S
    ta.coreset_attention(q, k, v, torch.from_numpy(idx).cuda())
    with pytest.raises(ThinAttnError):
        ta.status()
    pts = rng.choice(S, 256, replace=False).astype(np.int32)[None]
    pts[0, 100] = 1 << 30
    ta.halving(k, v, torch.from_numpy(pts).cuda())
    with pytest.raises(ThinAttnError):
        ta.status()
    ta.status()
