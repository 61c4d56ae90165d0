"""FP8 (OCP E4M3) inputs: the thinning reads fp8 keys and values (widened exactly to fp64),
coreset attention takes Q K^T on the gfx950 FP8 MFMA, and the streaming state keeps fp8 rows.
Parity against the float64 oracle on the same fp8 values (the generators round to E4M3)."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from sub_quadratic_attention_amd import inputs
from tests.parity import TOL, run_and_compare, sample_queries, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


@pytest.mark.parametrize("H,Hkv,T,S,n", [(1, 1, 100, 600, 64), (4, 2, 130, 4000, 333), (2, 2, 77, 6000, 2100)])
def test_fp8_coreset_attention(H, Hkv, T, S, n):
    """Weighted coresets of 64 .. 2100 keys (one to two windows), every output."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    say(f"[fp8-attn] H{H}/{Hkv} T{T} S{S} n{n}")
    rng = np.random.default_rng(n)
    B, E, D = 1, 128, 128
    q = inputs.fp8_round(rng.standard_normal((B, T, H, E)) * 1.5)
    k = inputs.fp8_round(rng.standard_normal((B, S, Hkv, E)))
    v = inputs.fp8_round(rng.standard_normal((B, S, Hkv, D)))
    units = B * Hkv
    idx = np.stack([np.sort(rng.choice(S, n, replace=False)) for _ in range(units)]).astype(np.int32)
    w = rng.uniform(0.5, 64.0, (units, n)).astype(np.float32)
    ta = ThinAttention(E, D, H, Hkv, torch.float8_e4m3fn)
    out = ta.coreset_attention(to_gpu(q, "fp8"), to_gpu(k, "fp8"), to_gpu(v, "fp8"), torch.from_numpy(idx).cuda(),
                               torch.from_numpy(w).cuda())
    ta.status()
    assert out.dtype == torch.bfloat16
    o = out.float().cpu().numpy()
    s = 1 / math.sqrt(E)
    group = H // Hkv
    worst = 0.0
    for h in range(H):
        u = h // group
        ref = att.weighted_attention(q[0, :, h].astype(np.float64), k[0, idx[u], u].astype(np.float64),
                                     v[0, idx[u], u].astype(np.float64), w[u].astype(np.float64), s)
        worst = max(worst, att.max_abs_error(o[0, :, h], ref))
    say(f"[fp8-attn] max abs {worst:.3g}")
    assert worst <= TOL["fp8"]


def test_fp8_exact_attention():
    """No thinning (all S keys, weight 1) against exact attention."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    rng = np.random.default_rng(3)
    B, T, S, H = 2, 90, 700, 2
    q = inputs.fp8_round(rng.standard_normal((B, T, H, 128)))
    k = inputs.fp8_round(rng.standard_normal((B, S, H, 128)))
    v = inputs.fp8_round(rng.standard_normal((B, S, H, 128)))
    ta = ThinAttention(128, 128, H, H, torch.float8_e4m3fn)
    o = ta.coreset_attention(to_gpu(q, "fp8"), to_gpu(k, "fp8"), to_gpu(v, "fp8")).float().cpu().numpy()
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ref = att.exact_attention(q[b, :, h].astype(np.float64), k[b, :, h].astype(np.float64),
                                      v[b, :, h].astype(np.float64), 1 / math.sqrt(128))
            worst = max(worst, att.max_abs_error(o[b, :, h], ref))
    assert worst <= TOL["fp8"], worst


def test_fp8_unmasked_forward():
    """Thinformer over fp8 keys and values: every decision, coreset entry and output."""
    d = inputs.unmasked_small(seed=4, B=2, H=2, S=1024, E=128, D=128, dtype="fp8")
    s = run_and_compare("fp8 unmasked S=1024", d, False, 2, 2, 128, 128, block_outputs=True)
    assert s["decisions"] > 0


def test_fp8_causal_three_halves():
    """Thinformer Express over fp8 inputs with outlier channels: HALVEs, batches, ragged tail."""
    d = inputs.causal_prefill(seed=5, H=2, S=4325, dtype="fp8")
    run_and_compare("fp8 causal S=4325 n_out=64", d, True, 2, 2, 128, 128, n_out=64, block_outputs=True)


def test_fp8_causal_prefill_full():
    """The 32-head, 32768-token decoder-layer prefill in fp8: every output."""
    d = inputs.causal_prefill(seed=0, dtype="fp8")
    qs = sample_queries(1, 32768, 32, 400, seed=6, always=[(0, 0, 0), (0, 32767, 31)])
    s = run_and_compare("fp8 causal prefill H=32 S=32768", d, True, 32, 32, 128, 128, block_outputs=True,
                        error_queries=qs)
    assert s["decisions"] == 131072


def test_fp8_decode_state():
    """The streaming state with fp8 rows: bulk ingest, then decode steps through a batch
    halving and a HALVE, against the oracle's token-by-token decode."""
    from tests.test_gpu_3_decode import _check
    d = inputs.kv_decode(seed=2, Hkv=2, H=8, S0=1900, steps=200, E=128, D=128, walk_len=2100, dtype="fp8")
    _check("fp8 bulk 1900 + 200 steps", d, 32, 8, 2, 128, 128)
