"""End-to-end GPU parity of thin_attn_forward against the float64 oracle (replay protocol)."""

import numpy as np
import pytest
import torch

from sub_quadratic_attention_amd import inputs
from oracle import attention as att
from tests.parity import TOL, run_and_compare, sample_queries, say, to_gpu, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


# ---- unmasked (Thinformer) ------------------------------------------------

def test_unmasked_small_full():
    """B=1, H=1, S=256, fp32: every output, coreset and decision."""
    d = inputs.unmasked_small(seed=0)
    run_and_compare("unmasked S=256", d, False, 1, 1, 64, 64)


def test_unmasked_small_unit_scale():
    d = inputs.unmasked_small(seed=0)
    run_and_compare("unmasked S=256 scale=1", d, False, 1, 1, 64, 64, scale=1.0)


def test_unmasked_disabled_is_exact():
    d = inputs.unmasked_small(seed=1)
    s = run_and_compare("unmasked g=4 (no thinning)", d, False, 1, 1, 64, 64, g=4)
    assert s["decisions"] == 0


def test_unmasked_oversampling():
    """Oversampling g = 1: Compress stops one level earlier (S=256: n_out 32 instead of 16)."""
    d = inputs.unmasked_small(seed=2)
    s = run_and_compare("unmasked g=1", d, False, 1, 1, 64, 64, g=1)
    assert s["decisions"] > 0


def test_unmasked_ragged_and_gqa():
    """S = 4^2 * 13 (base blocks of 13), T ragged, 2 query heads per KV head, bf16."""
    rng = np.random.default_rng(3)
    B, T, S, H, Hkv = 2, 83, 208, 4, 2
    d = dict(q=inputs.bf16_round(rng.standard_normal((B, T, H, 64)) * 0.5),
             k=inputs.bf16_round(rng.standard_normal((B, S, Hkv, 64)) * 0.5),
             v=inputs.bf16_round(rng.standard_normal((B, S, Hkv, 128))), dtype="bf16")
    run_and_compare("unmasked S=208 GQA", d, False, H, Hkv, 64, 128)


@pytest.mark.parametrize("S,dtype", [(48, "bf16"), (16, "f32"), (64 * 4, "bf16")])
def test_unmasked_small_bins(S, dtype):
    """Bins of at most 16 points (Gram and walk fused): S=48 gives 12-point bins (one per
    16-point tile), S=16 a tile holding a single 8-point bin, S=256 tiles of 4, 2 and 1 bins;
    six units."""
    rng = np.random.default_rng(S)
    B, T, H, Hkv = 3, 37, 4, 2
    cast = inputs.bf16_round if dtype == "bf16" else (lambda x: x.astype(np.float32))
    d = dict(q=cast(rng.standard_normal((B, T, H, 64)) * 0.5),
             k=cast(rng.standard_normal((B, S, Hkv, 64)) * 0.5), dtype=dtype)
    D = 128 if dtype == "bf16" else 64
    d["v"] = cast(rng.standard_normal((B, S, Hkv, D)))
    run_and_compare(f"unmasked small bins S={S} {dtype}", d, False, H, Hkv, 64, D)


@pytest.mark.parametrize("S,dtype", [(80, "f32"), (192, "bf16"), (1024, "bf16")])
def test_unmasked_medium_bins(S, dtype):
    """Bins of 20-32 points (one workgroup per bin, Gram and walk fused) beside the other
    paths: S=80 gives 20- and 40-point bins, S=192 12-, 24- and 48-point bins, S=1024 4- to
    64-point bins; six units."""
    rng = np.random.default_rng(7 + S)
    B, T, H, Hkv = 3, 29, 2, 2
    cast = inputs.bf16_round if dtype == "bf16" else (lambda x: x.astype(np.float32))
    D = 128 if dtype == "bf16" else 64
    d = dict(q=cast(rng.standard_normal((B, T, H, 64)) * 0.5), k=cast(rng.standard_normal((B, S, Hkv, 64)) * 0.5),
             v=cast(rng.standard_normal((B, S, Hkv, D))), dtype=dtype)
    run_and_compare(f"unmasked medium bins S={S} {dtype}", d, False, H, Hkv, 64, D)


def test_vit_token_mixing_reduced():
    """56x56 ViT tokens (S=3136, n_out=392), two batch entries, sampled outputs."""
    d = inputs.vit_token_mixing(seed=0, B=2)
    qs = sample_queries(2, 3136, 1, 400, always=[(0, 0, 0), (1, 3135, 0)])
    run_and_compare("vit B=2", d, False, 1, 1, 64, 64, queries=qs)


def test_biggan_reduced():
    d = inputs.biggan_self_attention(seed=0, B=2)
    qs = sample_queries(2, 4096, 1, 400, always=[(1, 4095, 0)])
    run_and_compare("biggan B=2", d, False, 1, 1, 64, 256, queries=qs)


def test_base_subsampling_full():
    """Base subsampling, S = 196 = 4 * 49: one point per stratum of 7, then one Compress level
    (14 points of weight 14), every output, fp32 with GQA."""
    rng = np.random.default_rng(21)
    B, S, H, Hkv = 2, 196, 4, 2
    d = dict(q=(rng.standard_normal((B, S, H, 64)) * 0.5).astype(np.float32),
             k=(rng.standard_normal((B, S, Hkv, 64)) * 0.5).astype(np.float32),
             v=rng.standard_normal((B, S, Hkv, 64)).astype(np.float32), dtype="f32")
    run_and_compare("base subsampling S=196", d, False, H, Hkv, 64, 64, subsample_base=True)


def test_base_subsampling_vit():
    """ViT tokens (S = 3136) with base subsampling: 56 = sqrt(S) coreset points instead of 392."""
    d = inputs.vit_token_mixing(seed=3, B=2)
    qs = sample_queries(2, 3136, 1, 300, always=[(1, 3135, 0)])
    s = run_and_compare("vit base subsampling", d, False, 1, 1, 64, 64, queries=qs, subsample_base=True)
    assert s["idx"].shape[1] == 56


def test_greedy_signs_with_base_subsampling():
    """Both flags: S = 784 = 4^2 * 49, strata of 7 (112 points), greedy walks, every output, bf16."""
    rng = np.random.default_rng(23)
    B, S, H, Hkv = 2, 784, 2, 1
    d = dict(q=inputs.bf16_round(rng.standard_normal((B, S, H, 64)) * 0.5),
             k=inputs.bf16_round(rng.standard_normal((B, S, Hkv, 64)) * 0.5),
             v=inputs.bf16_round(rng.standard_normal((B, S, Hkv, 128))), dtype="bf16")
    s = run_and_compare("greedy + base subsampling S=784", d, False, H, Hkv, 64, 128, greedy=True,
                        subsample_base=True)
    assert s["idx"].shape[1] == 28


def test_greedy_signs_unmasked():
    """Greedy signs (keep the first point iff alpha_i < 0, in every walk) over BigGAN-shaped bins, N = 4 .. 128
    (small, medium and Gram + sweep kernels).  The decisions do not depend on the seed."""
    d = inputs.biggan_self_attention(seed=5, B=1)
    qs = sample_queries(1, 4096, 1, 300, always=[(0, 4095, 0)])
    s0 = run_and_compare("biggan greedy seed 0", d, False, 1, 1, 64, 256, queries=qs, greedy=True)
    s1 = run_and_compare("biggan greedy seed 9", d, False, 1, 1, 64, 256, queries=qs, greedy=True, seed=9,
                         check_error=False)
    assert np.array_equal(s0["dec"], s1["dec"]) and np.array_equal(s0["idx"], s1["idx"])


# ---- causal (Thinformer Express) -------------------------------------------

def test_causal_three_halves_ragged():
    """n_out=64: exact phase, three HALVEs, six batches, ragged tail; every output."""
    d = inputs.causal_prefill(seed=0, H=2, S=4096 + 64 * 3 + 37)
    run_and_compare("causal S=4325 n=64", d, True, 2, 2, 128, 128, n_out=64)


def test_causal_small_cache_tiles_span_blocks():
    """n_out=16 < query tile: tiles see several blocks' states."""
    d = inputs.causal_prefill(seed=1, H=1, S=500, E=64, D=64)
    run_and_compare("causal S=500 n=16", d, True, 1, 1, 64, 64, n_out=16)


def test_greedy_signs_causal():
    """Greedy signs in Express: batch halvings and HALVEs (bins of 4n = 256 points take the
    Gram + sweep kernels with thresholds in the Gram's lower triangle)."""
    d = inputs.causal_prefill(seed=6, H=2, S=4096 + 64 * 3 + 37)
    run_and_compare("causal greedy S=4325 n=64", d, True, 2, 2, 128, 128, n_out=64, greedy=True)


def test_causal_gqa_fp32():
    rng = np.random.default_rng(4)
    S, H, Hkv = 1100, 4, 2
    d = dict(q=rng.standard_normal((1, S, H, 64)).astype(np.float32),
             k=rng.standard_normal((1, S, Hkv, 64)).astype(np.float32),
             v=rng.standard_normal((1, S, Hkv, 64)).astype(np.float32), dtype="f32")
    run_and_compare("causal fp32 GQA S=1100 n=32", d, True, H, Hkv, 64, 64, n_out=32)


def test_causal_disabled_is_exact():
    d = inputs.causal_prefill(seed=2, H=1, S=300)
    s = run_and_compare("causal n_out>=S", d, True, 1, 1, 128, 128, n_out=512)
    assert s["decisions"] == 0


def test_causal_prefill_reduced():
    """The 32k-token prefill shape on two heads, sampled outputs."""
    d = inputs.causal_prefill(seed=0, H=2, S=32768)
    qs = sample_queries(1, 32768, 2, 300, always=[(0, 32767, 1), (0, 0, 0), (0, 16384, 0)])
    run_and_compare("causal S=32768 H=2", d, True, 2, 2, 128, 128, queries=qs)


def test_determinism_and_seed():
    from sub_quadratic_attention_amd.binding import ThinAttention
    from tests.parity import to_gpu
    d = inputs.causal_prefill(seed=3, H=2, S=2048)
    ta = ThinAttention(128, 128, 2, 2, torch.bfloat16, n_out=32)
    q, k, v = (to_gpu(d[x], "bf16") for x in "qkv")
    a, ea = ta.forward(q, k, v, causal=True, seed=5, return_coreset=True)
    b, eb = ta.forward(q, k, v, causal=True, seed=5, return_coreset=True)
    c, ec = ta.forward(q, k, v, causal=True, seed=6, return_coreset=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ea["coreset_idx"], eb["coreset_idx"])
    assert not torch.equal(ea["coreset_idx"], ec["coreset_idx"])
    say("[determinism] ok")


# ---- degenerate shapes --------------------------------------------------------

@pytest.mark.parametrize("causal,S,T", [(False, 1, 5), (False, 3, 2), (False, 4, 7), (False, 5, 1),
                                        (True, 1, 1), (True, 2, 2), (True, 3, 3), (True, 9, 9)])
def test_tiny_sequences(causal, S, T):
    """S of 1 to 9 tokens: no thinning (S < 4, or a causal state that never fills), the
    smallest Compress (S=4: one 4-point bin), a 2-token cache with a partial block."""
    rng = np.random.default_rng(100 + S)
    B, H, Hkv = 2, 2, 1
    d = dict(q=rng.standard_normal((B, T, H, 64)).astype(np.float32),
             k=rng.standard_normal((B, S, Hkv, 64)).astype(np.float32),
             v=rng.standard_normal((B, S, Hkv, 64)).astype(np.float32), dtype="f32")
    run_and_compare(f"tiny causal={causal} S={S} T={T}", d, causal, H, Hkv, 64, 64, n_out=2 if causal else 0)


@pytest.mark.parametrize("B,T", [(0, 8), (2, 0)])
def test_empty_batch_or_queries(B, T):
    """B = 0 or T = 0: the call succeeds and touches nothing."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    ta = ThinAttention(64, 64, 1, 1, torch.float32)
    S = 16
    q = torch.zeros((B, T, 1, 64), device="cuda")
    k = torch.zeros((B, S, 1, 64), device="cuda")
    v = torch.zeros((B, S, 1, 64), device="cuda")
    out = ta.forward(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert out.shape == (B, T, 1, 64)


# ---- thinning after a KV selector -------------------------------------------

@pytest.mark.parametrize("S,L,dtype,sub", [(4096, 1024, "bf16", False), (3000, 768, "f32", False),
                                           (500, 192, "bf16", False), (300, 50, "f32", False),
                                           (3000, 784, "f32", True)])
def test_thinning_after_selector(S, L, dtype, sub):
    """thin_attn_forward_subset on a top-L selection: decisions, coreset (tokens through the
    list) and outputs against the replayed oracle; L = 50 is too short to thin (the list itself
    is the coreset), L = 192 and 768 run 12- to 96-point bins, L = 1024 4- to 64-point bins;
    L = 784 = 4^2 * 49 with base subsampling thins one point per 7 of the list to 112, then 28."""
    from oracle import forward as fwd
    from sub_quadratic_attention_amd.binding import ThinAttention
    rng = np.random.default_rng(S + L)
    B, T, H, Hkv = 2, 33, 4, 2
    D = 128 if dtype == "bf16" else 64
    cast = inputs.bf16_round if dtype == "bf16" else (lambda x: x.astype(np.float32))
    q = cast(rng.standard_normal((B, T, H, 64)) * 0.5)
    k = cast(rng.standard_normal((B, S, Hkv, 64)) * 0.5)
    v = cast(rng.standard_normal((B, S, Hkv, D)))
    sel = inputs.top_k_keys(k, q, L)
    ta = ThinAttention(64, D, H, Hkv, torch_dtype(dtype), subsample_base=sub)
    out, ex = ta.forward_subset(to_gpu(q, dtype), to_gpu(k, dtype), to_gpu(v, dtype), torch.from_numpy(sel).cuda(),
                                return_coreset=True, return_decisions=True)
    torch.cuda.synchronize()
    units = B * Hkv
    dec = ex["decisions"].cpu().numpy()
    ref = fwd.forward_subset(q, k, v, sel, decisions={u: dec[u] for u in range(units)}, subsample_base=sub)
    st = ref["stats"]
    say(f"[subset] S={S} L={L} {dtype}: decisions={st.decisions} near_ties={st.near_ties} fails={st.fails}")
    assert st.fails == 0 and st.near_ties <= 0.005 * max(st.decisions, 1)
    idx, w, ln = (x.cpu().numpy() for x in (ex["coreset_idx"], ex["coreset_w"], ex["coreset_len"]))
    for u in range(units):
        tok, wt = ref["coreset"][u]
        assert ln[u] == len(tok)
        assert np.array_equal(idx[u, :ln[u]], tok)
        assert np.array_equal(w[u, :ln[u]], wt.astype(np.float32))
    err = att.max_abs_error(out.float().cpu().numpy().astype(np.float64), ref["out"])
    say(f"[subset] S={S} L={L}: max|gpu - oracle| = {err:.3g}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("S,n", [(200, 64), (600, 64), (2000, 64), (4325, 64), (32768 // 4, 0)])
def test_causal_two_streams_equal_one_stream(S, n):
    """The causal path's second stream (batch halvings and finished epochs' attention beside
    the HALVE chain) gives bit-identical outputs, coreset and decisions to one stream: no
    HALVE (S = 200 at n = 64), one (600: the exact epoch's attention goes to the side), two
    (2000) and three (4325; 8192 at the default n_out of 128)."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    d = inputs.causal_prefill(seed=9, H=4, S=S)
    q, k, v = (to_gpu(d[x], "bf16") for x in ("q", "k", "v"))
    res = []
    for one in (False, True):
        ta = ThinAttention(128, 128, 4, 4, torch.bfloat16, n_out=n, one_stream=one)
        out, ex = ta.forward(q, k, v, causal=True, seed=3, return_coreset=True, return_decisions=True)
        torch.cuda.synchronize()
        res.append((out, ex))
    (o2, e2), (o1, e1) = res
    assert torch.equal(o1, o2)
    for key in ("coreset_idx", "coreset_w", "coreset_len", "decisions"):
        assert torch.equal(e1[key], e2[key]), key
