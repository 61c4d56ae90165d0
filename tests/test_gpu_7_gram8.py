"""The exact integer pair Gram (bf16 / fp8 rows split into int8 digits, products summed exactly
on the int8 MFMA; rows whose features do not fit the digits recomputed in fp64) against the
float64 oracle and against the library's fp64 Gram."""

import math

import numpy as np
import pytest
import torch

from oracle import kernel_halving as khm
from oracle import philox
from sub_quadratic_attention_amd import inputs
from tests.parity import run_and_compare, say, to_gpu, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


def plant_misfits(x, rows, rng, factor=2.0 ** -40):
    """Scale one feature of each listed row (token, head) by a power of two far below the row's
    largest: exact in bf16, and the row no longer fits four base-256 digits."""
    x = x.copy()
    for t, h in rows:
        f = rng.integers(0, x.shape[-1])
        x[0, t, h, f] *= factor
    return x


@pytest.mark.parametrize("dt,E,D,N,misfit", [
    ("bf16", 128, 128, 512, False), ("bf16", 128, 128, 1024, False), ("bf16", 128, 128, 2048, False),
    ("bf16", 64, 256, 512, False), ("fp8", 128, 128, 1024, False), ("bf16", 128, 128, 1024, True),
    ("bf16", 128, 128, 300, True),
])
def test_integer_gram_matches_oracle(dt, E, D, N, misfit):
    """Pair Gram to 1e-12 relative of the oracle's (and to 1e-13 of the fp64 Gram); every
    decision equal except near ties; rows planted not to fit take the fp64 recomputation."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    say(f"[gram8] {dt} E{E} D{D} N{N} misfit={misfit}")
    rng = np.random.default_rng(N + 7)
    S = 2 * N + 33
    if dt == "fp8":
        d = inputs.causal_prefill_fp8(seed=N, H=2, S=S)
    else:
        d = inputs.causal_prefill(seed=N, H=2, S=S, E=E, D=D)
    k, v = d["k"][:, :S], d["v"][:, :S]
    units = k.shape[2]
    pts = np.stack([np.sort(rng.choice(S, N, replace=False)) for _ in range(units)]).astype(np.int32)
    if misfit:   # ~3% of each unit's points get a misfit K row, ~2% a misfit V row
        rows_k = [(int(t), u) for u in range(units) for t in rng.choice(pts[u], N // 32, replace=False)]
        rows_v = [(int(t), u) for u in range(units) for t in rng.choice(pts[u], N // 48, replace=False)]
        k = plant_misfits(k, rows_k, rng)
        v = plant_misfits(v, rows_v, rng)
    ta = ThinAttention(E, D, units, units, torch_dtype(dt))
    assert ta.lib.thin_attn_halving_workspace_size(ta.h, 1, N) > 0
    seed, tag, bin_id = 91, philox.TAG_HALVE_FIRST, 3
    kg, vg, pg = to_gpu(k, dt), to_gpu(v, dt), torch.from_numpy(pts).cuda()
    kept, dec, gram = (x.cpu().numpy() for x in ta.halving(kg, vg, pg, seed, tag, bin_id))
    _, dec64, gram64 = (x.cpu().numpy() for x in ta.halving(kg, vg, pg, seed, tag, bin_id, workspace=False))
    s = 1 / math.sqrt(E)
    for u in range(units):
        K = k[0, pts[u], u].astype(np.float64)
        V = v[0, pts[u], u].astype(np.float64)
        G = khm.pair_gram(K, V, s)
        up = np.triu(np.ones_like(G, dtype=bool))
        rel = np.abs(gram[u][up] - G[up]) / np.abs(G).max()
        rel64 = np.abs(gram[u][up] - gram64[u][up]) / np.abs(G).max()
        say(f"[gram8] unit {u}: max rel Gram diff {rel.max():.3g} (vs fp64 Gram {rel64.max():.3g})")
        assert rel.max() <= 1e-12
        assert rel64.max() <= 1e-13
        st = khm.HalvingStats()
        keep, _ = khm.kernel_halving(K, V, s, 0.5, seed, u, bin_id, tag, override=dec[u].astype(bool), stats=st)
        say(f"[gram8] unit {u}: near ties {st.near_ties} fails {st.fails} of {st.decisions}; "
            f"{int((dec[u] != dec64[u]).sum())} differ from the fp64 Gram's")
        assert st.fails == 0
        assert np.array_equal(kept[u], pts[u][khm.kept_positions(keep)])


@pytest.mark.parametrize("n,nk,nv", [(64, 60, 40), (128, 400, 300)])
def test_causal_with_misfit_rows(n, nk, nv):
    """A causal forward (batch halvings and HALVEs on the integer Gram) whose keys and values
    hold rows that do not fit the digits: every output and decision against the oracle.  At
    n_out = 128 both halvings of a HALVE take the integer Gram, the second on the first's
    digits, so its fix-up workgroups find the planted rows through the kept points' numbers;
    the forward also equals the fp64 Gram's decision for decision."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    d = inputs.causal_prefill(seed=11, H=2, S=4096 + 64 * 3 + 37)
    rng = np.random.default_rng(5)
    S = d["k"].shape[1]
    d["k"] = plant_misfits(d["k"], [(int(t), int(h)) for t, h in zip(rng.integers(0, S, nk), rng.integers(0, 2, nk))], rng)
    d["v"] = plant_misfits(d["v"], [(int(t), int(h)) for t, h in zip(rng.integers(0, S, nv), rng.integers(0, 2, nv))], rng)
    r = run_and_compare(f"causal misfit rows S=4325 n={n}", d, True, 2, 2, 128, 128, n_out=n)
    q, k, v = (to_gpu(d[x], "bf16") for x in ("q", "k", "v"))
    ta = ThinAttention(128, 128, 2, 2, torch.bfloat16, n_out=n, fp64_gram=True)
    _, ex = ta.forward(q, k, v, causal=True, seed=0, return_coreset=True, return_decisions=True)
    torch.cuda.synchronize()
    dec64 = ex["decisions"].cpu().numpy()
    ndiff = int((r["dec"] != dec64).sum())
    say(f"[gram8] causal misfit n={n}: {ndiff} of {dec64.size} decisions differ from the fp64 Gram's")
    assert ndiff == 0
    assert np.array_equal(r["idx"], ex["coreset_idx"].cpu().numpy())


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_integer_and_fp64_gram_forwards_agree(dt):
    """The same causal forward with the integer Gram and with THIN_FP64_GRAM: decision logs equal
    (the two Grams differ by fp64 rounding only), coresets and outputs identical."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    d = inputs.causal_prefill(seed=3, H=4, S=6000) if dt == "bf16" else inputs.causal_prefill_fp8(seed=3, H=4, S=6000)
    q, k, v = (to_gpu(d[x], dt) for x in ("q", "k", "v"))
    res = []
    for fp64 in (False, True):
        ta = ThinAttention(128, 128, 4, 4, torch_dtype(dt), n_out=128, fp64_gram=fp64)
        out, ex = ta.forward(q, k, v, causal=True, seed=2, return_coreset=True, return_decisions=True)
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy(), ex["decisions"].cpu().numpy(), ex["coreset_idx"].cpu().numpy()))
    ndiff = int((res[0][1] != res[1][1]).sum())
    say(f"[gram8] {dt} forward: {ndiff} of {res[0][1].size} decisions differ between the two Grams")
    assert ndiff == 0
    assert np.array_equal(res[0][2], res[1][2])
    assert np.array_equal(res[0][0], res[1][0])
