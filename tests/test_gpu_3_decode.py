"""GPU parity of the streaming Express state (KV-cache thinning + decode) against the oracle."""

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import express as oexp
from oracle import forward as fwd
from sub_quadratic_attention_amd import inputs
from tests.parity import TOL, say, to_gpu, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


def _run_stream(d, n, H, Hkv, E, D, seed=0, chunks=None, greedy=False):
    """Ingest the history (in `chunks` appends, or one bulk append), then decode step by step.

    Returns (outputs [B, steps, H, D] float64, decisions per unit (flat, chronological), state)."""
    from sub_quadratic_attention_amd.binding import KVState, ThinAttention
    dt = d["dtype"]
    ta = ThinAttention(E, D, H, Hkv, torch_dtype(dt), greedy=greedy)
    B = d["k_hist"].shape[0]
    st = KVState(ta, B, n, seed=seed)
    kh, vh = to_gpu(d["k_hist"], dt), to_gpu(d["v_hist"], dt)
    decs = []
    S0 = kh.shape[1]
    bounds = [0, S0] if chunks is None else chunks
    for a, b in zip(bounds[:-1], bounds[1:]):
        decs.append(st.append(kh[:, a:b], vh[:, a:b], return_decisions=True))
    qs, ks, vs = to_gpu(d["q_steps"], dt), to_gpu(d["k_steps"], dt), to_gpu(d["v_steps"], dt)
    outs = []
    for i in range(qs.shape[1]):
        o, dd = st.decode(qs[:, i], ks[:, i], vs[:, i], return_decisions=True)
        outs.append(o.float())
        decs.append(dd)
    torch.cuda.synchronize()
    out = torch.stack(outs, dim=1).cpu().numpy().astype(np.float64)
    dec = torch.cat(decs, dim=1).cpu().numpy()
    return out, dec, st


def _check(name, d, n, H, Hkv, E, D, seed=0, chunks=None, greedy=False):
    say(f"[decode] {name}")
    out, dec, st = _run_stream(d, n, H, Hkv, E, D, seed, chunks, greedy)
    units = dec.shape[0]
    ref, stats, logs = fwd.decode(d["k_hist"], d["v_hist"], d["q_steps"], d["k_steps"], d["v_steps"],
                                  n_out=n, seed=seed, decisions={u: dec[u] for u in range(units)}, greedy=greedy)
    say(f"[decode] {name}: decisions={stats.decisions} near_ties={stats.near_ties} fails={stats.fails}")
    assert stats.decisions == dec.shape[1] * units
    assert stats.fails == 0 and stats.near_ties <= 0.005 * max(stats.decisions, 1)
    err = att.max_abs_error(out, ref)
    say(f"[decode] {name}: max|gpu - oracle| = {err:.3g}")
    assert err <= TOL[d["dtype"]]
    # the state's summary equals the oracle's cache / buffer / raw block after the stream
    idx, w, ln = (x.cpu().numpy() for x in st.coreset())
    total = d["k_hist"].shape[1] + d["q_steps"].shape[1]
    for u in range(units):
        assert w[u, :ln[u]].sum() == total - _in_progress(total, n)
    return out


def _in_progress(total, n):
    """Tokens of a subsampling group longer than a block still in progress after `total`
    tokens (they join the weights when the group completes); 0 while m / 2 <= n."""
    beta = total // n
    if beta < 4:
        return 0
    m = 4
    while m * 4 <= beta:
        m *= 4
    return (beta * n) % (m // 2)


def _stream(seed, S0, steps, Hkv, H, E=128, D=128, dtype="bf16"):
    return inputs.kv_decode(seed=seed, Hkv=Hkv, H=H, S0=S0, steps=steps, E=E, D=D, walk_len=S0 + steps, dtype=dtype)


def test_decode_crosses_batch_and_halve():
    """n=32: bulk history of 1900 tokens, 200 decode steps across a batch halving and a HALVE (token 2048)."""
    d = _stream(0, 1900, 200, Hkv=2, H=8)
    _check("bulk 1900 + 200 steps", d, 32, 8, 2, 128, 128)


def test_decode_greedy_signs():
    """Greedy-sign halvings in the streaming state: the same stream as above, keep-first iff alpha_i < 0 in every walk."""
    d = _stream(0, 1900, 200, Hkv=2, H=8)
    _check("greedy bulk 1900 + 200 steps", d, 32, 8, 2, 128, 128, greedy=True)


def test_decode_block_path_from_empty():
    """History streamed in uneven appends from an empty state (block-by-block ingest)."""
    d = _stream(1, 700, 100, Hkv=2, H=2, E=64, D=64)
    _check("appends 10/90/300/300 + 100 steps", d, 16, 2, 2, 64, 64, chunks=[0, 10, 100, 400, 700])


def test_decode_fp32_gqa8():
    d = _stream(2, 600, 80, Hkv=1, H=8, dtype="f32")
    _check("fp32 G=8", d, 32, 8, 1, 128, 128)


def test_decode_long_state_gqa8():
    """n=256, history of 3840 tokens: 768 cache + 384 buffer rows, so each decode step sees
    1153..1216 keys, split over workgroups of 128 keys (with 8 heads sharing a KV head the
    partials of smaller splits would not fit the merge's LDS)."""
    d = _stream(5, 3840, 64, Hkv=1, H=8)
    _check("n=256 long state, G=8", d, 256, 8, 1, 128, 128)


def test_decode_matches_causal_forward():
    """A decode step sees what a causal forward query at the same token sees."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    d = _stream(3, 1000, 64, Hkv=2, H=2)
    out, _, _ = _run_stream(d, 32, 2, 2, 128, 128)
    k = np.concatenate([d["k_hist"], d["k_steps"]], axis=1)
    v = np.concatenate([d["v_hist"], d["v_steps"]], axis=1)
    q = np.concatenate([np.zeros((1, 1000, 2, 128), np.float32), d["q_steps"]], axis=1)
    ta = ThinAttention(128, 128, 2, 2, torch.bfloat16, n_out=32)
    f = ta.forward(to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16"), causal=True)
    torch.cuda.synchronize()
    fo = f.float().cpu().numpy()[:, 1000:]
    assert att.max_abs_error(out, fo) <= 2 * TOL["bf16"]


def test_checkpoint_round_trip():
    """Export the counters and copy the device state mid-stream: the resumed stream is bit-identical."""
    from sub_quadratic_attention_amd.binding import KVState, ThinAttention
    d = _stream(4, 500, 120, Hkv=2, H=4)
    ta = ThinAttention(128, 128, 4, 2, torch.bfloat16)
    qs, ks, vs = (to_gpu(d[x], "bf16") for x in ("q_steps", "k_steps", "v_steps"))
    a = KVState(ta, 1, 32, seed=9)
    a.append(to_gpu(d["k_hist"], "bf16"), to_gpu(d["v_hist"], "bf16"))
    for i in range(50):
        a.decode(qs[:, i], ks[:, i], vs[:, i])
    meta = a.export_meta()
    b = KVState(ta, 1, 32, seed=9)
    b.buffer.copy_(a.buffer)
    b.import_meta(meta)
    assert b.tokens == a.tokens
    for i in range(50, 120):
        oa = a.decode(qs[:, i], ks[:, i], vs[:, i])
        ob = b.decode(qs[:, i], ks[:, i], vs[:, i])
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), i


def test_kv_decode_full_size_window():
    """The 131k-token, 8-KV-head state (n_out 512) and 1024 decode steps; every output checked."""
    d = inputs.kv_decode(seed=0)
    _check("kv_decode S0=131072 x 1024 steps", d, 512, 32, 8, 128, 128)


def test_long_generation():
    """Long generation: 8000 decode steps after a 16-token history with n_out = 128 cross two
    HALVEs and five batch halvings per KV head; every output and decision is checked."""
    d = _stream(6, 16, 8000, Hkv=2, H=4, E=64, D=64)
    _check("long generation n_out=128", d, 128, 4, 2, 64, 64)


def test_decode_cache_size_curve():
    """Cache size against error: 500 decode steps with n_out = 16, 32, 64 (two, two and one
    HALVEs); each stream matches the replayed oracle, and the error against exact causal
    attention falls as the cache grows."""
    S0, steps, H, Hkv = 16, 500, 4, 2
    d = _stream(7, S0, steps, Hkv=Hkv, H=H, E=64, D=64)
    k = np.concatenate([d["k_hist"], d["k_steps"]], axis=1)
    v = np.concatenate([d["v_hist"], d["v_steps"]], axis=1)
    B = k.shape[0]
    rows = np.array([(b, S0 + i, h) for b in range(B) for i in range(steps) for h in range(H)])
    q = np.zeros((B, S0 + steps, H, 64))
    q[:, S0:] = d["q_steps"]
    exact = fwd.exact(q, k, v, causal=True, queries=rows).reshape(B, steps, H, 64)
    sizes = (16, 32, 64)
    errs = []
    for n in sizes:
        out = _check(f"decode n_out={n}", d, n, H, Hkv, 64, 64)
        errs.append(att.rel_frobenius_error(out, exact))
    say("[decode] cache size vs error (relative Frobenius against exact): " +
        ", ".join(f"n_out={n}: {e:.4f}" for n, e in zip(sizes, errs)))
    assert errs[2] < errs[1] < errs[0]


# ---- subsampling groups longer than a block (m / 2 > n_out) -----------------------------

def test_decode_groups_longer_than_a_block():
    """n = 16: bulk history of 600 tokens, then 3000 decode steps through the HALVE at token
    1024 into the epoch m = 64 (groups of 32 tokens, two blocks each) and the next HALVE."""
    d = _stream(7, 600, 3000, Hkv=2, H=8)
    _check("n=16 bulk 600 + 3000 steps", d, 16, 8, 2, 128, 128)


def test_bulk_ingest_with_a_group_in_progress():
    """n = 16, bulk history of 4900 tokens: epoch m = 256 (groups of 128 tokens = 8 blocks) with a
    group in progress at the end of the chunk; 300 decode steps complete it and the next ones."""
    d = _stream(8, 4900, 300, Hkv=1, H=4)
    _check("n=16 bulk 4900 + 300 steps", d, 16, 4, 1, 128, 128)


def test_chunked_appends_groups_longer_than_a_block():
    """The same long stream appended in uneven chunks (block by block), then decoded."""
    d = _stream(9, 2300, 100, Hkv=2, H=4)
    _check("n=16 chunks", d, 16, 4, 2, 128, 128, chunks=[0, 37, 700, 1500, 2222, 2300])
