"""Helpers of the GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare them under the replay protocol.

Acceptance (the float64 oracle is the reference):
* every halving decision equal, except decisions whose oracle margin is below
  1e-6 (near ties), which the oracle then follows; at most 0.5% of the
  decisions may be near ties and none may differ above that margin;
* the coreset (indices and weights) bit-exact after that replay;
* outputs within max-abs 2e-3 (float32) or 2e-2 (bfloat16) of the replayed
  oracle;
* the approximation error against exact attention (relative Frobenius)
  within 5% relative of the oracle's own error.
"""

import sys

import numpy as np
import torch

from oracle import attention as att
from oracle import forward as fwd

# fp8 inputs: after Q K^T the kernel's arithmetic is the bf16 path's (P rounded to bf16,
# fp32 accumulation, bf16 output: the bf16 bound), but Q K^T itself runs on the FP8 MFMA,
# whose sums of 128 products carry errors up to 3.0e-4 of sum_i |q_i k_i| (measured on
# gfx950, both the 16x16x128 and the 16x16x32 form; about 2^-11.7, far coarser than fp32).
# On keys with x8 outlier channels |q.k| reaches ~1000, i.e. logit errors up to ~0.03,
# which move the softmax weights by up to ~3 % and the outputs by a few 1e-2 on top of the
# bf16 rounding: 5e-2
TOL = {"f32": 2e-3, "bf16": 2e-2, "fp8": 5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(d):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[d]


def to_gpu(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype)).cuda()


def sample_queries(B, T, H, n, seed=0, always=()):
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.integers(0, B, n), rng.integers(0, T, n), rng.integers(0, H, n)], axis=1)
    extra = np.array(list(always), dtype=np.int64).reshape(-1, 3)
    return np.unique(np.concatenate([rows, extra]), axis=0)


def run_and_compare(name, d, causal, H, Hkv, E, D, n_out=0, g=0, seed=0, queries=None, scale=0.0,
                    check_error=True, greedy=False, subsample_base=False, block_outputs=False,
                    error_queries=None, fp64_gram=False):
    """Run forward on the GPU and check it against the replayed oracle.  Returns a summary dict.

    queries None compares every output (block_outputs: the oracle forms them a
    unit or an Express block at a time); error_queries then restricts the
    approximation-error check against exact attention to those rows."""
    from sub_quadratic_attention_amd.binding import ThinAttention

    say(f"[parity] {name}: causal={causal} shapes q{d['q'].shape} k{d['k'].shape} v{d['v'].shape}")
    dt = d["dtype"]
    ta = ThinAttention(E, D, H, Hkv, torch_dtype(dt), g=g, n_out=n_out, scale=scale, greedy=greedy,
                       subsample_base=subsample_base, fp64_gram=fp64_gram)
    q, k, v = (to_gpu(d[x], dt) for x in ("q", "k", "v"))
    out, ex = ta.forward(q, k, v, causal=causal, seed=seed, return_coreset=True, return_decisions=True)
    torch.cuda.synchronize()
    B, T = d["q"].shape[:2]
    units = B * Hkv
    dec = ex["decisions"].cpu().numpy()
    decisions = {u: dec[u] for u in range(units)}
    ref = fwd.forward(d["q"], d["k"], d["v"], causal=causal, seed=seed, g=g,
                      n_out=(n_out or None), queries=queries, decisions=decisions,
                      scale=(scale or None), greedy=greedy, subsample_base=subsample_base,
                      block_outputs=block_outputs)
    st = ref["stats"]
    say(f"[parity] {name}: decisions={st.decisions} near_ties={st.near_ties} fails={st.fails} "
        f"min_margin={st.min_margin:.3g}")
    assert st.fails == 0, f"{st.fails} decisions differ above the near-tie margin"
    assert st.near_ties <= 0.005 * max(st.decisions, 1)

    idx = ex["coreset_idx"].cpu().numpy()
    w = ex["coreset_w"].cpu().numpy()
    ln = ex["coreset_len"].cpu().numpy()
    for u in range(units):
        ri, rw = ref["coreset"][u]
        assert ln[u] == len(ri), (u, ln[u], len(ri))
        assert np.array_equal(idx[u, :ln[u]], ri), f"coreset indices differ for unit {u}"
        assert np.array_equal(w[u, :ln[u]].astype(np.float64), rw), f"coreset weights differ for unit {u}"
        assert np.all(idx[u, ln[u]:] == -1) if causal else True

    o = out.float().cpu().numpy().astype(np.float64)
    if queries is None:
        go, ro = o, ref["out"]
    else:
        qr = np.asarray(queries)
        go, ro = o[qr[:, 0], qr[:, 1], qr[:, 2]], ref["out"]
    err = att.max_abs_error(go, ro)
    say(f"[parity] {name}: max|gpu - oracle| = {err:.3g} (tol {TOL[dt]})")
    assert np.all(np.isfinite(go))
    assert err <= TOL[dt]
    summary = {"max_abs": err, "near_ties": st.near_ties, "decisions": st.decisions, "dec": dec, "idx": idx}
    if check_error:
        eq = queries if error_queries is None else error_queries
        exact = fwd.exact(d["q"], d["k"], d["v"], causal=causal, queries=eq, scale=(scale or None))
        if error_queries is not None and queries is None:
            er = np.asarray(error_queries)
            go_e, ro_e = go[er[:, 0], er[:, 1], er[:, 2]], ro[er[:, 0], er[:, 1], er[:, 2]]
        else:
            go_e, ro_e = go, ro
        e_g = att.rel_frobenius_error(go_e, exact)
        e_o = att.rel_frobenius_error(ro_e, exact)
        say(f"[parity] {name}: rel error vs exact: gpu {e_g:.4g} oracle {e_o:.4g}")
        if e_o > 1e-6:
            assert abs(e_g - e_o) <= 0.05 * e_o
        else:
            assert e_g <= TOL[dt]
        summary.update(err_gpu=e_g, err_oracle=e_o)
    return summary
