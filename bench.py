"""Benchmark of the thinned-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one thin_attn_forward call (thinning + coreset attention) on one
batch of seeded synthetic input already resident in HBM.  The default
workload is the 56x56-token ViT token-mixing layer (B=64, S=3136, fp32).
Prints ONE JSON line with the throughput in effective queries*keys per
second (the pairs exact attention would evaluate), timed without
instrumentation, then the per-kernel launch times measured with HIP events
on the launch stream over a second run of the same steps (events around
every launch would slow the timed one, markedly for ~10 us decode launches),
the roofline of the dominant kernel, the exact-attention comparators on the
same GPU and the float64 CPU oracle's rate on a bounded sample.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "thinned-attention queries·keys/sec & ms/call vs exact attn; HBM GB/s, MFMA %"
PEAK = {"hbm_GBs": 8000.0, "f32": 157.3, "bf16": 2500.0, "f64": 78.6}   # MI355X: HBM GB/s, dense TFLOP/s

WORKLOADS = {
    # name: (generator kwargs, causal, H, H_kv, E, D)
    "unmasked_small": (dict(), False, 1, 1, 64, 64),
    "vit_token_mixing": (dict(), False, 1, 1, 64, 64),
    "biggan_self_attention": (dict(), False, 1, 1, 64, 256),
    "causal_prefill": (dict(), True, 32, 32, 128, 128),
    "kv_decode": (dict(), True, 32, 8, 128, 128),
    "selected_keys": (dict(), False, 32, 8, 128, 128),   # thinning after a KV selector (top 4096 of 32768 keys)
    # the ViT layer under the sqrt(S) size rule: base subsampling, then the Compress (56 coreset points)
    "vit_token_mixing_subsampled": (dict(), False, 1, 1, 64, 64),
}
FLAGS = {"vit_token_mixing_subsampled": dict(subsample_base=True)}   # ThinAttention options per workload


def _traffic(label, workload):
    """HBM bytes per launch from the committed counter runs, None if absent or the kernel changed since."""
    from sub_quadratic_attention_amd.profiling import traffic_for
    return traffic_for(label, workload)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="vit_token_mixing", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-exact", action="store_true")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (HBM counter calibration)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Algorithmic work (what the definition needs, not what a kernel happens to do)
# ---------------------------------------------------------------------------
def compress_depth(S, g=0):
    j = 0
    while S % (4 ** (j + 1)) == 0 and S // (4 ** (j + 1)) >= 4 ** g:
        j += 1
    return j, S // (4 ** j)


def base_stride(S, g=0):
    """Stratum length of base subsampling: largest divisor r of s0 with r^2 <= s0 (1 if no level)."""
    j, s0 = compress_depth(S, g)
    if j == 0:
        return 1
    return max(r for r in range(1, s0 + 1) if s0 % r == 0 and r * r <= s0 and s0 // r >= 4 ** g)


def express_visible_total(S, n):
    """Sum over queries t of |visible set| under the Express schedule (per unit)."""
    total = 0
    for beta in range((S + n - 1) // n):
        rows = min(n, S - beta * n)
        raw = rows * (rows + 1) // 2
        if beta < 4:
            total += rows * beta * n + raw
            continue
        E = 1
        while 4 ** (E + 1) <= beta:
            E += 1
        m = 4 ** E
        since = beta - m
        state = n + (since // m) * n + ((since % m) * 2 * n) // m
        total += rows * state + raw
    return total


def express_gram_entries(S, n):
    """Point-Gram entries N(N+1)/2 of every halving (batch and both HALVE passes), per unit."""
    nblk = S // n
    halves = 0
    while 4 ** (halves + 1) <= nblk:
        halves += 1
    done = 0
    e = 1
    while 4 ** e < nblk:
        for j in range(3):
            if 4 ** e * (2 + j) <= nblk:
                done += 1
        e += 1
    tri = lambda N: N * (N + 1) // 2
    return halves * (tri(4 * n) + tri(2 * n)) + done * tri(2 * n)


def work_model(name, B, T, S, H, Hkv, E, D, causal, elt, subsample_base=False):
    """Per-forward algorithmic flops / bytes of each kernel label."""
    units = B * Hkv
    if not causal:
        S_full = S
        S = S // base_stride(S) if subsample_base else S   # the list the Compress runs on
        j, s0 = compress_depth(S)
        n_out = S >> j
        # levels of bins of at most 16 points run in the fused small-bin kernel
        # (it reads each point of the level once: HBM-bound), the others on
        # the pair-Gram tiles
        small = lambda N: N <= 16 and E % 32 == 0 and D % 32 == 0
        # bins of 20-32 points: one workgroup per bin, Gram and walk fused (fp64 MFMA)
        medium = lambda N: 16 < N <= 32 and N % 4 == 0 and E % 32 == 0 and D % 32 == 0 and \
            N * ((E + D) * elt + 16) <= 96 * 1024
        levels = [(S // (s0 * 4 ** l), s0 * 2 ** (l + 1)) for l in range(1, j + 1)]   # (bins, N) per unit
        gram_entries = sum(bins * N * (N + 1) // 2 for bins, N in levels if not small(N) and not medium(N))
        medium_entries = sum(bins * N * (N + 1) // 2 for bins, N in levels if medium(N))
        small_bytes = units * sum(bins * N * (E + D) * elt + bins * (N // 2) * 5 for bins, N in levels if small(N))
        keys = n_out
        pairs_eff = B * H * T * S_full
        visible = B * H * T * keys
        attn_bytes = (B * T * H * (E + D) + units * n_out * (E + D)) * elt
    else:
        n_out = 2
        while n_out * n_out < S:
            n_out *= 2
        gram_entries = express_gram_entries(S, n_out)
        small_bytes = 0
        medium_entries = 0
        pairs_eff = B * H * T * (T + 1) // 2
        visible = B * H * express_visible_total(S, n_out)
        attn_bytes = (B * T * H * E + units * S * (E + D) + B * T * H * D) * elt
    return dict(
        n_out=n_out,
        pairs_eff=pairs_eff,
        attention=dict(flops=2.0 * visible * (E + D), bytes=attn_bytes),
        pair_gram=dict(flops=2.0 * (E + D) * gram_entries * units, bytes=None) if gram_entries else None,
        small_halving=dict(flops=None, bytes=small_bytes) if small_bytes else None,
        medium_halving=dict(flops=2.0 * (E + D) * medium_entries * units, bytes=None) if medium_entries else None,
    )


# ---------------------------------------------------------------------------
def decode_main(args):
    """KV-cache thinning + decode: one step = ingest the 131k-token history into a
    fresh Express state (thinned once), then 1024 one-token decode steps."""
    import torch
    from sub_quadratic_attention_amd import inputs
    from sub_quadratic_attention_amd.binding import KVState, ThinAttention

    _, _, H, Hkv, E, D = WORKLOADS["kv_decode"]
    d = inputs.kv_decode(seed=0)
    kh, vh = (torch.from_numpy(d[x]).to(torch.bfloat16).cuda() for x in ("k_hist", "v_hist"))
    qs, ks, vs = (torch.from_numpy(d[x]).to(torch.bfloat16).cuda() for x in ("q_steps", "k_steps", "v_steps"))
    B, S0 = kh.shape[:2]
    steps_dec = qs.shape[1]
    n_out = 2
    while n_out * n_out < S0:
        n_out *= 2
    ta = ThinAttention(E, D, H, Hkv, torch.bfloat16)
    st = KVState(ta, B, n_out)
    st._workspace(S0)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def one_pass(timing=False):
        nonlocal st
        st = KVState(ta, B, n_out)
        st._ws = ws
        st.append(kh, vh, stream=stream)
        for i in range(steps_dec):
            st.decode(qs[:, i], ks[:, i], vs[:, i], out=out, stream=stream)

    ws = torch.empty(max(int(ta.lib.thin_attn_kv_workspace_size(st.kv, S0)), 256), dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    # the timed region runs without per-launch events (two events per ~10 us
    # decode launch would be a visible part of it) ...
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_pass()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # ... and the same steps run again with events around every launch for the
    # per-kernel table and the roofline
    ta.set_timing(True)
    for _ in range(args.steps):
        one_pass()
    torch.cuda.synchronize()
    recs = ta.timing_records()
    ta.set_timing(False)
    per_kernel = {}
    for label, ms in recs:
        r = per_kernel.setdefault(label, dict(launches=0, total_ms=0.0))
        r["launches"] += 1
        r["total_ms"] += ms
    for r in per_kernel.values():
        r["avg_ms"] = r["total_ms"] / r["launches"]
        r["ms_per_step"] = r["total_ms"] / args.steps
        r["launches_per_step"] = r["launches"] / args.steps
    # decode-only timing of the 1024 steps (state ingested once, outside the region)
    st = KVState(ta, B, n_out)
    st._ws = ws
    st.append(kh, vh, stream=stream)
    torch.cuda.synchronize()
    a = time.perf_counter()
    for i in range(steps_dec):
        st.decode(qs[:, i], ks[:, i], vs[:, i], out=out, stream=stream)
    torch.cuda.synchronize()
    decode_us = (time.perf_counter() - a) * 1e6 / steps_dec
    pairs = sum(H * (S0 + i + 1) for i in range(steps_dec))
    # visible rows per step (algorithmic bytes of the decode attention): cache + buffer + raw block
    vis = 0
    tmp = KVState(ta, B, n_out)
    tmp._ws = ws
    tmp.append(kh, vh, stream=stream)
    torch.cuda.synchronize()
    _, _, ln = tmp.coreset()
    vis_rows = int(ln.sum().item())
    dec_bytes = vis_rows * (E + D) * 2 + B * H * (E + D) * 2
    kd = per_kernel.get("kv_decode", {})
    roof = None
    if kd:
        gbs = dec_bytes / (kd["avg_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK["hbm_GBs"], "unit": "GB/s",
                "frac": round(gbs / PEAK["hbm_GBs"], 4), "traffic": _traffic("kv_decode", "kv_decode"),
                "kernel": "kv_decode",
                "work_per_launch_bytes": dec_bytes, "avg_launch_ms": kd["avg_ms"]}
    exact = {}
    if not args.no_exact:
        # exact decode over the full cache (GQA by repeating KV heads), one step
        kt = torch.cat([kh, ks], dim=1).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1).contiguous()
        vt = torch.cat([vh, vs], dim=1).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1).contiguous()
        f = torch.nn.functional.scaled_dot_product_attention
        qq = qs[:, -1].reshape(B, H, 1, E)
        for _ in range(3):
            f(qq, kt, vt)
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(50):
            f(qq, kt, vt)
        torch.cuda.synchronize()
        exact["sdpa_decode_step_us"] = (time.perf_counter() - a) * 1e6 / 50
        exact["decode_speedup_vs_sdpa"] = exact["sdpa_decode_step_us"] / decode_us
        del kt, vt
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import forward as ofwd
        sub = dict(k_hist=d["k_hist"][:, :, :1], v_hist=d["v_hist"][:, :, :1], q_steps=d["q_steps"][:, :256, :H // Hkv],
                   k_steps=d["k_steps"][:, :256, :1], v_steps=d["v_steps"][:, :256, :1])
        with threadpool_limits(1):
            a = time.perf_counter()
            ofwd.decode(sub["k_hist"], sub["v_hist"], sub["q_steps"], sub["k_steps"], sub["v_steps"], n_out=n_out)
            sec = time.perf_counter() - a
        cpair = sum((H // Hkv) * (S0 + i + 1) for i in range(256))
        cpu = {"value": cpair / sec, "unit": "queries·keys/s", "cores": 1, "kind": "oracle",
               "sample": f"1 of {Hkv} KV heads with its {H // Hkv} query heads: ingest + 256 of {steps_dec} steps",
               "seconds": round(sec, 3)}
    line = {
        "metric": METRIC, "value": pairs / (ms_per_step * 1e-3), "unit": "queries·keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "kv_decode", "B": B, "H": H, "H_kv": Hkv, "S0": S0, "decode_steps": steps_dec,
                   "E": E, "D": D, "n_out": n_out, "seed": 0},
        "decode_us_per_token": decode_us,
        "kernels": {l: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                    for l, r in per_kernel.items()},
        "roofline": roof, "exact": exact, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(every (batch, KV head) unit is independent; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sub_quadratic_attention_amd import inputs
    from sub_quadratic_attention_amd.binding import ThinAttention

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return
    if args.workload == "kv_decode":
        return decode_main(args)
    gen_kw, causal, H, Hkv, E, D = WORKLOADS[args.workload]
    d = inputs.workload(args.workload, seed=0, **gen_kw)
    dt = d["dtype"]
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    elt = 4 if dt == "f32" else 2
    q, k, v = (torch.from_numpy(d[x]).to(tdt).cuda() for x in ("q", "k", "v"))
    B, T = q.shape[:2]
    S = k.shape[1]
    opts = FLAGS.get(args.workload, {})
    ta = ThinAttention(E, D, H, Hkv, tdt, **opts)
    out = torch.empty((B, T, H, D), dtype=tdt, device="cuda")
    stream = torch.cuda.current_stream()
    sel = d.get("key_idx")   # thinning after a selector: the list is the point set (L keys per unit)
    if sel is not None:
        key_idx = torch.from_numpy(sel).cuda()
        L = sel.shape[2]
        ws = ta.workspace(B, T, L, False)

        def step():
            ta.forward_subset(q, k, v, key_idx, seed=0, workspace=ws, out=out, stream=stream)
    else:
        L = S
        ws = ta.workspace(B, T, S, causal)

        def step():
            ta.forward(q, k, v, causal=causal, seed=0, workspace=ws, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the same steps again with events around every launch (per-kernel table, roofline)
    ta.set_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    recs = ta.timing_records()
    ta.set_timing(False)

    wm = work_model(args.workload, B, T, L, H, Hkv, E, D, causal, elt, **opts)   # (a selector's list: its L keys)
    per_kernel = {}
    for label, ms in recs:
        r = per_kernel.setdefault(label, dict(launches=0, total_ms=0.0))
        r["launches"] += 1
        r["total_ms"] += ms
    for label, r in per_kernel.items():
        r["avg_ms"] = r["total_ms"] / r["launches"]
        r["ms_per_step"] = r["total_ms"] / args.steps
        r["launches_per_step"] = r["launches"] / args.steps
    dom = max(per_kernel, key=lambda l: per_kernel[l]["total_ms"])

    def roof(label):
        r = per_kernel[label]
        w = wm.get(label)
        if not w:
            return None
        if w["flops"] is None:   # bandwidth-bound: algorithmic bytes only
            per_launch_bytes = w["bytes"] / r["launches_per_step"]
            gbs = per_launch_bytes / (r["avg_ms"] * 1e-3) / 1e9
            return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK["hbm_GBs"], "unit": "GB/s",
                    "frac": round(gbs / PEAK["hbm_GBs"], 4), "traffic": None, "kernel": label,
                    "work_per_launch_bytes": per_launch_bytes, "avg_launch_ms": r["avg_ms"]}
        per_launch_flops = w["flops"] / r["launches_per_step"]
        peak_key = "f64" if label in ("pair_gram", "medium_halving") else dt
        achieved = per_launch_flops / (r["avg_ms"] * 1e-3) / 1e12
        res = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK[peak_key], "unit": "TFLOP/s",
               "frac": round(achieved / PEAK[peak_key], 4), "traffic": None, "kernel": label,
               "work_per_launch_flops": per_launch_flops, "avg_launch_ms": r["avg_ms"],
               "dtype": peak_key}
        if w.get("bytes"):
            gbs = w["bytes"] / r["launches_per_step"] / (r["avg_ms"] * 1e-3) / 1e9
            res["hbm_GBs"] = round(gbs, 1)
            res["hbm_frac"] = round(gbs / PEAK["hbm_GBs"], 4)
        return res

    roofline = roof(dom) if wm.get(dom) else None
    if roofline:
        roofline["traffic"] = _traffic(dom, args.workload)
    rooflines = {l: roof(l) for l in per_kernel if wm.get(l)}

    # exact comparators on the same GPU
    exact = {}
    if not args.no_exact:
        if sel is not None:   # exact attention over the selected keys
            gi = key_idx.long().permute(0, 2, 1)[..., None]
            k, v = (torch.gather(x, 1, gi.expand(-1, -1, -1, x.shape[3])) for x in (k, v))
        qt, kt, vt = (x.permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
        if Hkv != H:
            kt = kt.repeat_interleave(H // Hkv, dim=1)
            vt = vt.repeat_interleave(H // Hkv, dim=1)
        f = torch.nn.functional.scaled_dot_product_attention
        for _ in range(2):
            f(qt, kt, vt, is_causal=causal)
        torch.cuda.synchronize()
        n_ex = max(3, min(args.steps, 10))
        a = time.perf_counter()
        for _ in range(n_ex):
            f(qt, kt, vt, is_causal=causal)
        torch.cuda.synchronize()
        exact["sdpa_ms"] = (time.perf_counter() - a) * 1e3 / n_ex
        del qt, kt, vt
        if not causal and sel is None:
            ex = ThinAttention(E, D, H, Hkv, tdt)
            for _ in range(2):
                ex.coreset_attention(q, k, v, out=out)
            torch.cuda.synchronize()
            a = time.perf_counter()
            for _ in range(n_ex):
                ex.coreset_attention(q, k, v, out=out)
            torch.cuda.synchronize()
            exact["own_exact_kernel_ms"] = (time.perf_counter() - a) * 1e3 / n_ex
        exact["speedup_vs_sdpa"] = exact["sdpa_ms"] / ms_per_step

    # float64 CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import forward as ofwd
        if causal:
            heads = min(H, 2)
            rows = np.array([[0, t, h] for h in range(heads) for t in range(0, T, 64)])
            sub = {x: d[x][:, :, :heads] for x in ("q", "k", "v")}
            pairs = sum(t + 1 for _, t, _ in rows)
            desc = f"{heads} of {H} heads (thinning in full), {len(rows)} sampled queries"
            with threadpool_limits(1):
                a = time.perf_counter()
                ofwd.forward(sub["q"], sub["k"], sub["v"], causal=True, queries=rows)
                sec = time.perf_counter() - a
        elif sel is not None:
            hk = min(Hkv, 2)
            g = H // Hkv
            sub = dict(q=d["q"][:, :, :hk * g], k=d["k"][:, :, :hk], v=d["v"][:, :, :hk])
            pairs = B * hk * g * T * L
            desc = f"{hk} of {Hkv} KV heads ({hk * g} query heads), every query (thinning + attention)"
            with threadpool_limits(1):
                a = time.perf_counter()
                ofwd.forward_subset(sub["q"], sub["k"], sub["v"], sel[:, :hk])
                sec = time.perf_counter() - a
        else:
            nb = B if args.workload != "biggan_self_attention" else min(B, 8)
            sub = {x: d[x][:nb] for x in ("q", "k", "v")}
            pairs = nb * H * T * S
            desc = f"{nb} of {B} batch entries, every query (thinning + attention)"
            with threadpool_limits(1):
                a = time.perf_counter()
                ofwd.forward(sub["q"], sub["k"], sub["v"], causal=False, **opts)
                sec = time.perf_counter() - a
        cpu = {"value": pairs / sec, "unit": "queries·keys/s", "cores": 1, "kind": "oracle",
               "sample": desc, "seconds": round(sec, 3)}

    line = {
        "metric": METRIC,
        "value": wm["pairs_eff"] / (ms_per_step * 1e-3),
        "unit": "queries·keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": dict({"workload": args.workload, "B": B, "H": H, "H_kv": Hkv, "T": T, "S": S, "E": E, "D": D,
                        "causal": causal, "n_out": wm["n_out"], "seed": 0}, **({"L": L} if sel is not None else {}),
                       **opts),
        "kernels": {l: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                    for l, r in per_kernel.items()},
        "roofline": roofline,
        "rooflines": rooflines,
        "exact": exact,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
