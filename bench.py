"""Benchmark of the thinned-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one thin_attn_forward call (thinning + coreset attention) on one
batch of seeded synthetic input already resident in HBM.  The default
workload is the largest single-GPU one, the causal Thinformer Express
prefill of a decoder layer (B=1, H=32, T=S=32768, E=D=128, bf16).
Prints ONE JSON line with the throughput in effective queries*keys per
second (the pairs exact attention would evaluate), timed without
instrumentation, then the per-kernel launch times measured with HIP events
on the launch stream over a second run of the same steps (events around
every launch would slow the timed one, markedly for ~10 us decode launches),
the roofline of the dominant kernel, the exact-attention comparators on the
same GPU (torch SDPA, and this library's own kernels with thinning
disabled) and the float64 CPU oracle's rate on the host cores: whole units
(batch entry, KV head) in parallel, one single-threaded process per core,
started before the GPU is touched.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "thinned-attention queries·keys/sec & ms/call vs exact attn; HBM GB/s, MFMA %"
PEAK = {"hbm_GBs": 8000.0, "f32": 157.3, "bf16": 2500.0, "fp8": 5000.0, "f64": 78.6,
        "i8": 5000.0}   # MI355X: HBM GB/s, dense TFLOP/s (int8: TOP/s)

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
    # the causal prefill and the decode state with FP8 (E4M3) inputs
    "causal_prefill_fp8": (dict(), True, 32, 32, 128, 128),
    "kv_decode_fp8": (dict(), True, 32, 8, 128, 128),
}
TORCH_DTYPE = {"f32": "float32", "bf16": "bfloat16", "fp8": "float8_e4m3fn"}
ELT = {"f32": 4, "bf16": 2, "fp8": 1}
FLAGS = {"vit_token_mixing_subsampled": dict(subsample_base=True)}   # ThinAttention options per workload


def _dense_exact_ms(q, k, v, scale, n_ex, cap_bytes=8 << 30):
    """Exact attention as dense products (q [.., T, E], k [.., S, E], v [.., S, D], the same
    leading dims): scores q k^T, softmax in fp32, then P v.  Every operand of a product is a
    contiguous tensor (K is transposed into a copy first).  None when the fp32 scores would
    exceed cap_bytes."""
    import torch
    S = k.shape[-2]
    if q.numel() // q.shape[-1] * S * 4 > cap_bytes:
        return None
    kT = k.transpose(-1, -2).contiguous()

    def run():
        sc = torch.matmul(q, kT).float() * scale
        return torch.matmul(torch.softmax(sc, dim=-1).to(v.dtype), v)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    a = time.perf_counter()
    for _ in range(n_ex):
        run()
    torch.cuda.synchronize()
    del kT
    return (time.perf_counter() - a) * 1e3 / n_ex


def _traffic(label, workload):
    """HBM bytes per launch from the committed counter runs, None if absent or the kernel changed since."""
    from sub_quadratic_attention_amd.profiling import traffic_for
    return traffic_for(label, workload)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="causal_prefill", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-exact", action="store_true")
    p.add_argument("--one-stream", action="store_true",
                   help="run the timed steps with every launch on one stream (as the per-kernel pass does)")
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


def express_halvings(S, n):
    """(bins per unit, points per bin) of every halving launch of the causal path, per unit."""
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
    return ([(done, 2 * n)] if done else []) + [(1, 4 * n), (1, 2 * n)] * halves


def gram8_runs(dt, E, D, N, fp64_gram=False):
    """Does the library take the exact integer Gram (int8 digit products) for bins of N points?"""
    return (not fp64_gram and dt in ("bf16", "fp8") and E % 64 == 0 and D % 64 == 0 and 64 <= E <= 256
            and 64 <= D <= 256 and N >= 256)


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


def work_model(name, B, T, S, H, Hkv, E, D, causal, elt, subsample_base=False, out_elt=None, dt="bf16"):
    """Per-forward algorithmic flops / bytes of each kernel label.  Pair-Gram launches of bf16 /
    fp8 bins of >= 256 points run as exact integer dot products on the int8 MFMA (nd^2 digit
    products per multiply-add of the definition, nd = 4 for bf16 and 3 for fp8) after a digit
    pass that reads every point once and writes its digits."""
    units = B * Hkv
    nd = 3 if dt == "fp8" else 4
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
        tiles = [(bins, N) for bins, N in levels if not small(N) and not medium(N)]
        gram_entries = sum(bins * N * (N + 1) // 2 for bins, N in levels if not small(N) and not medium(N))
        medium_entries = sum(bins * N * (N + 1) // 2 for bins, N in levels if medium(N))
        small_bytes = units * sum(bins * N * (E + D) * elt + bins * (N // 2) * 5 for bins, N in levels if small(N))
        keys = n_out
        pairs_eff = B * H * T * S_full
        visible = B * H * T * keys
        attn_bytes = (B * T * H * E + units * n_out * (E + D)) * elt + B * T * H * D * (out_elt or elt)
    else:
        n_out = 2
        while n_out * n_out < S:
            n_out *= 2
        gram_entries = express_gram_entries(S, n_out)
        tiles = express_halvings(S, n_out)
        small_bytes = 0
        medium_entries = 0
        pairs_eff = B * H * T * (T + 1) // 2
        visible = B * H * express_visible_total(S, n_out)
        attn_bytes = (B * T * H * E + units * S * (E + D)) * elt + B * T * H * D * (out_elt or elt)
    i8 = [(bins, N) for bins, N in tiles if gram8_runs(dt, E, D, N)]
    i8_entries = sum(bins * N * (N + 1) // 2 for bins, N in i8)
    i8_points = units * sum(bins * N for bins, N in i8)
    if causal and gram8_runs(dt, E, D, 4 * n_out):
        # a HALVE's second halving reads the digits of its first (its points are among them);
        # when the batches take the integer Gram too, HALVEs after the first read the digits of
        # HALVE 0's points and of the batch points (every later HALVE point is one of them)
        halves = sum(1 for bins, N in tiles if N == 4 * n_out)
        i8_points -= units * halves * 2 * n_out
        if halves and len(tiles) > 2 * halves and gram8_runs(dt, E, D, 2 * n_out):
            i8_points -= units * (halves - 1) * 4 * n_out
    pair_gram = None
    if gram_entries:
        pair_gram = dict(flops=2.0 * (E + D) * gram_entries * units, bytes=None)
        if i8_entries == gram_entries:   # every tile launch on the int8 MFMA
            pair_gram.update(int8_ops=nd * nd * pair_gram["flops"], nd=nd)
    return dict(
        n_out=n_out,
        gram_digits=dict(flops=None, bytes=i8_points * ((E + D) * (elt + nd) + 10)) if i8_points else None,
        pairs_eff=pairs_eff,
        attention=dict(flops=2.0 * visible * (E + D), bytes=attn_bytes, qk_flops=2.0 * visible * E,
                       pv_flops=2.0 * visible * D),
        pair_gram=pair_gram,
        small_halving=dict(flops=None, bytes=small_bytes) if small_bytes else None,
        medium_halving=dict(flops=2.0 * (E + D) * medium_entries * units, bytes=None) if medium_entries else None,
    )


# ---------------------------------------------------------------------------
# The float64 CPU oracle on the host cores
# ---------------------------------------------------------------------------
_CPU = {}   # inputs of the oracle workers (inherited through fork)


def host_cores():
    """Cores this process may run on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _oracle_unit(u):
    """One unit of the oracle, single-threaded: returns (effective pairs, seconds)."""
    from threadpoolctl import threadpool_limits
    from oracle import forward as ofwd
    c = _CPU
    d, name, H, Hkv = c["d"], c["name"], c["H"], c["Hkv"]
    g = H // Hkv
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if name == "kv_decode":
            hk = u
            ofwd.decode(d["k_hist"][:, :, hk:hk + 1], d["v_hist"][:, :, hk:hk + 1], d["q_steps"][:, :, hk * g:(hk + 1) * g],
                        d["k_steps"][:, :, hk:hk + 1], d["v_steps"][:, :, hk:hk + 1], n_out=c["n_out"])
            S0, steps = d["k_hist"].shape[1], d["q_steps"].shape[1]
            pairs = sum(g * (S0 + i + 1) for i in range(steps))
        else:
            b, hk = divmod(u, Hkv)
            sub = {x: d[x][b:b + 1, :, hk * g:(hk + 1) * g] if x == "q" else d[x][b:b + 1, :, hk:hk + 1]
                   for x in ("q", "k", "v")}
            T, S = sub["q"].shape[1], sub["k"].shape[1]
            if "key_idx" in d:
                sel = d["key_idx"][b:b + 1, hk:hk + 1]
                ofwd.forward_subset(sub["q"], sub["k"], sub["v"], sel, **c["opts"])
                pairs = g * T * sel.shape[2]
            elif c["causal"]:
                ofwd.forward(sub["q"], sub["k"], sub["v"], causal=True)
                pairs = g * T * (T + 1) // 2
            else:
                ofwd.forward(sub["q"], sub["k"], sub["v"], causal=False, **c["opts"])
                pairs = g * T * S
        return pairs, time.perf_counter() - t0


def cpu_baseline(name, d, H, Hkv, causal, opts, n_out=None):
    """The oracle as it stands, timed on the host cores: every unit of the workload (all
    queries of a batch entry and KV head, thinning included) mapped over a pool of
    single-threaded processes, one per core.  Runs before the GPU is initialised (fork)."""
    import multiprocessing as mp
    B = d["k_hist"].shape[0] if name == "kv_decode" else d["k"].shape[0]
    units = B * Hkv
    cores = host_cores()
    sample = units
    _CPU.update(d=d, name=name, H=H, Hkv=Hkv, causal=causal, opts=opts, n_out=n_out)
    ctx = mp.get_context("fork")
    with ctx.Pool(min(cores, sample)) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_unit, range(sample), chunksize=1)
        wall = time.perf_counter() - t0
    pairs = sum(p for p, _ in res)
    unit = "KV head" if Hkv > 1 or name == "kv_decode" else "batch entry"
    what = "ingest + every decode step" if name == "kv_decode" else "thinning + every query"
    return {"value": pairs / wall, "unit": "queries·keys/s", "cores": min(cores, sample), "kind": "oracle",
            "sample": f"all {units} units ({unit}) in full ({what}), one single-threaded process per core",
            "extrapolated": False, "seconds": round(wall, 3),
            "unit_seconds_mean": round(sum(t for _, t in res) / len(res), 3),
            "host_cpus": {"affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
                          "cpu_count": os.cpu_count()}}


# ---------------------------------------------------------------------------
def decode_main(args):
    """KV-cache thinning + decode: one step = ingest the 131k-token history into a
    fresh Express state (thinned once), then 1024 one-token decode steps."""
    import torch
    from sub_quadratic_attention_amd import inputs
    from sub_quadratic_attention_amd.binding import KVState, ThinAttention

    _, _, H, Hkv, E, D = WORKLOADS[args.workload]
    d = inputs.workload(args.workload, seed=0)
    dt = d["dtype"]
    tdt = getattr(torch, TORCH_DTYPE[dt])
    odt = torch.bfloat16 if dt == "fp8" else tdt
    S0 = d["k_hist"].shape[1]
    n_out = 2
    while n_out * n_out < S0:
        n_out *= 2
    # the oracle on the host cores first: its worker processes fork before the GPU is touched
    cpu = None if args.no_cpu_baseline else cpu_baseline("kv_decode", d, H, Hkv, True, {}, n_out=n_out)
    kh, vh = (torch.from_numpy(d[x]).to(tdt).cuda() for x in ("k_hist", "v_hist"))
    qs, ks, vs = (torch.from_numpy(d[x]).to(tdt).cuda() for x in ("q_steps", "k_steps", "v_steps"))
    B = kh.shape[0]
    steps_dec = qs.shape[1]
    ta = ThinAttention(E, D, H, Hkv, tdt)
    st = KVState(ta, B, n_out)
    st._workspace(S0)
    out = torch.empty((B, H, D), dtype=odt, device="cuda")
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
    dec_bytes = vis_rows * (E + D) * ELT[dt] + B * H * E * ELT[dt] + B * H * D * (2 if dt == "fp8" else ELT[dt])
    kd = per_kernel.get("kv_decode", {})
    roof = None
    if kd:
        gbs = dec_bytes / (kd["avg_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK["hbm_GBs"], "unit": "GB/s",
                "frac": round(gbs / PEAK["hbm_GBs"], 4), "traffic": _traffic("kv_decode", args.workload),
                "kernel": "kv_decode",
                "work_per_launch_bytes": dec_bytes, "avg_launch_ms": kd["avg_ms"]}
    exact = {}
    if not args.no_exact:
        # exact decode over the full cache (GQA by repeating KV heads), one step
        # (SDPA has no fp8 kernel: its comparator runs on the same values in bf16)
        sdt = odt
        kt = torch.cat([kh, ks], dim=1).to(sdt).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1).contiguous()
        vt = torch.cat([vh, vs], dim=1).to(sdt).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1).contiguous()
        f = torch.nn.functional.scaled_dot_product_attention
        qq = qs[:, -1].to(sdt).reshape(B, H, 1, E)
        for _ in range(3):
            f(qq, kt, vt)
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(50):
            f(qq, kt, vt)
        torch.cuda.synchronize()
        exact["sdpa_decode_step_us"] = (time.perf_counter() - a) * 1e6 / 50
        exact["decode_speedup_vs_sdpa"] = exact["sdpa_decode_step_us"] / decode_us
        # the same step as dense products over the KV heads: [G, E] x [E, S] scores per KV head
        G = H // Hkv
        kg = torch.cat([kh, ks], dim=1).to(sdt).permute(0, 2, 1, 3).contiguous()   # [B, Hkv, S, E]
        vg = torch.cat([vh, vs], dim=1).to(sdt).permute(0, 2, 1, 3).contiguous()   # [B, Hkv, S, D]
        qg = qs[:, -1].to(sdt).reshape(B, Hkv, G, E).contiguous()
        dense = _dense_exact_ms(qg, kg, vg, scale=1.0 / math.sqrt(E), n_ex=50)
        if dense is not None:
            exact["dense_matmul_decode_step_us"] = dense * 1e3
            exact["decode_speedup_vs_dense_matmul"] = dense * 1e3 / decode_us
        del kt, vt, kg, vg
        # this library's attention kernel with thinning disabled: the last step's 32 query
        # heads (one token each) against all S0 + steps keys (unmasked over the whole cache is
        # exactly the causal decode of the last token)
        kf, vf = torch.cat([kh, ks], dim=1).contiguous(), torch.cat([vh, vs], dim=1).contiguous()
        q1 = qs[:, -1:].contiguous()
        o1 = torch.empty((B, 1, H, D), dtype=odt, device="cuda")
        ex = ThinAttention(E, D, H, Hkv, tdt)
        for _ in range(3):
            ex.coreset_attention(q1, kf, vf, out=o1, stream=stream)
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(50):
            ex.coreset_attention(q1, kf, vf, out=o1, stream=stream)
        torch.cuda.synchronize()
        exact["own_exact_kernel_decode_step_us"] = (time.perf_counter() - a) * 1e6 / 50
        del kf, vf
    line = {
        "metric": METRIC, "value": pairs / (ms_per_step * 1e-3), "unit": "queries·keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "H_kv": Hkv, "S0": S0, "decode_steps": steps_dec,
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

    if args.calibrate_copy:
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        n = args.calibrate_copy << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return
    if args.workload.startswith("kv_decode"):
        return decode_main(args)
    gen_kw, causal, H, Hkv, E, D = WORKLOADS[args.workload]
    d = inputs.workload(args.workload, seed=0, **gen_kw)
    opts = FLAGS.get(args.workload, {})
    # the oracle on the host cores first: its worker processes fork before the GPU is touched
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload, d, H, Hkv, causal, opts)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dt = d["dtype"]
    tdt = getattr(torch, TORCH_DTYPE[dt])
    odt = torch.bfloat16 if dt == "fp8" else tdt   # fp8 inputs give bf16 outputs
    elt = ELT[dt]
    q, k, v = (torch.from_numpy(d[x]).to(tdt).cuda() for x in ("q", "k", "v"))
    B, T = q.shape[:2]
    S = k.shape[1]
    ta = ThinAttention(E, D, H, Hkv, tdt, one_stream=args.one_stream, **opts)
    # per-kernel launch times come from a handle whose launches all go on one
    # stream: with the causal path's second stream, kernels overlap and a
    # launch's event time would include its neighbours'
    ta1 = ThinAttention(E, D, H, Hkv, tdt, one_stream=True, **opts)
    out = torch.empty((B, T, H, D), dtype=odt, device="cuda")
    stream = torch.cuda.current_stream()
    sel = d.get("key_idx")   # thinning after a selector: the list is the point set (L keys per unit)
    if sel is not None:
        key_idx = torch.from_numpy(sel).cuda()
        L = sel.shape[2]
        ws = ta.workspace(B, T, L, False)

        def step(h=ta):
            h.forward_subset(q, k, v, key_idx, seed=0, workspace=ws, out=out, stream=stream)
    else:
        L = S
        ws = ta.workspace(B, T, S, causal)

        def step(h=ta):
            h.forward(q, k, v, causal=causal, seed=0, workspace=ws, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the same steps again, one stream: untimed per launch (the serial step time), then with
    # events around every launch (per-kernel table, roofline)
    for _ in range(2):
        step(ta1)
    torch.cuda.synchronize()
    a1 = time.perf_counter()
    for _ in range(args.steps):
        step(ta1)
    torch.cuda.synchronize()
    ms_one_stream = (time.perf_counter() - a1) * 1e3 / args.steps
    ta1.set_timing(True)
    for _ in range(args.steps):
        step(ta1)
    torch.cuda.synchronize()
    recs = ta1.timing_records()
    ta1.set_timing(False)

    wm = work_model(args.workload, B, T, L, H, Hkv, E, D, causal, elt, out_elt=2 if dt == "fp8" else elt, dt=dt,
                    **opts)   # (a selector's list: its L keys)
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
                    "frac": round(gbs / PEAK["hbm_GBs"], 4), "traffic": _traffic(label, args.workload), "kernel": label,
                    "work_per_launch_bytes": per_launch_bytes, "avg_launch_ms": r["avg_ms"]}
        per_launch_flops = w["flops"] / r["launches_per_step"]
        if w.get("int8_ops"):
            # exact dot products as int8 digit products: against the int8 MFMA peak, with the
            # definition's fp64 multiply-adds per second beside it (what an fp64 Gram would need)
            ops = w["int8_ops"] / r["launches_per_step"]
            achieved = ops / (r["avg_ms"] * 1e-3) / 1e12
            f64 = per_launch_flops / (r["avg_ms"] * 1e-3) / 1e12
            return {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK["i8"], "unit": "TOP/s",
                    "frac": round(achieved / PEAK["i8"], 4), "traffic": _traffic(label, args.workload),
                    "kernel": label, "work_per_launch_ops": ops, "avg_launch_ms": r["avg_ms"],
                    "dtype": f"i8 (exact digit products, {w['nd']} digits per feature)",
                    "fp64_equivalent": {"flops_per_launch": per_launch_flops, "achieved": round(f64, 3),
                                        "peak": PEAK["f64"], "unit": "TFLOP/s", "frac": round(f64 / PEAK["f64"], 4)}}
        peak_key = "f64" if label in ("pair_gram", "medium_halving") else dt
        peak = PEAK[peak_key]
        if label == "attention" and dt == "fp8":
            # Q K^T on the fp8 MFMA, P V on the bf16 MFMA: the peak of that mix of work
            peak = w["flops"] / (w["qk_flops"] / PEAK["fp8"] + w["pv_flops"] / PEAK["bf16"])
            peak_key = "fp8 (Q K^T) + bf16 (P V)"
        achieved = per_launch_flops / (r["avg_ms"] * 1e-3) / 1e12
        res = {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(peak, 1), "unit": "TFLOP/s",
               "frac": round(achieved / peak, 4), "traffic": _traffic(label, args.workload), "kernel": label,
               "work_per_launch_flops": per_launch_flops, "avg_launch_ms": r["avg_ms"],
               "dtype": peak_key}
        if w.get("bytes"):
            gbs = w["bytes"] / r["launches_per_step"] / (r["avg_ms"] * 1e-3) / 1e9
            res["hbm_GBs"] = round(gbs, 1)
            res["hbm_frac"] = round(gbs / PEAK["hbm_GBs"], 4)
        return res

    roofline = roof(dom) if wm.get(dom) else None
    rooflines = {l: roof(l) for l in per_kernel if wm.get(l)}

    # exact comparators on the same GPU
    exact = {}
    if not args.no_exact:
        k_all, v_all = k, v
        if sel is not None:   # exact attention over the selected keys
            gi = key_idx.long().permute(0, 2, 1)[..., None]
            k, v = (torch.gather(x, 1, gi.expand(-1, -1, -1, x.shape[3])) for x in (k, v))
        # (SDPA has no fp8 kernel: for fp8 inputs its comparator runs on the same values in bf16)
        qt, kt, vt = (x.to(odt).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
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
        if not causal:
            dense = _dense_exact_ms(qt, kt, vt, scale=1.0 / math.sqrt(E), n_ex=n_ex)
            if dense is not None:
                exact["dense_matmul_ms"] = dense
                exact["speedup_vs_dense_matmul"] = dense / ms_per_step
        del qt, kt, vt
        # this library's own kernels with thinning disabled: the unmasked coreset attention
        # over every key (over the selected keys for a selector's list), and the causal forward
        # with a cache of at least S tokens, which is exact causal attention
        if causal:
            n_ex_out = 2
            while n_ex_out < S:
                n_ex_out *= 2
            ex = ThinAttention(E, D, H, Hkv, tdt, n_out=n_ex_out)
            ws_ex = ex.workspace(B, T, S, True)
            own = lambda: ex.forward(q, k, v, causal=True, seed=0, workspace=ws_ex, out=out, stream=stream)
        else:
            ex = ThinAttention(E, D, H, Hkv, tdt)
            if sel is not None:
                own = lambda: ex.coreset_attention(q, k_all, v_all, idx=key_idx.reshape(B * Hkv, -1), out=out,
                                                   stream=stream)
            else:
                own = lambda: ex.coreset_attention(q, k, v, out=out, stream=stream)
        for _ in range(2):
            own()
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(n_ex):
            own()
        torch.cuda.synchronize()
        exact["own_exact_kernel_ms"] = (time.perf_counter() - a) * 1e3 / n_ex
        exact["speedup_vs_sdpa"] = exact["sdpa_ms"] / ms_per_step
        exact["speedup_vs_own_exact"] = exact["own_exact_kernel_ms"] / ms_per_step

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
        "kernel_timing": "HIP events around every launch, all launches on one stream",
        "streams": 1 if args.one_stream else 2,
        "ms_per_step_one_stream": ms_one_stream,
        "roofline": roofline,
        "rooflines": rooflines,
        "exact": exact,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
