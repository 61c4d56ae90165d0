"""Seeded synthetic inputs shaped like the Thinformer workloads.

This module only draws numbers: it holds none of the method's arithmetic, and
both the HIP path's tests / benchmark and the float64 oracle read its arrays.
The pages list the experiments (the "Thinformer" README, "Getting Started":
T2T-ViT ImageNet classification, BigGAN generation, long-context prefill,
KV-cache compression, long-form decoding) but ship no data; these generators
stand in for them with the shapes, dtypes and value structure of each
workload.  Every array is drawn in float64 from NumPy's PCG64 seeded by a
child of ``SeedSequence(seed)`` (one child per tensor), then rounded to the
workload dtype (round-to-nearest-even; "fp8" is OCP FP8 E4M3); the returned
float32 arrays hold values that are exact in that dtype.

Workloads (all sizes overridable for reduced test cases):

``unmasked_small``  B=1, H=1, T=S=256, E=D=64, fp32; q, k, v i.i.d. N(0,1)
                    times E^-1/4.
``vit_token_mixing`` B=64, H=1, T=S=3136 (56x56 patches), E=D=64, fp32;
                    q = Zq + P, k = Zk + P, v = Zv with Z ~ N(0,1) and P a
                    2-D sin-cos positional field of amplitude 0.5 on the grid
                    (token n = 56 r + c; channels 0..31 encode r, 32..63
                    encode c, as (sin, cos)(x * 10000^(-i/16)), i = 0..15).
``biggan_self_attention`` B=32, H=1, T=S=4096 (64x64 map), E=64, D=256,
                    bf16; every channel is a 64x64 N(0,1) field blurred by a
                    separable 8-tap Gaussian (weights ~ exp(-(i-3.5)^2/8),
                    circular), divided by its own standard deviation over the
                    map and flattened row-major.
``causal_prefill``  B=1, H=32, T=S=32768, E=D=128, bf16; q, k ~ N(0,1) with
                    4 channels per head (the same for q and k, drawn without
                    replacement) scaled x8; v ~ N(0,1).
``kv_decode``       B=1, H_kv=8, H=32 (4 query heads per KV head), E=D=128,
                    bf16; keys z_t + mu_h(t) with mu_h a Gaussian random walk
                    of N(0, I/131072) steps; v ~ N(0,1).  S0=131072 tokens of
                    history, then 1024 decode steps continuing the walk, with
                    q ~ N(0,1) for the 32 query heads.
"""

import numpy as np


def bf16_round(x):
    """Round float64/float32 values to the nearest bfloat16 (ties to even); float32 out."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(f)
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    out = np.where(nan, np.float32(np.nan), out)
    return out.astype(np.float32)


def fp8_round(x):
    """Round to the nearest OCP FP8 E4M3 value (E4M3FN: 1 sign, 4 exponent bits of bias 7,
    3 mantissa bits; subnormals down to 2^-9; largest finite 448), ties to even; magnitudes
    above 448 saturate (the generators draw none so large).  float32 out."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)   # binade; subnormals share 2^-6's
    q = 2.0 ** (e - 3)                                                  # spacing: 3 mantissa bits
    r = np.minimum(np.round(a / q) * q, 448.0)                          # np.round: ties to even
    return (np.sign(x) * r).astype(np.float32)


def _cast(x, dtype):
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp8":
        return fp8_round(x)
    raise ValueError(dtype)


def _streams(seed, n):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def unmasked_small(seed=0, B=1, H=1, S=256, E=64, D=64, dtype="f32"):
    rq, rk, rv, _ = _streams(seed, 4)
    c = E ** -0.25
    return dict(q=_cast(rq.standard_normal((B, S, H, E)) * c, dtype),
                k=_cast(rk.standard_normal((B, S, H, E)) * c, dtype),
                v=_cast(rv.standard_normal((B, S, H, D)) * c, dtype),
                dtype=dtype, causal=False)


def positional_field(side=56, E=64, amplitude=0.5):
    """[side*side, E] sin-cos field: first half of the channels encodes the row, second the column."""
    n = np.arange(side * side)
    r, c = n // side, n % side
    quarter = E // 4
    omega = 10000.0 ** (-np.arange(quarter) / quarter)
    P = np.zeros((side * side, E))
    for half, coord in ((0, r), (1, c)):
        ang = coord[:, None] * omega[None, :]
        P[:, half * (E // 2) + 0:(half + 1) * (E // 2):2] = np.sin(ang)
        P[:, half * (E // 2) + 1:(half + 1) * (E // 2):2] = np.cos(ang)
    return amplitude * P


def vit_token_mixing(seed=0, B=64, side=56, E=64, D=64, dtype="f32"):
    S = side * side
    rq, rk, rv, _ = _streams(seed, 4)
    P = positional_field(side, E)[None, :, None, :]
    return dict(q=_cast(rq.standard_normal((B, S, 1, E)) + P, dtype),
                k=_cast(rk.standard_normal((B, S, 1, E)) + P, dtype),
                v=_cast(rv.standard_normal((B, S, 1, D)), dtype),
                dtype=dtype, causal=False)


def _blurred_fields(rng, B, C, side):
    x = rng.standard_normal((B, C, side, side))
    taps = np.exp(-((np.arange(8) - 3.5) ** 2) / 8.0)
    taps /= taps.sum()
    for axis in (2, 3):
        y = np.zeros_like(x)
        for i, t in enumerate(taps):
            y += t * np.roll(x, 4 - i, axis=axis)       # y[n] = sum_i t_i x[n + i - 4]
        x = y
    x /= x.std(axis=(2, 3), keepdims=True)
    return x.reshape(B, C, side * side).transpose(0, 2, 1)[:, :, None, :]


def biggan_self_attention(seed=0, B=32, side=64, E=64, D=256, dtype="bf16"):
    rq, rk, rv, _ = _streams(seed, 4)
    return dict(q=_cast(_blurred_fields(rq, B, E, side), dtype),
                k=_cast(_blurred_fields(rk, B, E, side), dtype),
                v=_cast(_blurred_fields(rv, B, D, side), dtype),
                dtype=dtype, causal=False)


def causal_prefill(seed=0, B=1, H=32, S=32768, E=128, D=128, outliers=4,
                   outlier_scale=8.0, dtype="bf16"):
    rq, rk, rv, rx = _streams(seed, 4)
    q = rq.standard_normal((B, S, H, E))
    k = rk.standard_normal((B, S, H, E))
    for h in range(H):
        ch = rx.choice(E, outliers, replace=False)
        q[:, :, h, ch] *= outlier_scale
        k[:, :, h, ch] *= outlier_scale
    return dict(q=_cast(q, dtype), k=_cast(k, dtype),
                v=_cast(rv.standard_normal((B, S, H, D)), dtype),
                dtype=dtype, causal=True)


def kv_decode(seed=0, B=1, Hkv=8, H=32, S0=131072, steps=1024, E=128, D=128,
              walk_len=131072, dtype="bf16"):
    rq, rk, rv, rx = _streams(seed, 4)
    total = S0 + steps
    mu = np.cumsum(rx.standard_normal((B, total, Hkv, E)) / np.sqrt(walk_len), axis=1)
    k = _cast(rk.standard_normal((B, total, Hkv, E)) + mu, dtype)
    del mu
    v = _cast(rv.standard_normal((B, total, Hkv, D)), dtype)
    q = _cast(rq.standard_normal((B, steps, H, E)), dtype)
    return dict(k_hist=k[:, :S0], v_hist=v[:, :S0], k_steps=k[:, S0:],
                v_steps=v[:, S0:], q_steps=q, dtype=dtype, causal=True)


def top_k_keys(k, q, L):
    """Stand-in KV selector (the role SnapKV-style selection plays before thinning): per unit
    (b, h_kv), the L keys with the largest |<k, mean query of the unit's heads>|, in token order."""
    B, S, Hkv, E = k.shape
    group = q.shape[2] // Hkv
    qm = np.asarray(q, dtype=np.float64).reshape(B, q.shape[1], Hkv, group, E).mean(axis=(1, 3))
    score = np.abs(np.einsum("bshe,bhe->bhs", np.asarray(k, dtype=np.float64), qm))
    return np.sort(np.argsort(-score, axis=2, kind="stable")[:, :, :L], axis=2).astype(np.int32)


def selected_keys(seed=0, B=1, H=32, Hkv=8, S=32768, T=1024, L=4096, E=128, D=128, dtype="bf16"):
    """Thinning after a KV selector: an LLM layer's 32k keys (4 outlier channels per head, as
    in the causal prefill), T queries, and per KV head the top-L keys of the stand-in selector."""
    rq, rk, rv, rx = _streams(seed, 4)
    q = rq.standard_normal((B, T, H, E))
    k = rk.standard_normal((B, S, Hkv, E))
    for h in range(Hkv):
        ch = rx.choice(E, 4, replace=False)
        q[:, :, h * (H // Hkv):(h + 1) * (H // Hkv), ch] *= 8.0
        k[:, :, h, ch] *= 8.0
    q, k = _cast(q, dtype), _cast(k, dtype)
    return dict(q=q, k=k, v=_cast(rv.standard_normal((B, S, Hkv, D)), dtype), key_idx=top_k_keys(k, q, L),
                dtype=dtype, causal=False)


def causal_prefill_fp8(seed=0, **kw):
    """The causal prefill with its q, k, v rounded to FP8 E4M3."""
    return causal_prefill(seed=seed, dtype="fp8", **kw)


def kv_decode_fp8(seed=0, **kw):
    """The KV-cache decode stream with keys, values and queries rounded to FP8 E4M3."""
    return kv_decode(seed=seed, dtype="fp8", **kw)


WORKLOADS = {
    "unmasked_small": unmasked_small,
    "causal_prefill_fp8": causal_prefill_fp8,
    "kv_decode_fp8": kv_decode_fp8,
    "vit_token_mixing": vit_token_mixing,
    "biggan_self_attention": biggan_self_attention,
    "causal_prefill": causal_prefill,
    "kv_decode": kv_decode,
    "selected_keys": selected_keys,
    "vit_token_mixing_subsampled": vit_token_mixing,
}


def workload(name, seed=0, **sizes):
    return WORKLOADS[name](seed=seed, **sizes)
