"""C-ABI checks that need no GPU: exports, argument validation, size rules."""

import ctypes
import os
import re

import pytest

from oracle import compress as cmp
from oracle import express as exp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "thin_attn.h")

binding = pytest.importorskip("sub_quadratic_attention_amd.binding")


def _lib():
    try:
        return binding.load_library()
    except ImportError as e:       # not built here: build() must run first
        pytest.fail(str(e))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(thin_attn_\w+)\s*\(", text)))


def test_every_declared_function_is_exported():
    lib = _lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.exported_symbols())


def _cfg(**kw):
    base = dict(dtype=0, E=64, D=64, H=1, H_kv=1, g=0, n_out=0, delta=0.5, scale=0.0, flags=0)
    base.update(kw)
    return binding._Config(*[base[f] for f, _ in binding._Config._fields_])


def _create(**kw):
    lib = _lib()
    h = ctypes.c_void_p()
    rc = lib.thin_attn_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -1), (dict(H=3, H_kv=2), -1), (dict(n_out=3), -1), (dict(g=-1), -1),
    (dict(flags=16), -1), (dict(flags=0x80000001), -1), (dict(E=96), -2), (dict(dtype=0, E=64, D=256), -2), (dict(E=0), -1),
])
def test_create_rejects(kw, code):
    rc, h = _create(**kw)
    assert rc == code
    assert _lib().thin_attn_last_error(None)


@pytest.mark.parametrize("S,g", [(3136, 0), (196, 0), (144, 0), (4096, 0), (3136, 1), (7, 0), (192, 0)])
def test_subsample_base_sizes_match_oracle(S, g):
    lib = _lib()
    rc, h = _create(flags=binding.THIN_SUBSAMPLE_BASE, g=g)
    assert rc == 0
    try:
        assert lib.thin_attn_coreset_size(h, S, 0) == cmp.coreset_size(S, g, True)
        assert lib.thin_attn_decision_count(h, S, 0) == cmp.decisions_per_unit(S, g, True)
    finally:
        lib.thin_attn_destroy(h)


def test_create_accepts_greedy_signs():
    rc, h = _create(flags=binding.THIN_GREEDY_SIGNS)
    assert rc == 0
    _lib().thin_attn_destroy(h)


@pytest.mark.parametrize("S", [256, 3136, 4096, 16, 12, 7])
def test_unmasked_sizes_match_oracle(S):
    lib = _lib()
    rc, h = _create()
    assert rc == 0
    try:
        assert lib.thin_attn_coreset_size(h, S, 0) == cmp.coreset_size(S)
        assert lib.thin_attn_decision_count(h, S, 0) == cmp.decisions_per_unit(S)
        assert lib.thin_attn_coreset_capacity(h, S, 0) == cmp.coreset_size(S)
    finally:
        lib.thin_attn_destroy(h)


@pytest.mark.parametrize("S,n", [(32768, 0), (131072, 0), (4096 + 77, 64), (500, 16), (50, 64), (67, 4)])
def test_causal_sizes_match_oracle(S, n):
    lib = _lib()
    rc, h = _create(dtype=1, E=128, D=128, n_out=n)
    assert rc == 0
    try:
        size = n or exp.default_cache_size(S)
        assert lib.thin_attn_coreset_size(h, S, 1) == size
        assert lib.thin_attn_coreset_capacity(h, S, 1) == 6 * size
        expected = sum(p for _, _, p in exp.schedule(S, size))
        assert lib.thin_attn_decision_count(h, S, 1) == expected
        assert lib.thin_attn_workspace_size(h, 1, S, S, 1) >= 256
    finally:
        lib.thin_attn_destroy(h)


@pytest.mark.parametrize("S,n", [(4 * 64 + 4, 4), (300, 4), (4096 + 9, 16), (1 << 20, 16), (300000, 256)])
def test_causal_sizes_past_groups_longer_than_a_block(S, n):
    """Subsampling groups longer than a block (m / 2 > n_out) are supported: decision counts
    and workspace follow the oracle's schedule."""
    lib = _lib()
    rc, h = _create(dtype=1, E=128, D=128, n_out=n)
    try:
        assert lib.thin_attn_decision_count(h, S, 1) == sum(p for _, _, p in exp.schedule(S, n))
        assert lib.thin_attn_workspace_size(h, 1, S, S, 1) >= 256
    finally:
        lib.thin_attn_destroy(h)


def test_forward_argument_errors_before_any_launch():
    lib = _lib()
    rc, h = _create(dtype=1, E=128, D=128, H=4, H_kv=2)
    fake = ctypes.c_void_p(0x1000)
    try:
        # causal needs T == S
        rc = lib.thin_attn_forward(h, fake, fake, fake, 1, 10, 12, 1, 0, fake, None, None, None, None,
                                   fake, 1 << 20, None)
        assert rc == -1 and b"T == S" in lib.thin_attn_last_error(h)
        # null inputs
        rc = lib.thin_attn_forward(h, None, fake, fake, 1, 16, 16, 0, 0, fake, None, None, None, None,
                                   fake, 1 << 20, None)
        assert rc == -1
        # workspace too small
        need = lib.thin_attn_workspace_size(h, 2, 4096, 4096, 0)
        assert need > 256
        rc = lib.thin_attn_forward(h, fake, fake, fake, 2, 4096, 4096, 0, 0, fake, None, None, None, None,
                                   ctypes.c_void_p(0x100000), need - 1, None)
        assert rc == -3
        # misaligned workspace
        rc = lib.thin_attn_forward(h, fake, fake, fake, 2, 4096, 4096, 0, 0, fake, None, None, None, None,
                                   ctypes.c_void_p(0x100010), need, None)
        assert rc == -1
        # bad causal flag
        rc = lib.thin_attn_forward(h, fake, fake, fake, 1, 16, 16, 2, 0, fake, None, None, None, None,
                                   fake, 1 << 20, None)
        assert rc == -1
        # empty batch is a no-op
        rc = lib.thin_attn_forward(h, None, None, None, 0, 16, 16, 0, 0, None, None, None, None, None,
                                   None, 0, None)
        assert rc == 0
        # halving: N odd / too large
        rc = lib.thin_attn_halving(h, fake, fake, 1, 16, fake, 7, 0, 0, 0, fake, None, fake, None, 0, None)
        assert rc == -1
        rc = lib.thin_attn_halving(h, fake, fake, 1, 16, fake, 4096, 0, 0, 0, fake, None, fake, None, 0, None)
        assert rc == -1
        # coreset attention: idx NULL needs n == S
        rc = lib.thin_attn_coreset_attention(h, fake, fake, fake, 1, 8, 16, None, None, 8, fake, None)
        assert rc == -1
    finally:
        lib.thin_attn_destroy(h)


def test_timing_records_start_empty():
    lib = _lib()
    rc, h = _create()
    try:
        assert lib.thin_attn_timing_count(h) == 0
        assert lib.thin_attn_set_timing(h, 1) == 0
        assert lib.thin_attn_timing_count(h) == 0
        ms = ctypes.c_float()
        assert lib.thin_attn_timing_read(h, 0, None, 0, ctypes.byref(ms)) == -1
        assert lib.thin_attn_set_timing(h, 0) == 0
    finally:
        lib.thin_attn_destroy(h)


def test_compress_bin_beyond_walk_lds_is_rejected():
    """S = 16396 = 4 * 4099: one Compress level whose bin holds all 16396 points; its walk
    would need 263 KB of LDS.  Rejected before any launch (fake device pointers)."""
    lib = _lib()
    rc, h = _create()
    fake = ctypes.c_void_p(0x1000)
    try:
        rc = lib.thin_attn_forward(h, fake, fake, fake, 1, 16396, 16396, 0, 0, fake, None, None, None, None,
                                   ctypes.c_void_p(0x100000), 1 << 40, None)
        assert rc == -2 and b"LDS" in lib.thin_attn_last_error(h)
        key_idx = ctypes.c_void_p(0x2000)
        rc = lib.thin_attn_forward_subset(h, fake, fake, fake, key_idx, 1, 16, 20000, 16396, 0, fake, None, None,
                                          None, None, ctypes.c_void_p(0x100000), 1 << 40, None)
        assert rc == -2
    finally:
        lib.thin_attn_destroy(h)


def test_cache_halving_beyond_walk_lds_is_rejected():
    """n_out = 2048: a HALVE of 8192 points does not fit the walk's LDS."""
    lib = _lib()
    rc, h = _create(dtype=1, E=128, D=128, n_out=2048)
    fake = ctypes.c_void_p(0x1000)
    try:
        rc = lib.thin_attn_forward(h, fake, fake, fake, 1, 8192, 8192, 1, 0, fake, None, None, None, None,
                                   ctypes.c_void_p(0x100000), 1 << 40, None)
        assert rc == -2 and b"LDS" in lib.thin_attn_last_error(h)
        # below four blocks nothing is halved: accepted as far as the argument checks go
        assert lib.thin_attn_workspace_size(h, 1, 6000, 6000, 1) >= 256
        kv = ctypes.c_void_p()
        rc = lib.thin_attn_kv_create(h, ctypes.c_void_p(0x100000), 1 << 40, 1, 2048, 0, ctypes.byref(kv))
        assert rc == -2
    finally:
        lib.thin_attn_destroy(h)


def _kv_on_fake_state(lib, h, n=16):
    """A streaming state over a fake (never touched) device buffer: export / import are host-only."""
    kv = ctypes.c_void_p()
    need = lib.thin_attn_kv_state_size(h, 1, n)
    assert need > 0
    rc = lib.thin_attn_kv_create(h, ctypes.c_void_p(0x100000), need, 1, n, 7, ctypes.byref(kv))
    assert rc == 0
    return kv


def test_kv_import_rejects_tampered_counters():
    """Export of a fresh state, then records whose counters disagree with their token count
    (raw block past the block, oversized cache, buffer with no epoch) are refused."""
    import struct
    lib = _lib()
    rc, h = _create(dtype=1, E=128, D=128, H=4, H_kv=2)
    try:
        kv = _kv_on_fake_state(lib, h)
        size = lib.thin_attn_kv_export(kv, None, 0)
        buf = ctypes.create_string_buffer(size)
        assert lib.thin_attn_kv_export(kv, buf, size) == size
        fmt = "<IIiiiiiiiiqqQ"   # magic, version, B, units, n, nC, nBf, nRaw, nb, nh, tokens, m, seed
        assert struct.calcsize(fmt) <= size
        rec = list(struct.unpack_from(fmt, buf.raw))
        assert lib.thin_attn_kv_import(kv, buf, size) == 0          # the untouched record

        def imported(**kw):
            r = list(rec)
            names = ["magic", "version", "B", "units", "n", "nC", "nBf", "nRaw", "nb", "nh", "tokens", "m", "seed"]
            for k2, v2 in kw.items():
                r[names.index(k2)] = v2
            b2 = ctypes.create_string_buffer(size)
            struct.pack_into(fmt, b2, 0, *r)
            return lib.thin_attn_kv_import(kv, b2, size)

        n = rec[4]
        assert imported(tokens=5 * n + 3, nC=n, nBf=n // 2, nRaw=3, nb=0, nh=1, m=4) == 0   # a consistent record
        assert imported(nRaw=n + 5, tokens=n + 5) == -1           # raw block longer than a block
        assert imported(tokens=3 * n, nC=4 * n) == -1             # cache of 4n after 3 blocks
        assert imported(tokens=2 * n, nC=2 * n, nBf=5) == -1      # buffer before any thin phase
        assert imported(tokens=-1) == -1
        assert imported(n=32) == -1                               # another state's record
        lib.thin_attn_kv_destroy(kv)
    finally:
        lib.thin_attn_destroy(h)


def test_integer_gram_scratch_sizes():
    """The workspace holds the exact integer Gram's scratch exactly where that Gram runs: bf16 and
    fp8 handles with bins of >= 256 points; fp32 handles and THIN_FP64_GRAM need none of it."""
    lib = _lib()
    sizes = {}
    for name, kw in [("bf16", dict(dtype=1)), ("bf16_fp64", dict(dtype=1, flags=8)), ("fp8", dict(dtype=2)),
                     ("f32", dict(dtype=0))]:
        rc, h = _create(E=128, D=128, H=32, H_kv=32, **kw)
        assert rc == 0
        try:
            sizes[name] = (lib.thin_attn_workspace_size(h, 1, 32768, 32768, 1),
                           lib.thin_attn_halving_workspace_size(h, 1, 1024),
                           lib.thin_attn_halving_workspace_size(h, 1, 128))
        finally:
            lib.thin_attn_destroy(h)
    n, units = 256, 32
    # digits (4 per bf16 feature, 3 per fp8 one) of K and V, two scales and two flags per point
    halve = lambda nd: (units * 1024 * nd * 256 + 255) // 256 * 256 + units * 1024 * 10
    assert sizes["bf16"][1] == halve(4) and sizes["fp8"][1] == halve(3)
    assert sizes["bf16"][2] == sizes["fp8"][2] == 0          # bins below 256 points stay on fp64
    assert sizes["bf16_fp64"][1] == sizes["f32"][1] == 0
    # the causal prefill: one scratch for HALVE 0's points (4n per unit) and the batch points (7
    # batches of 2n), and the digit rows of the batch outputs (7n), a HALVE's input (4n) and the
    # HALVE outputs (3 HALVEs of n)
    rows = units * (4 * n + 7 * 2 * n)
    shared = lambda nd: (rows * nd * 256 + 255) // 256 * 256 + rows * 10
    al = lambda x: (x + 255) // 256 * 256
    lists = al(4 * units * 7 * n) + al(4 * units * 4 * n) + al(4 * units * 3 * n)
    assert sizes["bf16"][0] - sizes["bf16_fp64"][0] == al(shared(4)) + lists
