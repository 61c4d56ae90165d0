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
    (dict(flags=4), -1), (dict(flags=0x80000001), -1), (dict(E=96), -2), (dict(dtype=0, E=64, D=256), -2), (dict(E=0), -1),
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


def test_causal_schedule_range_is_enforced():
    lib = _lib()
    rc, h = _create(dtype=1, E=128, D=128, n_out=4)
    try:
        assert lib.thin_attn_decision_count(h, 4 * 64 + 4, 1) == -2     # groups longer than a block
        assert lib.thin_attn_workspace_size(h, 1, 300, 300, 1) == 0
        fake = ctypes.c_void_p(0x1000)
        rc = lib.thin_attn_forward(h, fake, fake, fake, 1, 300, 300, 1, 0, fake, None, None, None, None,
                                   fake, 1 << 20, None)
        assert rc == -2
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
        rc = lib.thin_attn_halving(h, fake, fake, 1, 16, fake, 7, 0, 0, 0, fake, None, fake, None)
        assert rc == -1
        rc = lib.thin_attn_halving(h, fake, fake, 1, 16, fake, 4096, 0, 0, 0, fake, None, fake, None)
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
