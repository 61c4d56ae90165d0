"""thin_attn_forward_static (no workspace argument: the library's static device scratch)
against thin_attn_forward on the same inputs, through the C ABI: two calls in a row, the
second on smaller inputs, for the unmasked and the causal path, and the size limit."""

import ctypes

import numpy as np
import pytest
import torch

from sub_quadratic_attention_amd import inputs
from tests.parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _static(ta, q, k, v, causal, seed=0):
    """Output, coreset and decisions of thin_attn_forward_static (plain C-ABI call)."""
    lib = ta.lib
    B, T = q.shape[:2]
    S = k.shape[1]
    units = B * ta.H_kv
    out = torch.full((B, T, ta.H, ta.D), float("nan"), dtype=ta.dtype, device="cuda")
    cap = ta.coreset_capacity(S, causal)
    idx = torch.full((units, cap), -7, dtype=torch.int32, device="cuda")
    w = torch.zeros((units, cap), dtype=torch.float32, device="cuda")
    ln = torch.zeros((units,), dtype=torch.int32, device="cuda")
    nd = max(ta.decision_count(S, causal), 1)
    dec = torch.full((units, nd), 9, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.thin_attn_forward_static(ta.h, _p(q), _p(k), _p(v), B, T, S, int(causal), ctypes.c_uint64(seed), _p(out),
                                      _p(idx), _p(w), _p(ln), _p(dec), stream)
    assert rc == 0, lib.thin_attn_last_error(ta.h)
    torch.cuda.synchronize()
    return out, idx, w, ln, dec[:, :ta.decision_count(S, causal)]


def _check(ta, d, causal, name):
    tdt = ta.dtype
    q, k, v = (torch.from_numpy(d[x]).to(tdt).cuda() for x in ("q", "k", "v"))
    say(f"[no-alloc] {name}: q{tuple(q.shape)} k{tuple(k.shape)} causal={causal}")
    o_s, i_s, w_s, l_s, d_s = _static(ta, q, k, v, causal)
    o_r, ex = ta.forward(q, k, v, causal=causal, seed=0, return_coreset=True, return_decisions=True)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_r), f"{name}: outputs differ"
    assert torch.equal(l_s, ex["coreset_len"])
    for u in range(l_s.shape[0]):
        n = int(l_s[u])
        assert torch.equal(i_s[u, :n], ex["coreset_idx"][u, :n]) and torch.equal(w_s[u, :n], ex["coreset_w"][u, :n])
    assert torch.equal(d_s, ex["decisions"])
    say(f"[no-alloc] {name}: identical to thin_attn_forward")


def test_unmasked_two_calls_second_smaller():
    from sub_quadratic_attention_amd.binding import ThinAttention
    ta = ThinAttention(64, 256, 1, 1, torch.bfloat16)
    _check(ta, inputs.biggan_self_attention(seed=1, B=4), False, "biggan B=4 S=4096")
    _check(ta, inputs.biggan_self_attention(seed=2, B=1, side=32), False, "biggan B=1 S=1024")


def test_causal_two_calls_second_smaller():
    from sub_quadratic_attention_amd.binding import ThinAttention
    ta = ThinAttention(128, 128, 2, 2, torch.bfloat16, n_out=64)
    _check(ta, inputs.causal_prefill(seed=3, H=2, S=4325), True, "causal S=4325 n_out=64")
    ta2 = ThinAttention(128, 128, 2, 2, torch.bfloat16, n_out=16)
    _check(ta2, inputs.causal_prefill(seed=4, H=2, S=600), True, "causal S=600 n_out=16")


def test_sizes_beyond_the_scratch_are_refused():
    """The ViT layer (B = 64, S = 3136) needs ~80 MB of scratch: THIN_ENOMEM, nothing enqueued."""
    from sub_quadratic_attention_amd.binding import ThinAttention
    ta = ThinAttention(64, 64, 1, 1, torch.float32)
    need = ta.workspace_size(64, 3136, 3136, False)
    assert need > (64 << 20)
    fake = ctypes.c_void_p(0x1000)
    rc = ta.lib.thin_attn_forward_static(ta.h, fake, fake, fake, 64, 3136, 3136, 0, ctypes.c_uint64(0), fake,
                                         None, None, None, None, None)
    assert rc == -3 and b"static scratch" in ta.lib.thin_attn_last_error(ta.h)
