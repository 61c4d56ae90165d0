"""Thin ctypes binding of libthin_attn.so (argument marshalling only).

Every step of the path runs in the HIP library; PyTorch provides device memory
and the stream.  There is no CPU fallback: if the library is missing or the
tensors are not on a GPU, the calls raise.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libthin_attn.so")

THIN_F32, THIN_BF16, THIN_FP8_E4M3 = 0, 1, 2
THIN_GREEDY_SIGNS = 1
THIN_SUBSAMPLE_BASE = 2
THIN_ONE_STREAM = 4
THIN_FP64_GRAM = 8
_STATUS = {0: "THIN_OK", -1: "THIN_EINVAL", -2: "THIN_ENOTSUP", -3: "THIN_ENOMEM", -4: "THIN_EHIP"}


class ThinAttnError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{_STATUS.get(code, code)}: {message}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("E", ctypes.c_int32), ("D", ctypes.c_int32),
                ("H", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("g", ctypes.c_int32),
                ("n_out", ctypes.c_int32), ("delta", ctypes.c_double), ("scale", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


_lib = None

# name -> (restype, argtypes)
_SIGNATURES = {
    "thin_attn_create": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_void_p)]),
    "thin_attn_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "thin_attn_last_error": (ctypes.c_char_p, [ctypes.c_void_p]),
    "thin_attn_status": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "thin_attn_coreset_size": (ctypes.c_int64, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]),
    "thin_attn_coreset_capacity": (ctypes.c_int64, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]),
    "thin_attn_decision_count": (ctypes.c_int64, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]),
    "thin_attn_workspace_size": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.c_int64, ctypes.c_int]),
    "thin_attn_forward": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3
                          + [ctypes.c_int, ctypes.c_uint64] + [ctypes.c_void_p] * 6
                          + [ctypes.c_size_t, ctypes.c_void_p]),
    "thin_attn_forward_static": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3
                                 + [ctypes.c_int, ctypes.c_uint64] + [ctypes.c_void_p] * 5 + [ctypes.c_void_p]),
    "thin_attn_forward_subset": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 4
                                 + [ctypes.c_uint64] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]),
    "thin_attn_coreset_attention": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 3
                                    + [ctypes.c_int64] * 3 + [ctypes.c_void_p, ctypes.c_void_p,
                                                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "thin_attn_halving": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 2
                          + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
                          + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]),
    "thin_attn_halving_workspace_size": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]),
    "thin_attn_philox": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "thin_attn_kv_state_size": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]),
    "thin_attn_kv_create": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_void_p)]),
    "thin_attn_kv_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "thin_attn_kv_tokens": (ctypes.c_int64, [ctypes.c_void_p]),
    "thin_attn_kv_decision_count": (ctypes.c_int64, [ctypes.c_void_p, ctypes.c_int64]),
    "thin_attn_kv_workspace_size": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int64]),
    "thin_attn_kv_append": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int64] + [ctypes.c_void_p] * 2
                            + [ctypes.c_size_t, ctypes.c_void_p]),
    "thin_attn_kv_decode": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p]),
    "thin_attn_kv_coreset": (ctypes.c_int, [ctypes.c_void_p] * 5),
    "thin_attn_kv_export": (ctypes.c_int64, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]),
    "thin_attn_kv_import": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]),
    "thin_attn_set_timing": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "thin_attn_timing_count": (ctypes.c_int64, [ctypes.c_void_p]),
    "thin_attn_timing_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_char_p, ctypes.c_size_t,
                                             ctypes.POINTER(ctypes.c_float)]),
}


def exported_symbols():
    return sorted(_SIGNATURES)


def load_library(path=LIB_PATH):
    """Load libthin_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sub_quadratic_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dtype):
    if dtype == torch.float32:
        return THIN_F32
    if dtype == torch.bfloat16:
        return THIN_BF16
    if dtype == torch.float8_e4m3fn:
        return THIN_FP8_E4M3
    raise ValueError(f"unsupported dtype {dtype}")


def output_dtype(dtype):
    """Element type of the outputs for inputs of `dtype` (bfloat16 for FP8 inputs)."""
    return torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype


class ThinAttention:
    """Handle of the thinned attention library for one head configuration.

    forward(q [B,T,H,E], k [B,S,H_kv,E], v [B,S,H_kv,D], causal) returns the
    attention output [B,T,H,D] and, on request, each unit's coreset (token
    indices and weights) and its kernel-halving decisions.
    """

    def __init__(self, E, D, H, H_kv=None, dtype=torch.float32, g=0, n_out=0, delta=0.5, scale=0.0,
                 greedy=False, subsample_base=False, one_stream=False, fp64_gram=False):
        self.lib = load_library()
        self.E, self.D, self.H = E, D, H
        self.H_kv = H if H_kv is None else H_kv
        self.dtype = dtype
        self.out_dtype = output_dtype(dtype)
        cfg = _Config(_dtype_code(dtype), E, D, H, self.H_kv, g, n_out, delta, scale,
                      (THIN_GREEDY_SIGNS if greedy else 0) | (THIN_SUBSAMPLE_BASE if subsample_base else 0)
                      | (THIN_ONE_STREAM if one_stream else 0) | (THIN_FP64_GRAM if fp64_gram else 0))
        h = ctypes.c_void_p()
        rc = self.lib.thin_attn_create(ctypes.byref(cfg), ctypes.byref(h))
        if rc != 0:
            raise ThinAttnError(rc, self.lib.thin_attn_last_error(None).decode())
        self.h = h

    def __del__(self):
        if getattr(self, "h", None) is not None and _lib is not None:
            _lib.thin_attn_destroy(self.h)
            self.h = None

    def _check(self, rc):
        if rc != 0:
            raise ThinAttnError(rc, self.lib.thin_attn_last_error(self.h).decode())

    def status(self, stream=None):
        """Wait for the stream; raise if a call on this handle read a token index outside [0, S)."""
        self._check(self.lib.thin_attn_status(self.h, _stream(stream)))

    def _out(self, out, B, T, dev):
        """The output tensor: a new one, or the caller's, checked against [B, T, H, D] and the dtype."""
        if out is None:
            return torch.empty((B, T, self.H, self.D), dtype=self.out_dtype, device=dev)
        if tuple(out.shape) != (B, T, self.H, self.D) or out.dtype != self.out_dtype or not out.is_contiguous() \
                or out.device != dev:
            raise ValueError(f"out must be a contiguous {self.out_dtype} tensor of shape {(B, T, self.H, self.D)} on {dev}")
        return out

    # sizes --------------------------------------------------------------
    def coreset_size(self, S, causal=False):
        return int(self.lib.thin_attn_coreset_size(self.h, S, int(causal)))

    def coreset_capacity(self, S, causal=False):
        return int(self.lib.thin_attn_coreset_capacity(self.h, S, int(causal)))

    def decision_count(self, S, causal=False):
        n = int(self.lib.thin_attn_decision_count(self.h, S, int(causal)))
        if n < 0:
            self._check(n)
        return n

    def workspace_size(self, B, T, S, causal=False):
        return int(self.lib.thin_attn_workspace_size(self.h, B, T, S, int(causal)))

    def workspace(self, B, T, S, causal=False, device="cuda"):
        return torch.empty(max(self.workspace_size(B, T, S, causal), 256), dtype=torch.uint8, device=device)

    # compute ------------------------------------------------------------
    def _inputs(self, q, k, v):
        for name, t in (("q", q), ("k", k), ("v", v)):
            if not t.is_cuda:
                raise ValueError(f"{name} must be a GPU tensor")
            if t.dtype != self.dtype:
                raise ValueError(f"{name} has dtype {t.dtype}, handle expects {self.dtype}")
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        B, T, H, E = q.shape
        if H != self.H or E != self.E:
            raise ValueError("query shape does not match the handle")
        if k.shape[0] != B or k.shape[2] != self.H_kv or k.shape[3] != self.E:
            raise ValueError("key shape does not match")
        if v.shape[:3] != k.shape[:3] or v.shape[3] != self.D:
            raise ValueError("value shape does not match")
        return q, k, v

    def forward(self, q, k, v, causal=False, seed=0, return_coreset=False, return_decisions=False,
                workspace=None, out=None, stream=None):
        q, k, v = self._inputs(q, k, v)
        B, T = q.shape[:2]
        S = k.shape[1]
        units = B * self.H_kv
        dev = q.device
        out = self._out(out, B, T, dev)
        if workspace is None:
            workspace = self.workspace(B, T, S, causal, dev)
        idx = w = ln = dec = None
        if return_coreset:
            cap = self.coreset_capacity(S, causal)
            idx = torch.empty((units, cap), dtype=torch.int32, device=dev)
            w = torch.empty((units, cap), dtype=torch.float32, device=dev)
            ln = torch.empty((units,), dtype=torch.int32, device=dev)
        if return_decisions:
            dec = torch.empty((units, max(self.decision_count(S, causal), 1)), dtype=torch.uint8, device=dev)
        rc = self.lib.thin_attn_forward(self.h, _ptr(q), _ptr(k), _ptr(v), B, T, S, int(causal),
                                        ctypes.c_uint64(seed), _ptr(out), _ptr(idx), _ptr(w), _ptr(ln),
                                        _ptr(dec), _ptr(workspace), workspace.numel(), _stream(stream))
        self._check(rc)
        extra = {}
        if return_coreset:
            extra.update(coreset_idx=idx, coreset_w=w, coreset_len=ln)
        if return_decisions:
            extra["decisions"] = dec[:, :self.decision_count(S, causal)]
        return (out, extra) if extra else out

    def forward_subset(self, q, k, v, key_idx, seed=0, return_coreset=False, return_decisions=False,
                       workspace=None, out=None, stream=None):
        """Unmasked attention against the coreset of a chosen key list per unit:
        key_idx [B, H_kv, L] int32 token indices into k / v (thin_attn_forward_subset)."""
        q, k, v = self._inputs(q, k, v)
        B, T = q.shape[:2]
        S = k.shape[1]
        if key_idx.device != q.device:
            raise ValueError(f"key_idx must be on {q.device}")
        key_idx = key_idx.to(torch.int32).contiguous()
        if key_idx.dim() != 3 or key_idx.shape[:2] != (B, self.H_kv):
            raise ValueError(f"key_idx must be [B, H_kv, L] = [{B}, {self.H_kv}, L]; got {tuple(key_idx.shape)}")
        L = key_idx.shape[2]
        units = B * self.H_kv
        dev = q.device
        out = self._out(out, B, T, dev)
        if workspace is None:
            workspace = self.workspace(B, T, L, False, dev)
        idx = w = ln = dec = None
        if return_coreset:
            cap = self.coreset_capacity(L, False)
            idx = torch.empty((units, cap), dtype=torch.int32, device=dev)
            w = torch.empty((units, cap), dtype=torch.float32, device=dev)
            ln = torch.empty((units,), dtype=torch.int32, device=dev)
        if return_decisions:
            dec = torch.empty((units, max(self.decision_count(L, False), 1)), dtype=torch.uint8, device=dev)
        rc = self.lib.thin_attn_forward_subset(self.h, _ptr(q), _ptr(k), _ptr(v), _ptr(key_idx), B, T, S, L,
                                               ctypes.c_uint64(seed), _ptr(out), _ptr(idx), _ptr(w), _ptr(ln),
                                               _ptr(dec), _ptr(workspace), workspace.numel(), _stream(stream))
        self._check(rc)
        extra = {}
        if return_coreset:
            extra.update(coreset_idx=idx, coreset_w=w, coreset_len=ln)
        if return_decisions:
            extra["decisions"] = dec[:, :self.decision_count(L, False)]
        return (out, extra) if extra else out

    def coreset_attention(self, q, k, v, idx=None, w=None, out=None, stream=None):
        """Attention of every query against given per-unit coresets (idx [units, n], w [units, n])."""
        q, k, v = self._inputs(q, k, v)
        B, T = q.shape[:2]
        S = k.shape[1]
        units = B * self.H_kv
        n = S if idx is None else idx.shape[-1]
        if idx is not None:
            if idx.device != q.device or idx.numel() != units * n:
                raise ValueError(f"idx must hold [B * H_kv, n] = [{units}, n] indices on {q.device}")
            idx = idx.to(torch.int32).contiguous()
        if w is not None:
            if idx is None or w.device != q.device or w.numel() != units * n:
                raise ValueError(f"w needs idx and must hold [B * H_kv, n] = [{units}, {n}] weights on {q.device}")
            w = w.to(torch.float32).contiguous()
        out = self._out(out, B, T, q.device)
        rc = self.lib.thin_attn_coreset_attention(self.h, _ptr(q), _ptr(k), _ptr(v), B, T, S, _ptr(idx), _ptr(w),
                                                  n, _ptr(out), _stream(stream))
        self._check(rc)
        return out

    def halving(self, k, v, points, seed=0, tag=0, bin_id=0, stream=None, workspace=True):
        """One kernel halving per unit on points [units, N]; returns (kept, decisions, gram).
        workspace=False runs the fp64 Gram (no integer-Gram scratch)."""
        if not (k.is_cuda and v.is_cuda) or k.dtype != self.dtype or v.dtype != self.dtype:
            raise ValueError("k and v must be GPU tensors of the handle dtype")
        k, v = k.contiguous(), v.contiguous()
        B, S = k.shape[:2]
        points = points.to(torch.int32).contiguous()
        units, N = points.shape
        P = N // 2
        kept = torch.empty((units, P), dtype=torch.int32, device=k.device)
        dec = torch.empty((units, P), dtype=torch.uint8, device=k.device)
        gram = torch.zeros((units, P, P), dtype=torch.float64, device=k.device)
        nws = int(self.lib.thin_attn_halving_workspace_size(self.h, B, N)) if workspace else 0
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=k.device)
        rc = self.lib.thin_attn_halving(self.h, _ptr(k), _ptr(v), B, S, _ptr(points), N, ctypes.c_uint64(seed),
                                        tag, ctypes.c_uint64(bin_id), _ptr(kept), _ptr(dec), _ptr(gram),
                                        _ptr(ws) if nws else None, nws, _stream(stream))
        self._check(rc)
        return kept, dec, gram

    def set_timing(self, enable=True):
        self._check(self.lib.thin_attn_set_timing(self.h, int(enable)))

    def timing_records(self):
        """[(kernel label, milliseconds)] of every launch since set_timing(True) (waits for them)."""
        out = []
        buf = ctypes.create_string_buffer(64)
        ms = ctypes.c_float()
        for i in range(int(self.lib.thin_attn_timing_count(self.h))):
            self._check(self.lib.thin_attn_timing_read(self.h, i, buf, 64, ctypes.byref(ms)))
            out.append((buf.value.decode(), ms.value))
        return out


def philox(counters, seed, stream=None):
    """Philox4x64-10 blocks for counters [n, 4] (int64 GPU tensor holding uint64 words)."""
    lib = load_library()
    counters = counters.contiguous()
    out = torch.empty_like(counters)
    rc = lib.thin_attn_philox(_ptr(counters), counters.shape[0], ctypes.c_uint64(seed), _ptr(out), _stream(stream))
    if rc != 0:
        raise ThinAttnError(rc, "philox launch failed")
    return out


class KVState:
    """Streaming Express state for decoding, backed by a caller-owned device buffer.

    append(k [B, n, H_kv, E], v) streams tokens in; decode(q [B, H, E],
    k1 [B, H_kv, E], v1) appends one token and returns its attention output
    [B, H, D].  Both can return the halving decisions they made.
    """

    def __init__(self, attn, B, n_out, seed=0, device="cuda"):
        self.attn = attn
        self.lib = attn.lib
        self.B = B
        self.n_out = n_out
        nbytes = int(self.lib.thin_attn_kv_state_size(attn.h, B, n_out))
        if nbytes == 0:
            raise ValueError("invalid state size arguments")
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        attn._check(self.lib.thin_attn_kv_create(attn.h, _ptr(self.buffer), nbytes, B, n_out, ctypes.c_uint64(seed),
                                                 ctypes.byref(h)))
        self.kv = h
        self._ws = None

    def __del__(self):
        if getattr(self, "kv", None) is not None and _lib is not None:
            _lib.thin_attn_kv_destroy(self.kv)
            self.kv = None

    @property
    def tokens(self):
        return int(self.lib.thin_attn_kv_tokens(self.kv))

    def decision_count(self, n_new):
        n = int(self.lib.thin_attn_kv_decision_count(self.kv, n_new))
        if n < 0:
            self.attn._check(n)
        return n

    def _workspace(self, n_new):
        need = max(int(self.lib.thin_attn_kv_workspace_size(self.kv, n_new)), 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.buffer.device)
        return self._ws

    def _decisions(self, n_new, want):
        if not want:
            return None
        return torch.zeros((self.B * self.attn.H_kv, max(self.decision_count(n_new), 1)), dtype=torch.uint8,
                           device=self.buffer.device)

    def append(self, k, v, return_decisions=False, stream=None):
        k, v = k.contiguous(), v.contiguous()
        n_new = k.shape[1]
        dec = self._decisions(n_new, return_decisions)
        cnt = self.decision_count(n_new) if return_decisions else 0
        ws = self._workspace(n_new)
        self.attn._check(self.lib.thin_attn_kv_append(self.kv, _ptr(k), _ptr(v), n_new, _ptr(dec), _ptr(ws),
                                                      ws.numel(), _stream(stream)))
        return dec[:, :cnt] if return_decisions else None

    def decode(self, q, k1, v1, out=None, return_decisions=False, stream=None):
        q, k1, v1 = q.contiguous(), k1.contiguous(), v1.contiguous()
        if out is None:
            out = torch.empty((self.B, self.attn.H, self.attn.D), dtype=self.attn.out_dtype, device=q.device)
        dec = self._decisions(1, return_decisions)
        cnt = self.decision_count(1) if return_decisions else 0
        ws = self._workspace(1)
        self.attn._check(self.lib.thin_attn_kv_decode(self.kv, _ptr(q), _ptr(k1), _ptr(v1), _ptr(out), _ptr(dec),
                                                      _ptr(ws), ws.numel(), _stream(stream)))
        return (out, dec[:, :cnt]) if return_decisions else out

    def coreset(self, stream=None):
        units = self.B * self.attn.H_kv
        cap = 7 * self.n_out
        idx = torch.empty((units, cap), dtype=torch.int32, device=self.buffer.device)
        w = torch.empty((units, cap), dtype=torch.float32, device=self.buffer.device)
        ln = torch.empty((units,), dtype=torch.int32, device=self.buffer.device)
        self.attn._check(self.lib.thin_attn_kv_coreset(self.kv, _ptr(idx), _ptr(w), _ptr(ln), _stream(stream)))
        return idx, w, ln

    def export_meta(self):
        n = int(self.lib.thin_attn_kv_export(self.kv, None, 0))
        buf = ctypes.create_string_buffer(n)
        self.attn._check(0 if self.lib.thin_attn_kv_export(self.kv, buf, n) == n else -1)
        return bytes(buf.raw)

    def import_meta(self, meta):
        buf = ctypes.create_string_buffer(meta, len(meta))
        self.attn._check(self.lib.thin_attn_kv_import(self.kv, buf, len(meta)))
