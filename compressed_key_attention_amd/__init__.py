"""Python binding of libtq (include/tq.h): argument marshalling only.

Every step of compression, decode attention, sign indexing, top-k selection and the bulk
scan runs in the HIP kernels of ``libtq.so``; this module converts torch tensors to device
pointers, picks the caller's current HIP stream, allocates workspaces with torch, and
raises ``TqError`` on any non-OK status.  Importing it fails loudly when the library has
not been built (``python -m compressed_key_attention_amd._build``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libtq.so is not built at {LIB_PATH}; run "
                      "`python -m compressed_key_attention_amd._build` first")

_lib = ctypes.CDLL(LIB_PATH)

TQ_OK, TQ_ERR_INVALID_ARGUMENT, TQ_ERR_UNSUPPORTED = 0, 1, 2
TQ_ERR_WORKSPACE_TOO_SMALL, TQ_ERR_OUT_OF_MEMORY, TQ_ERR_DEVICE = 3, 4, 5
TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2

EXPORTED = [
    "tq_last_error", "tq_create", "tq_destroy", "tq_host_constants", "tq_record_bytes",
    "tq_compress_kv", "tq_debug_quantize", "tq_decode_workspace_size", "tq_decode_attention",
    "tq_index_workspace_size", "tq_build_sign_index", "tq_select_workspace_size",
    "tq_select_topk", "tq_scan_workspace_size", "tq_score_scan", "tq_set_profile_events",
    "tq_stream_read", "tq_monarch_workspace_size", "tq_monarch_step", "tq_sparse_workspace_size",
    "tq_sparse_attention", "tq_polar_host_constants", "tq_decode_attention_noalloc",
]
TQ_KEY_SCALAR, TQ_KEY_POLAR = 0, 1


class TqConfig(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("key_bits", ctypes.c_int32),
                ("qjl_dim", ctypes.c_int32), ("value_bits", ctypes.c_int32),
                ("rotation_seed", ctypes.c_uint64), ("qjl_seed", ctypes.c_uint64),
                ("key_codec", ctypes.c_int32), ("polar_upper_bits", ctypes.c_int32)]


class MonarchConfig(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("cold_gate", ctypes.c_float),
                ("promote_weight", ctypes.c_float), ("promote_steps", ctypes.c_int32)]


class MonarchState(ctypes.Structure):
    _fields_ = [("hot_k", ctypes.c_void_p), ("hot_v", ctypes.c_void_p), ("hot_dt", ctypes.c_int),
                ("hot_capacity", ctypes.c_int64), ("hot_start", ctypes.c_void_p),
                ("hot_len", ctypes.c_void_p), ("records", ctypes.c_void_p),
                ("cold_capacity", ctypes.c_int64), ("cold_len", ctypes.c_void_p),
                ("hits", ctypes.c_void_p), ("overflow", ctypes.c_void_p)]


class TqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"tq status {status}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_I32, _I64, _SZ, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_PSZ = ctypes.POINTER(ctypes.c_size_t)


def _sig(name, *argtypes):
    f = getattr(_lib, name)
    f.argtypes = list(argtypes)
    f.restype = ctypes.c_int
    return f


_lib.tq_last_error.restype = ctypes.c_char_p
_lib.tq_last_error.argtypes = []
_create = _sig("tq_create", ctypes.POINTER(TqConfig), ctypes.POINTER(_P))
_destroy = _sig("tq_destroy", _P)
_host_constants = _sig("tq_host_constants", ctypes.POINTER(TqConfig), _P, _P, _P, _P, _P, _P)
_polar_host_constants = _sig("tq_polar_host_constants", ctypes.POINTER(TqConfig), _P, _P)
_record_bytes = _sig("tq_record_bytes", _P, _PSZ, _PSZ)
_compress = _sig("tq_compress_kv", _P, _P, _P, ctypes.c_int, _I32, _I64, _I32, _I64, _I64, _I64,
                 _P, _I64, _I64, _P)
_debug_quantize = _sig("tq_debug_quantize", _P, _P, _P, _P, _P, _P, _P, _I64, _P, _P)
_decode_ws = _sig("tq_decode_workspace_size", _P, _I32, _I32, _I32, _I64, _I32, _PSZ)
_decode = _sig("tq_decode_attention", _P, _P, ctypes.c_int, _I32, _I32, _I32, _P, _I64, _P, _P, _P,
               ctypes.c_int, _P, _I64, _P, _I32, _F, _P, _P, _P, _P, _SZ, _P)
_decode_noalloc = _sig("tq_decode_attention_noalloc", _P, _P, ctypes.c_int, _I32, _I32, _I32, _P, _I64, _P, _P,
                       _P, ctypes.c_int, _P, _I64, _P, _I32, _F, _P, _P, _P, _P)
_index_ws = _sig("tq_index_workspace_size", _P, _I32, _I32, _PSZ)
_index = _sig("tq_build_sign_index", _P, _P, ctypes.c_int, _I32, _I64, _I32, _I64, _I64, _I64, _P,
              _P, _P, _I64, _I64, _P, _SZ, _P)
_select_ws = _sig("tq_select_workspace_size", _P, _I32, _I32, _I64, _PSZ)
_select = _sig("tq_select_topk", _P, _P, ctypes.c_int, _I32, _I32, _I32, _P, _P, _I64, _P, _I32,
               _P, _P, _P, _P, _SZ, _P)
_sparse_ws = _sig("tq_sparse_workspace_size", _P, _I32, _I32, _I32, _I64, _PSZ)
_sparse = _sig("tq_sparse_attention", _P, _P, ctypes.c_int, _I32, _I32, _I32, _P, _P, _P, _I64, _P, _I32,
               _P, _P, ctypes.c_int, _P, _I64, _F, _P, _P, _P, _SZ, _P)
_scan_ws = _sig("tq_scan_workspace_size", _P, _I32, _I32, _I32, _PSZ)
_scan = _sig("tq_score_scan", _P, _P, ctypes.c_int, _I32, _I32, _I32, _P, _I64, _I64, _P, _P, _SZ, _P)
_set_events = _sig("tq_set_profile_events", _P, _P)
_stream_read = _sig("tq_stream_read", _P, _SZ, _P, _SZ, _P)
_monarch_ws = _sig("tq_monarch_workspace_size", _P, _I32, _I32, _I32, _I64, _I64, _PSZ)
_monarch_step = _sig("tq_monarch_step", _P, ctypes.POINTER(MonarchConfig), ctypes.POINTER(MonarchState), _P,
                     ctypes.c_int, _I32, _I32, _I32, _P, _P, _F, _P, _P, _P, _P, _SZ, _P)


def set_profile_events(start, stop):
    """Arm raw hipEvent_t handles (ints) around the main kernel of the next call on this thread."""
    check(_set_events(_P(start) if start else None, _P(stop) if stop else None))


def stream_read(buf, sink, stream=None):
    """Enqueue the library's streaming read of `buf` (a 16-byte aligned device tensor) into
    `sink` (device uint32 tensor) - measurement support for the bench's read ceiling."""
    check(_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink.numel(), _stream(stream)))


def last_error() -> str:
    return _lib.tq_last_error().decode()


def check(status: int):
    if status != TQ_OK:
        raise TqError(status, last_error())


def _config(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed, polar_upper_bits=0) -> TqConfig:
    """polar_upper_bits > 0 selects the polar key codec (key_bits = level-1 angle bits)."""
    codec = TQ_KEY_POLAR if polar_upper_bits else TQ_KEY_SCALAR
    return TqConfig(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed, codec,
                    polar_upper_bits)


def polar_host_constants(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed,
                         polar_upper_bits):
    """The polar angle grids computed on the host (no GPU): levels, bounds [L][16]."""
    cfg = _config(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed, polar_upper_bits)
    L = head_dim.bit_length() - 1
    lv = np.full((L, 16), np.nan, np.float32)
    bd = np.full((L, 16), np.nan, np.float32)
    check(_polar_host_constants(ctypes.byref(cfg), lv.ctypes.data_as(_P), bd.ctypes.data_as(_P)))
    return lv, bd


def host_constants(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed):
    """The handle constants computed on the host (no GPU): Pi, S and the codebooks."""
    cfg = _config(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed)
    pi = np.zeros((head_dim, head_dim), np.float32)
    s = np.zeros((max(qjl_dim, 1), head_dim), np.float32)
    kl = np.zeros(1 << key_bits, np.float32)
    kb = np.zeros((1 << key_bits) - 1, np.float32)
    vl = np.zeros(1 << value_bits, np.float32)
    vb = np.zeros((1 << value_bits) - 1, np.float32)
    ptr = lambda a: a.ctypes.data_as(_P)
    check(_host_constants(ctypes.byref(cfg), ptr(pi), ptr(s), ptr(kl), ptr(kb), ptr(vl), ptr(vb)))
    return dict(pi=pi, s=s[:qjl_dim], key_levels=kl, key_bounds=kb, val_levels=vl, val_bounds=vb)


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: TQ_F32, torch.float16: TQ_F16, torch.bfloat16: TQ_BF16}[t.dtype]


def _ptr(t):
    return None if t is None else _P(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return _P(s.cuda_stream)


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Handle:
    """A tq_handle: the seeded rotation, QJL matrix and codebooks on the current device."""

    def __init__(self, head_dim=128, key_bits=3, qjl_dim=128, value_bits=4,
                 rotation_seed=1, qjl_seed=2, polar_upper_bits=0):
        self.head_dim, self.key_bits, self.qjl_dim, self.value_bits = head_dim, key_bits, qjl_dim, value_bits
        self.rotation_seed, self.qjl_seed = rotation_seed, qjl_seed
        self.polar_upper_bits = polar_upper_bits
        cfg = _config(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed, polar_upper_bits)
        h = _P()
        check(_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h
        rb, ib = ctypes.c_size_t(), ctypes.c_size_t()
        check(_record_bytes(self._h, ctypes.byref(rb), ctypes.byref(ib)))
        self.record_bytes, self.index_record_bytes = rb.value, ib.value

    def close(self):
        if getattr(self, "_h", None):
            check(_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---------------------------------------------------------------- compress ---------
    def new_cache(self, batch, kv_heads, capacity, device="cuda"):
        import torch
        return torch.zeros((batch, kv_heads, capacity, self.record_bytes), dtype=torch.uint8, device=device)

    def compress_kv(self, k, v, records, first_slot=0, stream=None):
        """k, v: [batch, tokens, kv_heads, head_dim] views with a contiguous last dim."""
        assert k.shape == v.shape and k.stride() == v.stride() and k.dtype == v.dtype
        B, T, H, d = k.shape
        check(_compress(self._h, _ptr(k), _ptr(v), _dtype_code(k), B, T, H, k.stride(0), k.stride(1),
                        k.stride(2), _ptr(records), records.shape[2], first_slot, _stream(stream)))
        return records

    def debug_quantize(self, z_k, p, r_k, rho, z_v, r_v, records, stream=None):
        check(_debug_quantize(self._h, _ptr(z_k), _ptr(p), _ptr(r_k), _ptr(rho), _ptr(z_v), _ptr(r_v),
                              z_k.shape[0], _ptr(records), _stream(stream)))
        return records

    # ---------------------------------------------------------------- decode -----------
    def decode_workspace_size(self, batch, q_heads, kv_heads, capacity, k_sel=0) -> int:
        n = ctypes.c_size_t()
        check(_decode_ws(self._h, batch, q_heads, kv_heads, capacity, k_sel, ctypes.byref(n)))
        return n.value

    def decode_attention(self, q, records, seq_lens, hot_k=None, hot_v=None, hot_lens=None,
                         sel_idx=None, scale=0.0, out=None, lse=None, logits=None, workspace=None,
                         stream=None):
        """q [batch, q_heads, d]; records [batch, kv_heads, capacity, R]; seq_lens int32 [batch].
        Returns out [batch, q_heads, d] float32 (and fills lse / logits when given)."""
        import torch
        B, Hq, d = q.shape
        Hkv, cap = records.shape[1], records.shape[2]
        k_sel = 0 if sel_idx is None else sel_idx.shape[-1]
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = _workspace(self.decode_workspace_size(B, Hq, Hkv, cap, k_sel), q.device)
        hot_cap = 0 if hot_k is None else hot_k.shape[2]
        hot_dt = TQ_F32 if hot_k is None else _dtype_code(hot_k)
        check(_decode(self._h, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(records), cap, _ptr(seq_lens),
                      _ptr(hot_k), _ptr(hot_v), hot_dt, _ptr(hot_lens), hot_cap, _ptr(sel_idx), k_sel,
                      float(scale), _ptr(out), _ptr(lse), _ptr(logits), _ptr(workspace),
                      workspace.numel(), _stream(stream)))
        return out

    def decode_attention_noalloc(self, q, records, seq_lens, out, hot_k=None, hot_v=None, hot_lens=None,
                                 sel_idx=None, scale=0.0, lse=None, logits=None, stream=None):
        """tq_decode_attention_noalloc: decode_attention with the library's fixed device scratch
        instead of a workspace (nothing is allocated; `out` must be given).  Returns out."""
        B, Hq, d = q.shape
        Hkv, cap = records.shape[1], records.shape[2]
        k_sel = 0 if sel_idx is None else sel_idx.shape[-1]
        hot_cap = 0 if hot_k is None else hot_k.shape[2]
        hot_dt = TQ_F32 if hot_k is None else _dtype_code(hot_k)
        check(_decode_noalloc(self._h, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(records), cap, _ptr(seq_lens),
                              _ptr(hot_k), _ptr(hot_v), hot_dt, _ptr(hot_lens), hot_cap, _ptr(sel_idx), k_sel,
                              float(scale), _ptr(out), _ptr(lse), _ptr(logits), _stream(stream)))
        return out

    # ---------------------------------------------------------------- sign index / top-k
    def index_workspace_size(self, batch, kv_heads) -> int:
        n = ctypes.c_size_t()
        check(_index_ws(self._h, batch, kv_heads, ctypes.byref(n)))
        return n.value

    def build_sign_index(self, k, index, codebook, mean=None, first_slot=0, workspace=None, stream=None):
        B, T, H, d = k.shape
        if workspace is None:
            workspace = _workspace(self.index_workspace_size(B, H), k.device)
        check(_index(self._h, _ptr(k), _dtype_code(k), B, T, H, k.stride(0), k.stride(1), k.stride(2),
                     _ptr(index), _ptr(codebook), _ptr(mean), index.shape[2], first_slot,
                     _ptr(workspace), workspace.numel(), _stream(stream)))

    def select_workspace_size(self, batch, kv_heads, capacity) -> int:
        n = ctypes.c_size_t()
        check(_select_ws(self._h, batch, kv_heads, capacity, ctypes.byref(n)))
        return n.value

    def select_topk(self, q, index, codebook, seq_lens, k, out_idx=None, out_count=None,
                    out_scores=None, workspace=None, stream=None):
        import torch
        B, Hq, d = q.shape
        H, cap = index.shape[1], index.shape[2]
        if out_idx is None:
            out_idx = torch.empty((B, H, k), dtype=torch.int32, device=q.device)
        if out_count is None:
            out_count = torch.empty((B, H), dtype=torch.int32, device=q.device)
        if workspace is None:
            workspace = _workspace(self.select_workspace_size(B, H, cap), q.device)
        check(_select(self._h, _ptr(q), _dtype_code(q), B, Hq, H, _ptr(index), _ptr(codebook), cap,
                      _ptr(seq_lens), k, _ptr(out_idx), _ptr(out_count), _ptr(out_scores),
                      _ptr(workspace), workspace.numel(), _stream(stream)))
        return out_idx, out_count

    # ---------------------------------------------------------------- sparse attention -
    def sparse_workspace_size(self, batch, q_heads, kv_heads, capacity) -> int:
        n = ctypes.c_size_t()
        check(_sparse_ws(self._h, batch, q_heads, kv_heads, capacity, ctypes.byref(n)))
        return n.value

    def sparse_attention(self, q, index, codebook, records, seq_lens, k, hot_k=None, hot_v=None,
                         hot_lens=None, scale=0.0, out=None, lse=None, workspace=None, stream=None):
        """Top-k selection from the sign index and attention over the selected compressed
        tokens (plus an optional exact segment) in one call; q [batch, q_heads, d]."""
        import torch
        B, Hq, d = q.shape
        Hkv, cap = records.shape[1], records.shape[2]
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = _workspace(self.sparse_workspace_size(B, Hq, Hkv, cap), q.device)
        hot_cap = 0 if hot_k is None else hot_k.shape[2]
        hot_dt = TQ_F32 if hot_k is None else _dtype_code(hot_k)
        check(_sparse(self._h, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(index), _ptr(codebook),
                      _ptr(records), cap, _ptr(seq_lens), k, _ptr(hot_k), _ptr(hot_v), hot_dt,
                      _ptr(hot_lens), hot_cap, scale, _ptr(out), _ptr(lse), _ptr(workspace),
                      workspace.numel(), _stream(stream)))
        return out

    # ---------------------------------------------------------------- bulk scan --------
    def scan_workspace_size(self, batch, kv_heads, n_queries) -> int:
        n = ctypes.c_size_t()
        check(_scan_ws(self._h, batch, kv_heads, n_queries, ctypes.byref(n)))
        return n.value

    def score_scan(self, q, records, n_tokens, scores=None, workspace=None, stream=None):
        """q [batch, kv_heads, n_queries, d] -> scores [batch, kv_heads, n_queries, n_tokens]."""
        import torch
        B, H, nq, d = q.shape
        if scores is None:
            scores = torch.empty((B, H, nq, n_tokens), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = _workspace(self.scan_workspace_size(B, H, nq), q.device)
        check(_scan(self._h, _ptr(q), _dtype_code(q), B, H, nq, _ptr(records), records.shape[2], n_tokens,
                    _ptr(scores), _ptr(workspace), workspace.numel(), _stream(stream)))
        return scores


class HotCold:
    """Device state of the hot/cold step: the exact ring and the compressed cold region of
    every sequence (tensors owned here, laid out as tq_monarch_state describes)."""

    def __init__(self, handle, batch, kv_heads, hot_capacity, cold_capacity, dtype, device="cuda"):
        import torch
        d = handle.head_dim
        self.hot_k = torch.zeros((batch, kv_heads, hot_capacity, d), dtype=dtype, device=device)
        self.hot_v = torch.zeros_like(self.hot_k)
        self.hot_start = torch.zeros((batch,), dtype=torch.int32, device=device)
        self.hot_len = torch.zeros((batch,), dtype=torch.int32, device=device)
        self.records = handle.new_cache(batch, kv_heads, cold_capacity, device)
        self.cold_len = torch.zeros((batch,), dtype=torch.int32, device=device)
        self.hits = torch.zeros((batch, max(cold_capacity, 1)), dtype=torch.int32, device=device)
        self.overflow = torch.zeros((batch,), dtype=torch.int32, device=device)

    def c_state(self):
        return MonarchState(self.hot_k.data_ptr(), self.hot_v.data_ptr(), _dtype_code(self.hot_k),
                            self.hot_k.shape[2], self.hot_start.data_ptr(), self.hot_len.data_ptr(),
                            self.records.data_ptr(), self.records.shape[2], self.cold_len.data_ptr(),
                            self.hits.data_ptr(), self.overflow.data_ptr())


def monarch_workspace_size(h, batch, q_heads, kv_heads, hot_cap, cold_cap) -> int:
    """Workspace bytes tq_monarch_step needs for these shapes."""
    n = ctypes.c_size_t()
    check(_monarch_ws(h._h, batch, q_heads, kv_heads, hot_cap, cold_cap, ctypes.byref(n)))
    return n.value


def monarch_step(h, state, q, k_new, v_new, window, cold_gate=float("inf"), promote_weight=0.15,
                 promote_steps=3, scale=0.0, out=None, lse=None, gate_out=None, workspace=None, stream=None):
    """One hot/cold decode step (tq_monarch_step) on `state` (a HotCold); q [batch, q_heads, d],
    k_new / v_new [batch, kv_heads, d] in the state's hot dtype.  Returns out [batch, q_heads, d]."""
    import torch
    B, Hq, d = q.shape
    Hkv = k_new.shape[1]
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(monarch_workspace_size(h, B, Hq, Hkv, state.hot_k.shape[2], state.records.shape[2]),
                               q.device)
    cfg = MonarchConfig(window, cold_gate, promote_weight, promote_steps)
    st = state.c_state()
    check(_monarch_step(h._h, ctypes.byref(cfg), ctypes.byref(st), _ptr(q), _dtype_code(q), B, Hq, Hkv,
                        _ptr(k_new), _ptr(v_new), scale, _ptr(out), _ptr(lse), _ptr(gate_out), _ptr(workspace),
                        workspace.numel(), _stream(stream)))
    return out

