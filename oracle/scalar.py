"""ctypes glue for the scalar C oracle (oracle/tq_scalar.c).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use it.  This
module does argument marshalling and the loops over sequences and heads; every step of the
arithmetic runs in the C library.  It imports nothing from the product package.

The library is built in place with gcc (``build()``); loading builds it first when it is
missing.  The definitions it follows are listed at the top of tq_scalar.c (TurboQuant page,
"Funktionsweise von TurboQuant" and "QJL"; Self-Indexing page, "Methodologie"; Monarch v3
page, "Wie es funktioniert").
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "tq_scalar.c")
LIBRARY = os.path.join(HERE, "libtq_scalar.so")
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]

_lib = None


def build() -> str:
    """Compile tq_scalar.c into oracle/libtq_scalar.so (always recompiles)."""
    tmp = LIBRARY + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SOURCE, "-lm"], check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        _lib = _declare(C.CDLL(LIBRARY))
    return _lib


_P = C.c_void_p
_I64, _I32, _U64, _D = C.c_int64, C.c_int, C.c_uint64, C.c_double


def _declare(L):
    sig = {
        "sc_splitmix64": (None, [_U64, _I64, _P]),
        "sc_gaussians": (None, [_U64, _I64, _P]),
        "sc_rotation": (_I32, [_U64, _I32, _P]),
        "sc_qjl_matrix": (None, [_U64, _I32, _I32, _P]),
        "sc_lloyd_max": (_I32, [_I32, _P, _P]),
        "sc_codec_new": (_P, [_I32, _I32, _I32, _I32, _U64, _U64]),
        "sc_codec_free": (None, [_P]),
        "sc_record_bytes": (_I32, [_P]),
        "sc_codec_tables": (None, [_P, _P, _P, _P, _P, _P, _P]),
        "sc_unpack_record": (None, [_P, _P, _P, _P, _P, _P]),
        "sc_compress": (_I32, [_P, _P, _P, _I64, _P]),
        "sc_rotated": (_I32, [_P, _P, _I32, _I64, _P, _P]),
        "sc_residual": (_I32, [_P, _P, _P, _P, _I64, _P, _P]),
        "sc_quantize_from_rotated": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I64, _P]),
        "sc_decode_head": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _I64, _D, _P, _P, _P]),
        "sc_score_scan": (_I32, [_P, _P, _I64, _P, _I64, _P]),
        "sc_channel_mean": (None, [_I32, _P, _I64, _P]),
        "sc_sign_index": (None, [_I32, _P, _I64, _P, _P, _P]),
        "sc_lut_scale_exponent": (_I32, [_D, _I32]),
        "sc_select_topk": (_I32, [_I32, _I32, _P, _P, _P, _I64, _I32, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, np.float32))


# ---------------------------------------------------------------------------------------
# Init
# ---------------------------------------------------------------------------------------
def splitmix64(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.uint64)
    lib().sc_splitmix64(seed, n, _ptr(out))
    return out


def gaussians(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.float64)
    lib().sc_gaussians(seed, n, _ptr(out))
    return out


def rotation(seed: int, d: int) -> np.ndarray:
    out = np.zeros((d, d), np.float32)
    if lib().sc_rotation(seed, d, _ptr(out)):
        raise MemoryError("sc_rotation")
    return out


def qjl_matrix(seed: int, m: int, d: int) -> np.ndarray:
    out = np.zeros((m, d), np.float32)
    lib().sc_qjl_matrix(seed, m, d, _ptr(out))
    return out


def lloyd_max(bits: int):
    lev = np.zeros(1 << bits)
    bnd = np.zeros(max(1, (1 << bits) - 1))
    lib().sc_lloyd_max(bits, _ptr(lev), _ptr(bnd))
    return lev, bnd[: (1 << bits) - 1]


def lut_scale_exponent(maxabs: float, n_terms: int) -> int:
    return int(lib().sc_lut_scale_exponent(float(maxabs), int(n_terms)))


# ---------------------------------------------------------------------------------------
# Codec
# ---------------------------------------------------------------------------------------
class ScalarCodec:
    """One configuration of the scalar oracle: Pi, S and the two codebooks live in C."""

    def __init__(self, head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed):
        self.head_dim, self.key_bits, self.qjl_dim, self.value_bits = head_dim, key_bits, qjl_dim, value_bits
        self._L = lib()
        self._c = self._L.sc_codec_new(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed)
        if not self._c:
            raise ValueError("scalar oracle: unsupported configuration")
        self.record_bytes = int(self._L.sc_record_bytes(self._c))

    def __del__(self):
        c, self._c = getattr(self, "_c", None), None
        if c:
            self._L.sc_codec_free(c)

    def tables(self) -> dict:
        d, m = self.head_dim, self.qjl_dim
        Pi = np.zeros((d, d), np.float32)
        S = np.zeros((max(m, 1), d), np.float32)
        kl, kt = np.zeros(16, np.float32), np.zeros(16, np.float32)
        vl, vt = np.zeros(16, np.float32), np.zeros(16, np.float32)
        self._L.sc_codec_tables(self._c, _ptr(Pi), _ptr(S), _ptr(kl), _ptr(kt), _ptr(vl), _ptr(vt))
        Lk, Lv = 1 << self.key_bits, 1 << self.value_bits
        return dict(Pi=Pi, S=S[:m], key_levels=kl[:Lk], key_bounds=kt[:Lk - 1],
                    val_levels=vl[:Lv], val_bounds=vt[:Lv - 1])

    # compression -----------------------------------------------------------------------
    def compress(self, k, v) -> np.ndarray:
        """k, v [n, d] -> records [n, record_bytes]."""
        k, v = _f32(k), _f32(v)
        n = k.shape[0]
        out = np.zeros((n, self.record_bytes), np.uint8)
        if self._L.sc_compress(self._c, _ptr(k), _ptr(v), n, _ptr(out)):
            raise MemoryError("sc_compress")
        return out

    def compress_cache(self, K, V, capacity=None) -> np.ndarray:
        """K, V [B, T, Hkv, d] -> records [B, Hkv, capacity, R] (slots >= T zero)."""
        B, T, H, d = K.shape
        cap = T if capacity is None else capacity
        out = np.zeros((B, H, cap, self.record_bytes), np.uint8)
        for b in range(B):
            for h in range(H):
                out[b, h, :T] = self.compress(K[b, :, h], V[b, :, h])
        return out

    def rotated(self, x, is_value=False):
        """Step 1's intermediates for x [n, d]: (z [n, d] float32 coordinates that are coded,
        r [n] float64 norms)."""
        x = _f32(x)
        n = x.shape[0]
        z = np.zeros((n, self.head_dim), np.float32)
        r = np.zeros(n)
        if self._L.sc_rotated(self._c, _ptr(x), int(bool(is_value)), n, _ptr(z), _ptr(r)):
            raise MemoryError("sc_rotated")
        return z, r

    def residual(self, k, kc, r_k):
        """Step 2 from given key codes kc [n, d] and stored norms r_k [n]: (rho [n], p [n, m])."""
        k = _f32(k)
        n = k.shape[0]
        kc = np.ascontiguousarray(kc, np.int32)
        rho, p = np.zeros(n), np.zeros((n, max(self.qjl_dim, 1)))
        if self._L.sc_residual(self._c, _ptr(k), _ptr(kc), _ptr(_f32(r_k)), n, _ptr(rho), _ptr(p)):
            raise MemoryError("sc_residual")
        return rho, p[:, :self.qjl_dim]

    def quantize_from_rotated(self, z_k, p, r_k, rho, z_v, r_v) -> np.ndarray:
        z_k, z_v = _f32(z_k), _f32(z_v)
        n = z_k.shape[0]
        p = _f32(p).reshape(n, self.qjl_dim)
        out = np.zeros((n, self.record_bytes), np.uint8)
        if self._L.sc_quantize_from_rotated(self._c, _ptr(z_k), _ptr(p), _ptr(_f32(r_k)), _ptr(_f32(rho)),
                                            _ptr(z_v), _ptr(_f32(r_v)), n, _ptr(out)):
            raise MemoryError("sc_quantize_from_rotated")
        return out

    def unpack(self, rec) -> dict:
        """records [n, R] -> fields (kc, bits, vc int64; r_k, rho, r_v float32)."""
        rec = np.ascontiguousarray(rec, np.uint8).reshape(-1, self.record_bytes)
        n, d, m = rec.shape[0], self.head_dim, self.qjl_dim
        kc, vc = np.zeros((n, d), np.int32), np.zeros((n, d), np.int32)
        bits, norms = np.zeros((n, max(m, 1)), np.int32), np.zeros((n, 3), np.float32)
        for t in range(n):
            self._L.sc_unpack_record(self._c, _ptr(rec[t]), _ptr(kc[t]), _ptr(bits[t]), _ptr(vc[t]), _ptr(norms[t]))
        return dict(kc=kc.astype(np.int64), bits=bits[:, :m].astype(np.int64), vc=vc.astype(np.int64),
                    r_k=norms[:, 0], rho=norms[:, 1], r_v=norms[:, 2])

    # attention ------------------------------------------------------------------------
    def decode_head(self, q, records, n, idx=None, hot_k=None, hot_v=None, scale=0.0, want_logits=False):
        """One query head [d] over one KV head's records [cap, R]: (out [d], lse, logits)."""
        d = self.head_dim
        q = _f32(q)
        records = np.ascontiguousarray(records, np.uint8)
        idx = None if idx is None else np.ascontiguousarray(idx, np.int32)
        nh = 0 if hot_k is None else int(hot_k.shape[0])
        hk = _f32(hot_k) if nh else None
        hv = _f32(hot_v) if nh else None
        out = np.zeros(d)
        lse = np.zeros(1)
        lg = np.zeros(n + nh) if want_logits else None
        if self._L.sc_decode_head(self._c, _ptr(q), _ptr(records), _ptr(idx), n, _ptr(hk), _ptr(hv), nh,
                                  float(scale or 0.0), _ptr(out), _ptr(lse), _ptr(lg)):
            raise MemoryError("sc_decode_head")
        return out, float(lse[0]), lg

    def decode_attention(self, q, records, seq_lens, hot_k=None, hot_v=None, hot_lens=None, sel_idx=None,
                         scale=None, heads=None, want_logits=True):
        """q [B, Hq, d] over records [B, Hkv, cap, R]; the same contract as the numpy oracle's
        decode_attention: out [B, Hq, d], lse [B, Hq], logits {(b, h): (cold, hot)}."""
        q = np.asarray(q)
        B, Hq, d = q.shape
        Hkv = records.shape[1]
        G = Hq // Hkv
        out = np.zeros((B, Hq, d))
        lse = np.full((B, Hq), -np.inf)
        logits = {}
        for b in range(B):
            for h in range(Hq) if heads is None else heads:
                g = h // G
                idx = None
                if sel_idx is not None:
                    idx = np.asarray(sel_idx[b, g])
                    idx = idx[idx >= 0]
                    n = len(idx)
                else:
                    n = int(seq_lens[b])
                nh = 0 if hot_lens is None else int(hot_lens[b])
                hk = np.asarray(hot_k[b, g, :nh]) if nh else None
                hv = np.asarray(hot_v[b, g, :nh]) if nh else None
                o, l, lg = self.decode_head(q[b, h], records[b, g], n, idx, hk, hv, scale or 0.0, want_logits)
                out[b, h], lse[b, h] = o, l
                if want_logits:
                    logits[(b, h)] = (lg[:n], lg[n:])
        return out, lse, logits

    def score_scan(self, q, records, n_tokens: int) -> np.ndarray:
        """q [B, Hkv, nq, d] against records [B, Hkv, :n_tokens] -> [B, Hkv, nq, n_tokens]."""
        B, H, nq, d = q.shape
        out = np.zeros((B, H, nq, n_tokens))
        for b in range(B):
            for h in range(H):
                qq = _f32(q[b, h])
                rec = np.ascontiguousarray(records[b, h, :n_tokens], np.uint8)
                o = np.zeros((nq, n_tokens))
                if self._L.sc_score_scan(self._c, _ptr(qq), nq, _ptr(rec), n_tokens, _ptr(o)):
                    raise MemoryError("sc_score_scan")
                out[b, h] = o
        return out


# ---------------------------------------------------------------------------------------
# Self-Indexing sign index and top-k
# ---------------------------------------------------------------------------------------
def channel_mean(k) -> np.ndarray:
    k = _f32(k)
    n, d = k.shape
    mu = np.zeros(d, np.float32)
    lib().sc_channel_mean(d, _ptr(k), n, _ptr(mu))
    return mu


def sign_index(k, mu):
    """k [n, d], mu [d] -> index [n, d/8] u8, codebook [d/4, 16, 4] f32."""
    k, mu = _f32(k), _f32(mu)
    n, d = k.shape
    index = np.zeros((n, d // 8), np.uint8)
    book = np.zeros((d // 4, 16, 4), np.float32)
    lib().sc_sign_index(d, _ptr(k), n, _ptr(mu), _ptr(index), _ptr(book))
    return index, book


def build_sign_index(K, n_tokens: int):
    """K [B, T, Hkv, d] -> index [B, Hkv, T, d/8], codebook [B, Hkv, d/4, 16, 4], mu [B, Hkv, d]."""
    B, T, H, d = K.shape
    index = np.zeros((B, H, T, d // 8), np.uint8)
    book = np.zeros((B, H, d // 4, 16, 4), np.float32)
    mus = np.zeros((B, H, d), np.float32)
    for b in range(B):
        for h in range(H):
            k = _f32(K[b, :n_tokens, h])
            mus[b, h] = channel_mean(k)
            index[b, h, :n_tokens], book[b, h] = sign_index(k, mus[b, h])
    return index, book, mus


def select_unit(q_group, index, book, n: int, k: int):
    """One (sequence, KV head): q_group [G, d] -> (idx [k], count, scores [k])."""
    q_group = _f32(q_group)
    G, d = q_group.shape
    index = np.ascontiguousarray(index, np.uint8)
    book = _f32(book)
    idx = np.zeros(max(k, 1), np.int32)
    sc = np.zeros(max(k, 1), np.int32)
    cnt = lib().sc_select_topk(d, G, _ptr(q_group), _ptr(index), _ptr(book), n, k, _ptr(idx), _ptr(sc))
    if cnt < 0:
        raise OverflowError("a sign-index score left int32")
    return idx[:k], cnt, sc[:k]


def select_topk(q, index, book, seq_lens, k: int):
    """q [B, Hq, d], index [B, Hkv, cap, d/8], book [B, Hkv, d/4, 16, 4] -> idx, count, scores."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    H = index.shape[1]
    G = Hq // H
    idx = np.full((B, H, k), -1, np.int32)
    cnt = np.zeros((B, H), np.int32)
    sc = np.zeros((B, H, k), np.int32)
    for b in range(B):
        for h in range(H):
            idx[b, h], cnt[b, h], sc[b, h] = select_unit(q[b, h * G:(h + 1) * G], index[b, h],
                                                         book[b, h], int(seq_lens[b]), k)
    return idx, cnt, sc
