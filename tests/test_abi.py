"""CPU checks of the C ABI: the library loads, exports what include/tq.h declares, builds the
same constants as the oracle from independent code, and rejects bad arguments on the host."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:tq_status|const char\*)\s+(tq_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    import compressed_key_attention_amd as tq
    names = _declared()
    assert len(names) >= 15
    lib = ctypes.CDLL(tq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(tq.EXPORTED) == names


@pytest.mark.parametrize("cfg", [(128, 3, 128, 4, 303, 304), (64, 3, 64, 4, 1, 2),
                                 (128, 4, 0, 4, 7, 8), (64, 2, 32, 2, 11, 12), (128, 2, 256, 3, 5, 6),
                                 (64, 1, 32, 1, 3, 4), (128, 1, 128, 4, 9, 10)])
def test_host_constants_equal_oracle(cfg):
    """Library (C++ SplitMix64 + Box-Muller + Householder QR + Lloyd-Max) and oracle
    (Python generator + LAPACK QR + scipy Lloyd-Max) are independent implementations of one
    definition; their float32 constants must agree bit for bit (one ulp tolerated in Pi)."""
    import compressed_key_attention_amd as tq
    from oracle import tq_oracle as O
    d, kb, m, vb, rs, qs = cfg
    lib = tq.host_constants(d, kb, m, vb, rs, qs)
    ref = O.Codec(d, kb, m, vb, rs, qs)
    ulp = np.abs(lib["pi"].view(np.int32).astype(np.int64) - ref.Pi.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, ulp.max()
    assert np.array_equal(lib["s"], ref.S)
    assert np.array_equal(lib["key_levels"], ref.key_levels)
    assert np.array_equal(lib["key_bounds"], ref.key_bounds)
    assert np.array_equal(lib["val_levels"], ref.val_levels)
    assert np.array_equal(lib["val_bounds"], ref.val_bounds)


def _cfg(**kw):
    import compressed_key_attention_amd as tq
    base = dict(head_dim=128, key_bits=3, qjl_dim=128, value_bits=4, rotation_seed=1, qjl_seed=2)
    base.update(kw)
    return tq.TqConfig(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=100), 2), (dict(head_dim=264), 2), (dict(head_dim=0), 1),
    (dict(key_codec=1, key_bits=3, polar_upper_bits=2), 2), (dict(key_codec=1, polar_upper_bits=3), 2),
    (dict(key_codec=2), 1), (dict(polar_upper_bits=1), 1),
    (dict(key_codec=1, head_dim=200, key_bits=4, polar_upper_bits=2), 2), (dict(key_bits=5), 1), (dict(value_bits=0), 1),
    (dict(qjl_dim=48), 1), (dict(qjl_dim=512), 1), (dict(key_codec=1, key_bits=1, polar_upper_bits=2), 2),
    (dict(qjl_dim=-32), 1)])
def test_config_validation_on_host(kw, status):
    import compressed_key_attention_amd as tq
    cfg = _cfg(**kw)
    assert tq._host_constants(ctypes.byref(cfg), None, None, None, None, None, None) == status
    assert tq.last_error() != ""
    h = ctypes.c_void_p()
    assert tq._create(ctypes.byref(cfg), ctypes.byref(h)) == status
    assert not h.value


def test_polar_and_head_dim_200_host_constants():
    """Polar grids come back for a polar config (and are refused for a scalar one); a
    head_dim of 200 builds the scalar constants (orthogonal Pi, codebooks)."""
    import compressed_key_attention_amd as tq
    lv, bd = tq.polar_host_constants(128, 4, 128, 4, 1, 2, 2)
    assert lv.shape == (7, 16) and np.all(np.diff(lv[0]) > 0) and np.all(np.diff(lv[1, :4]) > 0)
    assert np.all(np.isnan(lv[1, 4:])) and np.all((bd[1, :3] > 0) & (bd[1, :3] < np.pi / 2))
    cfg = _cfg()
    out = (ctypes.c_float * 256)()
    assert tq._polar_host_constants(ctypes.byref(cfg), out, out) == tq.TQ_ERR_INVALID_ARGUMENT
    c = tq.host_constants(200, 2, 192, 2, 5, 6)
    pi = c["pi"].astype(np.float64)
    assert np.abs(pi.T @ pi - np.eye(200)).max() < 1e-5


def test_null_handle_is_rejected_everywhere():
    import compressed_key_attention_amd as tq
    n = ctypes.c_size_t()
    assert tq._destroy(None) == 1
    assert tq._record_bytes(None, ctypes.byref(n), None) == 1
    assert tq._decode_ws(None, 1, 1, 1, 1, 0, ctypes.byref(n)) == 1
    assert tq._compress(None, None, None, 0, 1, 1, 1, 0, 0, 0, None, 1, 0, None) == 1
    assert tq._decode(None, None, 0, 1, 1, 1, None, 1, None, None, None, 0, None, 0, None, 0, 0.0,
                      None, None, None, None, 0, None) == 1
    assert tq._select(None, None, 0, 1, 1, 1, None, None, 1, None, 1, None, None, None, None, 0, None) == 1
    assert tq._scan(None, None, 0, 1, 1, 1, None, 1, 1, None, None, 0, None) == 1
    assert tq._sparse_ws(None, 1, 1, 1, 1, ctypes.byref(n)) == 1
    assert tq._sparse(None, None, 0, 1, 1, 1, None, None, None, 1, None, 1, None, None, 0, None, 0, 0.0,
                      None, None, None, 0, None) == 1
    assert tq._monarch_ws(None, 1, 1, 1, 1, 1, ctypes.byref(n)) == 1
    assert "NULL" in tq.last_error()


def test_record_size_formula_matches_oracle():
    from oracle import tq_oracle as O
    for d, kb, m, vb in [(128, 3, 128, 4), (64, 3, 64, 4), (128, 4, 0, 4), (64, 2, 32, 2)]:
        payload = d * kb // 8 + m // 8 + d * vb // 8 + 12
        assert O.Codec(d, kb, m, vb, 1, 2).record_bytes == (payload + 15) // 16 * 16


def _header_codes(field: np.ndarray, d: int, b: int) -> np.ndarray:
    """Codes of one key or value field [n, bytes] read exactly as include/tq.h states the layout
    (2/4-bit bitstreams; 3-bit groups of 32 codes in three words, a plain stream for the tail)."""
    n = field.shape[0]
    out = np.zeros((n, d), np.int64)
    stream = lambda buf, i, bits: sum(((int(buf[(bits * i + t) // 8]) >> ((bits * i + t) % 8)) & 1) << t
                                      for t in range(bits))
    for r in range(n):
        f = field[r]
        if b != 3:
            out[r] = [stream(f, i, b) for i in range(d)]
            continue
        for g in range(d // 32):
            W = [int.from_bytes(bytes(f[12 * g + 4 * w: 12 * g + 4 * w + 4]), "little") for w in range(3)]
            for j in range(24):
                out[r, 32 * g + j] = (W[j // 8] >> (8 * (j % 4) + 3 * ((j % 8) // 4))) & 7
            for rr in range(8):
                k = rr % 4
                T = sum(((W[t // 2] >> (8 * k + 6 + t % 2)) & 1) << t for t in range(6))
                out[r, 32 * g + 24 + rr] = (T >> (3 * (rr // 4))) & 7
        tail = f[12 * (d // 32):]
        for i in range(d % 32):
            out[r, 32 * (d // 32) + i] = stream(tail, i, 3)
    return out


@pytest.mark.parametrize("d,kb,m,vb", [(64, 3, 64, 4), (128, 3, 128, 4), (128, 2, 256, 3), (200, 3, 192, 2),
                                       (200, 2, 96, 3), (128, 4, 0, 4)])
def test_header_record_layout_matches_the_oracle_packer(d, kb, m, vb):
    """The record layout include/tq.h states (field sizes and offsets on 32-bit words, the 3-bit
    group layout, the plain tail, the 16-byte record padding), read back from records the oracle
    packs, gives the codes, bits and norms that went in."""
    from oracle import tq_oracle as O
    codec = O.Codec(d, kb, m, vb, 1, 2)
    KB, VB = 4 * -(-d * kb // 32), 4 * -(-d * vb // 32)
    rec_bytes = 16 * -(-(KB + m // 8 + VB + 12) // 16)
    assert (codec.kbytes, codec.sbytes, codec.vbytes, codec.record_bytes) == (KB, m // 8, VB, rec_bytes)
    rng = np.random.default_rng(d + kb + m + vb)
    n = 5
    f = dict(kc=rng.integers(0, 1 << kb, (n, d)), bits=rng.integers(0, 2, (n, m)),
             vc=rng.integers(0, 1 << vb, (n, d)), r_k=rng.random(n).astype(np.float32),
             rho=rng.random(n).astype(np.float32), r_v=rng.random(n).astype(np.float32))
    rec = O.pack_records(codec, f)
    assert rec.shape == (n, rec_bytes)
    assert np.array_equal(_header_codes(rec[:, :KB], d, kb), f["kc"])
    signs = rec[:, KB:KB + m // 8]
    assert np.array_equal(np.stack([[(signs[r, j // 8] >> (j % 8)) & 1 for j in range(m)] for r in range(n)])
                          .reshape(n, m), f["bits"])
    assert np.array_equal(_header_codes(rec[:, KB + m // 8:KB + m // 8 + VB], d, vb), f["vc"])
    norms = np.ascontiguousarray(rec[:, KB + m // 8 + VB:KB + m // 8 + VB + 12]).view("<f4")
    assert np.array_equal(norms, np.stack([f["r_k"], f["rho"], f["r_v"]], -1))
    assert np.all(rec[:, KB + m // 8 + VB + 12:] == 0)
    # bits past the last code of a field are zero padding
    for off, nb, b in ((0, KB, kb), (KB + m // 8, VB, vb)):
        used = d * b
        tailbits = np.unpackbits(rec[:, off:off + nb], axis=1, bitorder="little")[:, used:]
        assert not tailbits.any()
