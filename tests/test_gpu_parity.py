"""GPU parity: the HIP path (through the C ABI) against the oracle on identical seeded inputs.

Rules (checked element by element):
* packing from given rotated inputs: records bytewise equal;
* compress end to end: norms within 1e-6 relative; a key/value code may differ only where
  the oracle's rotated coordinate lies within 1e-6 of a boundary; a QJL bit may differ only
  where |p/rho| <= 1e-6, with p recomputed from the GPU's own codes;
* decode on identical records: logits and outputs within 1e-4 + 1e-3 |oracle|;
* sign index: patterns equal except where a key equals its channel mean to rounding;
  centroids within float32 rounding; top-k sets, counts and scores bit-exact given the same
  index and codebook;
* determinism: two runs give identical bytes.
"""
import math

import numpy as np
import pytest
import torch

from compressed_key_attention_amd import workloads as W
from oracle import polar as P
from oracle import tq_oracle as O

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 1e-3


def _tq():
    import compressed_key_attention_amd as tq
    return tq


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.detach().cpu().numpy()


def _close(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = ATOL + RTOL * np.abs(ref)
    bad = np.abs(gpu - ref) > tol
    if gpu.size:
        print(f"[tolerance] {what}: worst |gpu - ref| / tol = {np.max(np.abs(gpu - ref) / tol):.3f}", flush=True)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                           f"{np.max(np.abs(gpu - ref) - RTOL * np.abs(ref)):.3e}")


_CODECS = {}


def _codec(h):
    key = (h.head_dim, h.key_bits, h.qjl_dim, h.value_bits, h.rotation_seed, h.qjl_seed)
    ub = getattr(h, "polar_upper_bits", 0)
    if (key, ub) not in _CODECS:
        _CODECS[(key, ub)] = P.PolarCodec(*key, upper_bits=ub) if ub else O.Codec(*key)
    return _CODECS[(key, ub)]


def _handle(w: W.Workload):
    return _tq().Handle(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2,
                        polar_upper_bits=w.polar_upper_bits)


def check_compress(codec, K, V, rec_gpu):
    """End-to-end compress rule on one set of tokens: K, V [n, d] float, rec_gpu [n, R] u8."""
    d = codec.head_dim
    fg = O.unpack_records(codec, rec_gpu)
    ref = O.compress(codec, K, V)
    for key in ("r_k", "r_v"):
        assert np.allclose(fg[key], ref[key], rtol=1e-6, atol=0), key
    assert np.all(rec_gpu[:, codec.kbytes + codec.sbytes + codec.vbytes + 12:] == 0)   # zero pad
    stats = {}
    for which, X, bounds in (("kc", K, codec.key_bounds), ("vc", V, codec.val_bounds)):
        _, _, z32, _ = O._rotate_and_code(codec, X, bounds)
        mism = fg[which] != ref[which]
        if mism.any():
            dist = np.min(np.abs(z32[..., None].astype(np.float64) - bounds.astype(np.float64)), axis=-1)
            assert np.all(dist[mism] <= 1e-6), f"{which}: code mismatch away from a boundary"
        stats[which] = int(mism.sum())
    # residual sketch, recomputed from the GPU's codes
    if codec.qjl_dim:
        k64 = K.astype(np.float64)
        x = k64 @ codec.Pi64.T
        xhat = (fg["r_k"].astype(np.float64) / math.sqrt(d))[:, None] * codec.key_levels.astype(np.float64)[fg["kc"]]
        e = x - xhat
        rho = np.sqrt(np.sum(e * e, -1))
        assert np.allclose(fg["rho"], rho.astype(np.float32), rtol=2e-6, atol=1e-30)
        p = e @ codec.S64.T
        want = (p.astype(np.float32) >= 0)
        mism = (fg["bits"] == 1) != want
        if mism.any():
            rel = np.abs(p) / np.maximum(rho, 1e-300)[:, None]
            assert np.all(rel[mism] <= 1e-6), "QJL bit mismatch away from zero"
        stats["bits"] = int(mism.sum())
    return stats


def _compress(w, h, K, V, capacity=None, first_slot=0):
    B, T, H, d = K.shape
    cap = T + first_slot if capacity is None else capacity
    rec = torch.full((B, H, cap, h.record_bytes), 0xAB, dtype=torch.uint8, device="cuda")
    h.compress_kv(K, V, rec, first_slot=first_slot)
    torch.cuda.synchronize()
    return rec


# ------------------------------------------------------------------ packing -------------
@pytest.mark.parametrize("cfg", [(128, 3, 128, 4), (64, 3, 64, 4), (128, 4, 0, 4), (128, 2, 256, 3),
                                 (64, 4, 32, 2), (128, 3, 64, 2)])
def test_debug_quantize_is_bit_exact(cfg):
    tq = _tq()
    d, kb, m, vb = cfg
    h = tq.Handle(d, kb, m, vb, 5, 6)
    codec = _codec(h)
    n = 333
    rng = np.random.default_rng(sum(cfg))
    zk = rng.standard_normal((n, d)).astype(np.float32) * 1.5
    zv = rng.standard_normal((n, d)).astype(np.float32) * 1.5
    # exact boundaries, their neighbours, signed zeros and far tails
    zk[0, : len(codec.key_bounds)] = codec.key_bounds
    zk[1, : len(codec.key_bounds)] = np.nextafter(codec.key_bounds, np.float32(-np.inf))
    zk[2, :4] = [0.0, -0.0, 1e30, -1e30]
    zv[0, : len(codec.val_bounds)] = codec.val_bounds
    p = rng.standard_normal((n, max(m, 1))).astype(np.float32)[:, :m]
    if m:
        p[0, :3] = [0.0, -0.0, -1e-40]
    rk, rho, rv = (rng.random(n).astype(np.float32) + 0.1 for _ in range(3))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    rec = torch.full((n, h.record_bytes), 0xCD, dtype=torch.uint8, device="cuda")
    h.debug_quantize(dev(zk), dev(p) if m else dev(np.zeros((n, 1), np.float32)), dev(rk), dev(rho), dev(zv),
                     dev(rv), rec)
    torch.cuda.synchronize()
    ref = O.quantize_from_rotated(codec, zk, p, rk, rho, zv, rv)
    assert np.array_equal(rec.cpu().numpy(), ref)


@pytest.mark.parametrize("d,kb,m,vb", [(64, 3, 64, 4), (128, 3, 128, 4), (200, 3, 192, 2), (200, 2, 96, 3),
                                       (128, 4, 0, 4), (128, 2, 256, 3)])
def test_record_bytes_as_the_header_states(d, kb, m, vb):
    """tq_record_bytes = 16 ceil((4 ceil(d kb / 32) + m / 8 + 4 ceil(d vb / 32) + 12) / 16), and
    the sign-index record is d / 8 bytes."""
    h = _tq().Handle(d, kb, m, vb, 1, 2)
    KB, VB = 4 * -(-d * kb // 32), 4 * -(-d * vb // 32)
    assert h.record_bytes == 16 * -(-(KB + m // 8 + VB + 12) // 16)
    assert h.index_record_bytes == d // 8


# ------------------------------------------------------------------ compress ------------
@pytest.mark.parametrize("name,tokens,batch", [("single_head_1k", 1024, 1), ("tinyllama_layer", 1024, 1),
                                               ("llama8b_decode_32k", 1000, 2), ("sparse_128k_top2048", 777, 1),
                                               ("bulk_64k_scan", 2000, 1)])
def test_compress_end_to_end(name, tokens, batch):
    w = W.small(W.WORKLOADS[name], tokens=tokens, batch=batch)
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cpu")
    K[0, 5] = 0          # a zero key/value vector (codes at the middle cell, rho = 0)
    V[0, 5] = 0
    Kc, Vc = K.cuda(), V.cuda()
    rec = _compress(w, h, Kc, Vc)
    rec2 = _compress(w, h, Kc, Vc)
    assert torch.equal(rec, rec2), "compress is not deterministic"
    r = rec.cpu().numpy()
    Kn, Vn = _np(K), _np(V)
    total = {}
    for b in range(w.batch):
        for hh in range(w.kv_heads):
            st = check_compress(codec, Kn[b, :, hh], Vn[b, :, hh], r[b, hh])
            for k2, v2 in st.items():
                total[k2] = total.get(k2, 0) + v2
    f = O.unpack_records(codec, r[0, 0, 5:6])
    assert np.all(f["kc"] == 1 << (w.key_bits - 1)) and f["rho"][0] == 0
    if w.qjl_dim:
        assert np.all(f["bits"] == 1)
    print(name, "exempt mismatches", total)


def test_compress_strided_layout_offset_slots_and_ragged_tail():
    w = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=203, batch=2)
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cpu")
    # [B, H, T, d] storage viewed as [B, T, H, d]
    Kh = K.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    Vh = V.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    rec = _compress(w, h, Kh, Vh, capacity=300, first_slot=50)
    ref = _compress(w, h, K.cuda(), V.cuda())
    r = rec.cpu().numpy()
    assert np.array_equal(r[:, :, 50:253], ref.cpu().numpy())
    assert np.all(r[:, :, :50] == 0xAB) and np.all(r[:, :, 253:] == 0xAB)   # untouched slots
    check_compress(codec, _np(K)[1, :, 3], _np(V)[1, :, 3], r[1, 3, 50:253])


def test_compress_rejects_bad_arguments():
    tq = _tq()
    h = tq.Handle(128, 3, 128, 4, 1, 2)
    K = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    rec = torch.zeros((1, 1, 8, h.record_bytes), dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TqError) as e:
        h.compress_kv(K, K, rec, first_slot=1)        # exceeds capacity
    assert e.value.status == tq.TQ_ERR_INVALID_ARGUMENT
    Kodd = torch.zeros((1, 8, 1, 130), dtype=torch.bfloat16, device="cuda")[..., 1:129]
    with pytest.raises(tq.TqError):
        h.compress_kv(Kodd, Kodd, rec)                # misaligned rows


# ------------------------------------------------------------------ decode --------------
def _decode_case(w, seq_lens, hot_lens=None, scale=0.0, sel=None, heads_to_check=None):
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = _compress(w, h, K, V)
    q = W.make_queries(w, "cuda")
    B = w.batch
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    hk = hv = hl = None
    if hot_lens is not None:
        hk, hv = W.make_hot(w, "cuda")
        hl = torch.tensor(hot_lens, dtype=torch.int32, device="cuda")
    k_sel = 0 if sel is None else sel.shape[-1]
    ncold = k_sel if sel is not None else rec.shape[2]
    lw = ncold + (0 if hk is None else hk.shape[2])
    out = torch.full((B, w.q_heads, w.head_dim), float("nan"), device="cuda")
    lse = torch.full((B, w.q_heads), float("nan"), device="cuda")
    logits = torch.full((B, w.q_heads, lw), float("nan"), device="cuda")
    h.decode_attention(q, rec, sl, hot_k=hk, hot_v=hv, hot_lens=hl, sel_idx=sel, scale=scale,
                       out=out, lse=lse, logits=logits)
    out2 = h.decode_attention(q, rec, sl, hot_k=hk, hot_v=hv, hot_lens=hl, sel_idx=sel, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "decode is not deterministic"
    r = rec.cpu().numpy()
    qn = _np(q)
    ref_out, ref_lse, ref_lg = O.decode_attention(
        codec, qn, r, seq_lens, None if hk is None else _np(hk), None if hv is None else _np(hv),
        hot_lens, None if sel is None else sel.cpu().numpy(), scale, heads=heads_to_check)
    o, L, lg = out.cpu().numpy(), lse.cpu().numpy(), logits.cpu().numpy()
    for (b, hq), (lc, lh) in ref_lg.items():
        _close(o[b, hq], ref_out[b, hq], f"out[{b},{hq}]")
        if np.isinf(ref_lse[b, hq]):
            assert np.isneginf(L[b, hq]) and np.all(o[b, hq] == 0)
        else:
            _close(L[b, hq], ref_lse[b, hq], f"lse[{b},{hq}]")
        if sel is None:
            _close(lg[b, hq, : len(lc)], lc, f"cold logits[{b},{hq}]")
        else:
            idx = sel.cpu().numpy()[b, hq // w.group]
            pos = np.nonzero(idx >= 0)[0]
            _close(lg[b, hq, pos], lc, f"gathered logits[{b},{hq}]")
        if len(lh):
            _close(lg[b, hq, ncold: ncold + len(lh)], lh, f"hot logits[{b},{hq}]")
    return out


def test_decode_single_head_1k_full_size():
    w = W.WORKLOADS["single_head_1k"]
    _decode_case(w, [1024])


def test_decode_tinyllama_layer_full_size_with_exact_segment():
    w = W.WORKLOADS["tinyllama_layer"]
    _decode_case(w, [1024], hot_lens=[512])


def test_decode_llama8b_shape_reduced_ragged():
    w = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=3000, batch=3)
    _decode_case(w, [3000, 1, 2049])


def test_decode_group_sizes_and_empty_sequences():
    base = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=700, batch=2)
    for hq in (8, 16, 64):           # G = 1, 2, 8
        w = W.Workload(**{**base.__dict__, "q_heads": hq, "name": "llama8b_decode_32k"})
        _decode_case(w, [700, 0])
    w2 = W.small(W.WORKLOADS["tinyllama_layer"], tokens=300, batch=2, hot_tokens=40)
    _decode_case(w2, [0, 299], hot_lens=[17, 0], scale=0.3)


@pytest.mark.parametrize("base,hq,hkv,tokens", [
    ("single_head_1k", 4, 1, 320), ("single_head_1k", 4, 1, 1100), ("single_head_1k", 4, 1, 2500),
    ("single_head_1k", 2, 1, 1100), ("single_head_1k", 2, 1, 2500),
    ("single_head_1k", 1, 1, 320), ("single_head_1k", 1, 1, 2047), ("single_head_1k", 1, 1, 2100),
    ("tinyllama_layer", 2, 2, 3000), ("tinyllama_layer", 2, 2, 4500)])
def test_decode_merge_paths_by_chunk_count(base, hq, hkv, tokens):
    """The merge without an exact segment at chunk counts on each side of its paths: one block
    per query head with every chunk in one round trip (at most 8 chunks), chunks split over the
    block's threads (up to 16 * 256 / head_dim chunks), and the running-maximum pass beyond
    (or the general merge for one query head per KV head); 64-token chunks at these sizes."""
    b = W.WORKLOADS[base]
    w = W.Workload(**{**W.small(b, tokens=tokens, batch=1).__dict__, "q_heads": hq, "kv_heads": hkv,
                      "name": base})
    _decode_case(w, [tokens])


def test_decode_cache_run_beyond_32_bit_offsets():
    """A cache whose (sequence, KV head) runs exceed 2^31 bytes (15,000,000 slots of 144 bytes
    per head, 4.3 GB of records): the host sends the matrix-core shape (head_dim 128, 4 query
    heads per KV head) to the 64-bit-offset scan, and the second head's records, 2.16 GB into
    the buffer, decode as the oracle says."""
    base = W.WORKLOADS["llama8b_decode_32k"]
    w = W.Workload(**{**W.small(base, tokens=1000, batch=1).__dict__, "q_heads": 8, "kv_heads": 2,
                      "name": "llama8b_decode_32k"})
    cap = 15_000_000
    h = _handle(w)
    assert cap * h.record_bytes >= 2 ** 31
    K, V = W.make_kv(w, "cuda")
    rec = h.new_cache(1, w.kv_heads, cap, "cuda")
    h.compress_kv(K, V, rec)
    q = W.make_queries(w, "cuda")
    sl = torch.tensor([w.tokens], dtype=torch.int32, device="cuda")
    out = torch.full((1, w.q_heads, w.head_dim), float("nan"), device="cuda")
    lse = torch.full((1, w.q_heads), float("nan"), device="cuda")
    h.decode_attention(q, rec, sl, out=out, lse=lse)
    torch.cuda.synchronize()
    small = rec[:, :, : w.tokens].cpu().numpy()
    del rec
    torch.cuda.empty_cache()
    ref_out, ref_lse, _ = O.decode_attention(_codec(h), _np(q), small, [w.tokens])
    _close(out.cpu().numpy(), ref_out, "out (15M-slot cache)")
    _close(lse.cpu().numpy(), ref_lse, "lse (15M-slot cache)")


def test_decode_long_exact_segment():
    """Exact segments longer than the merge kernel keeps in LDS (logits recomputed past 2,048),
    float32 and bfloat16 hot tokens, head_dim 128, ragged hot lengths."""
    w = W.small(W.WORKLOADS["single_head_1k"], tokens=500, hot_tokens=2600)
    _decode_case(w, [500], hot_lens=[2600])
    w2 = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=900, batch=2, hot_tokens=2100)
    _decode_case(w2, [900, 333], hot_lens=[2100, 2049])


def test_decode_gather_mode():
    w = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=4000, batch=2)
    rng = np.random.default_rng(1)
    sel = np.full((2, w.kv_heads, 300), -1, np.int32)
    for b in range(2):
        for hh in range(w.kv_heads):
            k = rng.integers(1, 300)
            sel[b, hh, :k] = np.sort(rng.choice(4000, size=k, replace=False))
    _decode_case(w, [4000, 4000], sel=torch.from_numpy(sel).cuda())


@pytest.mark.parametrize("kb,m", [(3, 128), (2, 128), (3, 0), (2, 0)])
def test_decode_matrix_core_path_variants(kb, m):
    """head_dim 128 with 4 query heads per KV head and 4-bit values runs the matrix-core scan;
    cover each of its key widths with and without the QJL sketch, ragged lengths, gather."""
    base = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=1500, batch=2)
    w = W.Workload(**{**base.__dict__, "key_bits": kb, "qjl_dim": m})
    _decode_case(w, [1500, 777])
    rng = np.random.default_rng(kb + m)
    sel = np.full((2, w.kv_heads, 200), -1, np.int32)
    for b in range(2):
        for hh in range(w.kv_heads):
            k = rng.integers(1, 200)
            sel[b, hh, :k] = np.sort(rng.choice(1500, size=k, replace=False))
    _decode_case(w, [1500, 1500], sel=torch.from_numpy(sel).cuda())


@pytest.mark.parametrize("d,kb,vb,m,hq", [(64, 2, 2, 0, 16), (128, 4, 3, 64, 32), (64, 3, 3, 128, 32),
                                           (128, 2, 4, 128, 64), (64, 4, 4, 32, 16)])
def test_decode_short_cache_direct_kernel(d, kb, vb, m, hq):
    """Short caches with 4 or more query heads per KV head off the matrix-core path run the
    direct kernel (codes unpacked per chunk, no per-query tables): key and value widths 2-4,
    sketches of 0-128 bits, group sizes 4-16, ragged lengths, an empty chunk tail, gather."""
    base = W.small(W.WORKLOADS["tinyllama_layer"], tokens=900, batch=2, hot_tokens=0)
    w = W.Workload(**{**base.__dict__, "head_dim": d, "key_bits": kb, "value_bits": vb, "qjl_dim": m,
                      "q_heads": hq})
    _decode_case(w, [900, 333])
    rng = np.random.default_rng(d + kb + vb + m)
    sel = np.full((2, w.kv_heads, 150), -1, np.int32)
    for b in range(2):
        for hh in range(w.kv_heads):
            k = rng.integers(1, 150)
            sel[b, hh, :k] = np.sort(rng.choice(900, size=k, replace=False))
    _decode_case(w, [900, 900], sel=torch.from_numpy(sel).cuda())


def test_decode_rejects_small_workspace():
    tq = _tq()
    h = tq.Handle(128, 3, 128, 4, 1, 2)
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    rec = torch.zeros((1, 1, 64, h.record_bytes), dtype=torch.uint8, device="cuda")
    sl = torch.tensor([64], dtype=torch.int32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TqError) as e:
        h.decode_attention(q, rec, sl, workspace=ws)
    assert e.value.status == tq.TQ_ERR_WORKSPACE_TOO_SMALL


# ------------------------------------------------------------------ sign index + top-k ---
def check_sign_index_unit(k, gmu, gpat, gbook, rmu, rpat, rbook, pat_at_gmu, book_at_gpat, what):
    """Sign index of one (sequence, KV head) unit against the oracle, with no skipped case.

    k [n, d] float32 keys; gmu / gpat / gbook the GPU's mean, patterns [n, d/4] and codebook;
    rmu / rpat / rbook the oracle's own; pat_at_gmu and book_at_gpat the oracle's pattern and
    centroid steps taken at the GPU's mean and patterns.  Both sides sum the mean and the
    centroids in float64 and round once to float32, so they may differ by one float32 rounding;
    given the same mean the patterns are bit-exact; against the oracle's own mean a pattern bit
    may differ only where the key lies between the two means.  Returns the flipped-bit count."""
    n, d = k.shape
    ulp = np.spacing(np.abs(rmu).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(gmu.astype(np.float64) - rmu) <= ulp), f"{what}: channel means"
    assert np.array_equal(gpat, pat_at_gmu), f"{what}: patterns at the GPU's mean"
    bits_g = ((gpat[..., None] >> np.arange(4)) & 1).reshape(n, d)
    bits_r = ((rpat[..., None] >> np.arange(4)) & 1).reshape(n, d)
    diff = bits_g != bits_r
    if diff.any():
        lo = np.broadcast_to(np.minimum(gmu, rmu), diff.shape)
        hi = np.broadcast_to(np.maximum(gmu, rmu), diff.shape)
        assert np.all((k[diff] >= lo[diff]) & (k[diff] <= hi[diff])), f"{what}: index bits away from the mean"
    np.testing.assert_allclose(gbook, book_at_gpat, rtol=2.4e-7, atol=1e-12,
                               err_msg=f"{what}: codebook at the GPU's patterns")
    if not diff.any():
        np.testing.assert_allclose(gbook, rbook, rtol=2.4e-7, atol=1e-12, err_msg=f"{what}: codebook")
    return int(diff.sum())


def _index_case(w, seq_lens, k, q_heads=None):
    h = _handle(w)
    codec = _codec(h)
    K, _ = W.make_kv(w, "cuda")
    B, T, H, d = K.shape
    index = torch.full((B, H, T, d // 8), 0xEE, dtype=torch.uint8, device="cuda")
    book = torch.full((B, H, d // 4, 16, 4), float("nan"), device="cuda")
    mean = torch.empty((B, H, d), device="cuda")
    h.build_sign_index(K, index, book, mean)
    torch.cuda.synchronize()
    Kn = _np(K)
    ref_idx, ref_book, ref_mu = O.build_sign_index(codec, Kn, T)
    mu = mean.cpu().numpy()
    gi, gb = index.cpu().numpy(), book.cpu().numpy()
    ng = d // 4
    for b in range(B):
        for hh in range(H):
            kf = Kn[b, :, hh].astype(np.float32)
            gpat = O._unpack_stream(gi[b, hh], ng, 4)
            check_sign_index_unit(kf, mu[b, hh], gpat, gb[b, hh], ref_mu[b, hh],
                                  O._unpack_stream(ref_idx[b, hh], ng, 4), ref_book[b, hh],
                                  O.sign_patterns(kf, mu[b, hh]), O.pattern_centroids(kf, mu[b, hh], gpat),
                                  f"unit {(b, hh)}")
    # selection: GPU vs oracle on the GPU-built index and codebook -> bit-exact
    Hq = q_heads or w.q_heads
    q = W.make_queries(W.Workload(**{**w.__dict__, "q_heads": Hq}), "cuda")
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    out_idx = torch.full((B, H, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
    scs = torch.full((B, H, k), -7, dtype=torch.int32, device="cuda")
    h.select_topk(q, index, book, sl, k, out_idx=out_idx, out_count=cnt, out_scores=scs)
    torch.cuda.synchronize()
    ri, rc, rs = O.select_topk(codec, _np(q), gi, gb, seq_lens, k)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(out_idx.cpu().numpy(), ri)
    assert np.array_equal(scs.cpu().numpy(), rs)
    return h, K, q, index, book, out_idx


def test_sign_index_and_topk_reduced():
    w = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=9000, batch=2)
    _index_case(w, [9000, 4097], 512)


@pytest.mark.parametrize("k,lens", [(0, [100, 100]), (100, [100, 37]), (1, [100, 1]), (300, [300, 0])])
def test_topk_edge_cases(k, lens):
    w = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=300, batch=2)
    _index_case(w, lens, k)


def test_topk_with_ties_and_grouped_heads():
    w = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=2048, batch=1)
    _index_case(w, [2048], 333, q_heads=32)       # G = 4: one selection per KV head


@pytest.mark.parametrize("patterns,k", [(3, 5000), (1, 777), (40, 9000)])
def test_topk_heavy_ties(patterns, k):
    """Index rows drawn from a few distinct patterns: long runs of equal scores across chunks,
    so the cut falls inside a tie and the lowest indices must win."""
    w = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=20000, batch=1)
    h = _handle(w)
    codec = _codec(h)
    K, _ = W.make_kv(w, "cuda")
    B, T, H, d = K.shape
    index = torch.empty((B, H, T, d // 8), dtype=torch.uint8, device="cuda")
    book = torch.empty((B, H, d // 4, 16, 4), device="cuda")
    h.build_sign_index(K, index, book)
    g = torch.Generator().manual_seed(patterns)
    rows = torch.randint(0, T, (patterns,), generator=g)
    pick = torch.randint(0, patterns, (T,), generator=g)
    index = index[:, :, rows[pick]].contiguous()
    q = W.make_queries(w, "cuda")
    sl = torch.tensor([T], dtype=torch.int32, device="cuda")
    out_idx = torch.full((B, H, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
    scs = torch.full((B, H, k), -7, dtype=torch.int32, device="cuda")
    h.select_topk(q, index, book, sl, k, out_idx=out_idx, out_count=cnt, out_scores=scs)
    torch.cuda.synchronize()
    ri, rc, rs = O.select_topk(codec, _np(q), index.cpu().numpy(), book.cpu().numpy(), [T], k)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(out_idx.cpu().numpy(), ri)
    assert np.array_equal(scs.cpu().numpy(), rs)


def test_select_then_gather_attention():
    w = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=6000, batch=2, top_k=256)
    h, K, q, index, book, sel = _index_case(w, [6000, 6000], 256)
    codec = _codec(h)
    _, V = W.make_kv(w, "cuda")
    rec = _compress(w, h, K, V)
    sl = torch.tensor([6000, 6000], dtype=torch.int32, device="cuda")
    out = h.decode_attention(q, rec, sl, sel_idx=sel)
    torch.cuda.synchronize()
    ref, _, _ = O.decode_attention(codec, _np(q), rec.cpu().numpy(), [6000, 6000], sel_idx=sel.cpu().numpy())
    _close(out.cpu().numpy(), ref, "gather attention")


@pytest.mark.parametrize("kb,vb", [(4, 4), (2, 2)])
def test_sparse_with_exact_sinks(kb, vb):
    """Self-Indexing decode with 64 full-precision sink tokens always attended (as the exact
    segment, outside the compressed and indexed range) and top-k gather over the rest, for the
    4-bit payload and the 2-bit variant."""
    base = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=5000, batch=2, top_k=300)
    w = W.Workload(**{**base.__dict__, "key_bits": kb, "value_bits": vb})
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    B, T, H, d = K.shape
    S = 64
    Kc, Vc = K[:, S:].contiguous(), V[:, S:].contiguous()       # compressed + indexed: tokens S..T-1
    sinks_k = K[:, :S].permute(0, 2, 1, 3).contiguous()          # exact: [B, H, S, d]
    sinks_v = V[:, :S].permute(0, 2, 1, 3).contiguous()
    index = torch.empty((B, H, T - S, d // 8), dtype=torch.uint8, device="cuda")
    book = torch.empty((B, H, d // 4, 16, 4), device="cuda")
    h.build_sign_index(Kc, index, book)
    rec = _compress(w, h, Kc, Vc)
    q = W.make_queries(w, "cuda")
    lens = [T - S, 3000]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    hl = torch.tensor([S, S], dtype=torch.int32, device="cuda")
    sel, cnt = h.select_topk(q, index, book, sl, w.top_k)
    out = torch.full((B, w.q_heads, d), float("nan"), device="cuda")
    h.decode_attention(q, rec, sl, hot_k=sinks_k, hot_v=sinks_v, hot_lens=hl, sel_idx=sel, out=out)
    torch.cuda.synchronize()
    ri, rc, _ = O.select_topk(codec, _np(q), index.cpu().numpy(), book.cpu().numpy(), lens, w.top_k)
    assert np.array_equal(sel.cpu().numpy(), ri) and np.array_equal(cnt.cpu().numpy(), rc)
    ref, _, _ = O.decode_attention(codec, _np(q), rec.cpu().numpy(), lens, _np(sinks_k), _np(sinks_v), [S, S],
                                   sel_idx=ri)
    _close(out.cpu().numpy(), ref, f"sparse + sinks kb={kb} vb={vb}")


@pytest.mark.parametrize("kb,vb,m,hq,k,lens,sinks,ub,d", [
    (4, 4, 0, 8, 300, [5000, 4097], 0, 0, 128),       # one query head per KV head (the sparse family)
    (2, 2, 0, 8, 1000, [9000, 123], 64, 0, 128),      # 2-bit payload, 64 exact sink tokens
    (3, 4, 128, 32, 500, [6000, 6000], 0, 0, 128),    # 4 query heads per KV head, 128-bit sketch
    (4, 4, 64, 16, 0, [300, 300], 16, 0, 128),        # k = 0: the sink tokens only
    (4, 4, 0, 8, 5000, [4500, 100], 0, 0, 128),       # k >= n: every token
    (4, 4, 0, 8, 700, [5000, 4097], 0, 2, 128),       # polar keys (4-bit level-1, 2-bit upper angles)
    (4, 4, 128, 32, 500, [6000, 3000], 64, 4, 128),   # polar keys, sketch, G = 4, sinks
    (2, 3, 64, 16, 400, [3000, 2500], 32, 1, 64),     # polar keys at head_dim 64
    (4, 4, 0, 8, 900, [7000, 3000], 64, 0, 128),      # the lean kernel (G = 1, 4/4-bit, no sketch) with sinks
    (4, 4, 0, 8, 500, [5000, 2000], 0, 0, 64),        # the lean kernel at head_dim 64
    (4, 4, 0, 8, 0, [300, 300], 16, 0, 128),          # the lean kernel, k = 0: sinks only
    (4, 4, 0, 8, 3000, [3000, 2999], 0, 0, 128),      # the lean kernel, whole chunks selected (47 batches)
])
def test_sparse_attention_one_call(kb, vb, m, hq, k, lens, sinks, ub, d):
    """tq_sparse_attention (selection and attention in one call, no index list) against the
    oracle's select_topk followed by its gathered decode, with the exact segment as sinks;
    scalar and polar key codes."""
    T = max(lens) + sinks
    base = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=T, batch=len(lens), top_k=max(k, 1))
    w = W.Workload(**{**base.__dict__, "key_bits": kb, "value_bits": vb, "qjl_dim": m, "q_heads": hq,
                      "polar_upper_bits": ub, "head_dim": d})
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    B, _, H, d = K.shape
    S = sinks
    Kc, Vc = K[:, S:].contiguous(), V[:, S:].contiguous()
    index = torch.empty((B, H, T - S, d // 8), dtype=torch.uint8, device="cuda")
    book = torch.empty((B, H, d // 4, 16, 4), device="cuda")
    h.build_sign_index(Kc, index, book)
    rec = _compress(w, h, Kc, Vc)
    q = W.make_queries(w, "cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    hot, hk, hv, hlens = {}, None, None, None
    if S:
        hk = K[:, :S].permute(0, 2, 1, 3).contiguous()
        hv = V[:, :S].permute(0, 2, 1, 3).contiguous()
        hlens = [S] * B
        hot = dict(hot_k=hk, hot_v=hv, hot_lens=torch.tensor(hlens, dtype=torch.int32, device="cuda"))
    out = torch.full((B, hq, d), float("nan"), device="cuda")
    lse = torch.full((B, hq), float("nan"), device="cuda")
    h.sparse_attention(q, index, book, rec, sl, k, out=out, lse=lse, **hot)
    out2 = h.sparse_attention(q, index, book, rec, sl, k, **hot)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "sparse attention is not deterministic"
    gi, gb = index.cpu().numpy(), book.cpu().numpy()
    if k > 0:
        ri, _, _ = O.select_topk(codec, _np(q), gi, gb, lens, k)
    else:
        ri = np.full((B, H, 1), -1, np.int32)
    ref, ref_lse, _ = O.decode_attention(codec, _np(q), rec.cpu().numpy(), lens,
                                         None if hk is None else _np(hk), None if hv is None else _np(hv),
                                         hlens, sel_idx=ri)
    o, L = out.cpu().numpy(), lse.cpu().numpy()
    _close(o, ref, f"sparse attention kb={kb} vb={vb} m={m} G={hq // H} k={k}")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(L), fin)
    _close(L[fin], ref_lse[fin], "sparse attention lse")
    assert np.all(o[~fin] == 0)


# ------------------------------------------------------------------ bulk scan -----------
def test_score_scan_reduced():
    w = W.small(W.WORKLOADS["bulk_64k_scan"], tokens=1000, scan_queries=70)
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = _compress(w, h, K, V)
    q = W.make_queries(w, "cuda")
    sc = torch.full((1, w.kv_heads, 70, 1000), float("nan"), device="cuda")
    h.score_scan(q, rec, 1000, scores=sc)
    torch.cuda.synchronize()
    ref = O.score_scan(codec, _np(q), rec.cpu().numpy(), 1000)
    _close(sc.cpu().numpy(), ref, "scan scores")


@pytest.mark.parametrize("kb,m,d,nq,T,n_tok", [(3, 128, 128, 70, 1000, 1000), (2, 128, 128, 37, 2100, 2093),
                                                (3, 0, 128, 33, 4097, 4097), (2, 0, 128, 5, 300, 17),
                                                (3, 128, 128, 150, 3000, 2996), (3, 64, 64, 20, 500, 500)])
def test_score_scan_variants(kb, m, d, nq, T, n_tok):
    """Matrix-core scan for both key widths with and without the sketch, query counts that are
    not multiples of the 16-query tiles or 64-query workgroup blocks, token counts past the
    1024-token blocks, below the capacity, with and without whole 16-byte score groups (2996,
    2093); head_dim 64 (and m = 64) takes the generic kernel."""
    base = W.small(W.WORKLOADS["bulk_64k_scan"], tokens=T, scan_queries=nq)
    w = W.Workload(**{**base.__dict__, "key_bits": kb, "qjl_dim": m, "head_dim": d})
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = _compress(w, h, K, V)
    q = W.make_queries(w, "cuda")
    sc = torch.full((1, w.kv_heads, nq, n_tok), float("nan"), device="cuda")
    h.score_scan(q, rec, n_tok, scores=sc)
    torch.cuda.synchronize()
    ref = O.score_scan(codec, _np(q), rec.cpu().numpy(), n_tok)
    _close(sc.cpu().numpy(), ref, f"scan scores kb={kb} m={m} d={d}")


# ------------------------------------------------------------------ full sizes, sampled --
def test_llama8b_decode_full_size_sampled():
    w = W.WORKLOADS["llama8b_decode_32k"]
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = _compress(w, h, K, V)
    # compress: sampled tokens of sampled (b, h)
    r = rec[[0, 15]][:, [0, 7]].cpu().numpy()
    for bi, b in enumerate([0, 15]):
        for hi, hh in enumerate([0, 7]):
            toks = np.r_[0:64, 32700:32768]
            check_compress(codec, _np(K[b, toks, hh]), _np(V[b, toks, hh]), r[bi, hi, toks])
    q = W.make_queries(w, "cuda")
    sl = torch.full((w.batch,), w.tokens, dtype=torch.int32, device="cuda")
    lse = torch.empty((w.batch, w.q_heads), device="cuda")
    out = h.decode_attention(q, rec, sl, lse=lse)
    torch.cuda.synchronize()
    for b, hq in [(0, 0), (7, 13), (15, 31)]:
        ref, ref_lse, _ = O.decode_attention(codec, _np(q[b:b + 1]), rec[b:b + 1].cpu().numpy(), [w.tokens],
                                             heads=[hq])
        _close(out[b, hq].cpu().numpy(), ref[0, hq], f"out[{b},{hq}]")
        _close(lse[b, hq].item(), ref_lse[0, hq], f"lse[{b},{hq}]")


def test_sparse_128k_full_size_sampled():
    w = W.WORKLOADS["sparse_128k_top2048"]
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    B, T, H, d = K.shape
    index = torch.empty((B, H, T, d // 8), dtype=torch.uint8, device="cuda")
    book = torch.empty((B, H, d // 4, 16, 4), device="cuda")
    h.build_sign_index(K, index, book)
    q = W.make_queries(w, "cuda")
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    sel, cnt = h.select_topk(q, index, book, sl, w.top_k)
    rec = _compress(w, h, K, V)
    out = h.decode_attention(q, rec, sl, sel_idx=sel)
    torch.cuda.synchronize()
    gi, gb = index.cpu().numpy(), book.cpu().numpy()
    qn = _np(q)
    for b, hh in [(0, 0), (3, 5)]:
        ri, rc, _ = O.select_topk(codec, qn[b:b + 1, hh:hh + 1], gi[b:b + 1, hh:hh + 1], gb[b:b + 1, hh:hh + 1], [T],
                                  w.top_k)
        assert np.array_equal(sel[b, hh].cpu().numpy(), ri[0, 0]) and cnt[b, hh].item() == w.top_k
        ref, _, _ = O.decode_attention(codec, qn[b:b + 1, hh:hh + 1], rec[b:b + 1, hh:hh + 1].cpu().numpy(), [T],
                                       sel_idx=ri)
        _close(out[b, hh].cpu().numpy(), ref[0, 0], f"sparse out[{b},{hh}]")


def test_bulk_scan_full_size_sampled():
    w = W.WORKLOADS["bulk_64k_scan"]
    h = _handle(w)
    codec = _codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = _compress(w, h, K, V)
    q = W.make_queries(w, "cuda")
    sc = h.score_scan(q, rec, w.tokens)
    torch.cuda.synchronize()
    for hh, qi in [(0, 0), (4, 200), (7, 255)]:
        ref = O.score_scan(codec, _np(q[:, hh:hh + 1, qi:qi + 1]), rec[:, hh:hh + 1].cpu().numpy(), w.tokens)
        _close(sc[0, hh, qi].cpu().numpy(), ref[0, 0, 0], f"scan[{hh},{qi}]")
    r = rec[0, 2].cpu().numpy()
    toks = np.r_[0:100, 65000:65536]
    check_compress(codec, _np(K[0, toks, 2]), _np(V[0, toks, 2]), r[toks])
