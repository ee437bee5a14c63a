"""GPU parity against the scalar C oracle (oracle/tq_scalar.c), at the sizes the benchmark times.

The same rules as the numpy-oracle parity tests:
* compress end to end: records byte-identical except that a code may differ where the oracle's
  rotated coordinate lies within 1e-6 of a codebook boundary, and a sign bit where the oracle's
  projection (recomputed from the GPU's own codes) is within 1e-6 |residual| of zero;
* attention outputs, lse and logits within 1e-4 + 1e-3 |oracle|, the GPU accumulating in fp32;
* sign index bit-exact at the GPU's channel mean (the mean itself within one float32 ulp), top-k
  sets and scores bit-exact.

Covered: every config family's compress (single_head_1k, tinyllama_layer, two whole sequences
of llama8b_decode_32k, the 4-bit payload of sparse_128k_top2048, the whole bulk_64k_scan
cache, vector_search_d200); the decode of single_head_1k and tinyllama_layer (512 exact
tokens) and of llama8b_decode_32k at full size, every head and every logit; the 131,072-token
sign index, top-2,048 and one-call sparse attention for all 32 units; bulk-scan rows at full
size.  The C oracle runs on host threads (ctypes releases the GIL during its calls).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import test_gpu_parity as GP
from compressed_key_attention_amd import workloads as W
from oracle import scalar as S

pytestmark = pytest.mark.gpu

_CODECS = {}


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _threads():
    return 16


def _pmap(fn, jobs):
    jobs = list(jobs)
    with ThreadPoolExecutor(max_workers=min(_threads(), max(1, len(jobs)))) as ex:
        return list(ex.map(fn, jobs))


def _codec(w):
    key = (w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2)
    if key not in _CODECS:
        _CODECS[key] = S.ScalarCodec(*key)
    return _CODECS[key]


def check_compress(c, K, V, rec_gpu):
    """K, V [n, d] float32, rec_gpu [n, R]: the end-to-end compress rule against the C oracle."""
    ref = c.compress(K, V)
    same = np.all(rec_gpu == ref, axis=1)
    if same.all():
        return 0
    t = c.tables()
    fg, fr = c.unpack(rec_gpu[~same]), c.unpack(ref[~same])
    Kd, Vd = K[~same], V[~same]
    for key in ("r_k", "r_v"):
        assert np.array_equal(fg[key], fr[key]), key
    for which, X, bounds, is_v in (("kc", Kd, t["key_bounds"], False), ("vc", Vd, t["val_bounds"], True)):
        mism = fg[which] != fr[which]
        if mism.any():
            z, _ = c.rotated(X, is_value=is_v)
            dist = np.min(np.abs(z[..., None].astype(np.float64) - bounds.astype(np.float64)), axis=-1)
            assert np.all(dist[mism] <= 1e-6), f"{which}: a code differs away from a boundary"
    if c.qjl_dim:
        rho, p = c.residual(Kd, fg["kc"], fg["r_k"])
        assert np.allclose(fg["rho"], rho.astype(np.float32), rtol=2e-6, atol=1e-30), "rho"
        mism = (fg["bits"] == 1) != (p.astype(np.float32) >= 0)
        if mism.any():
            rel = np.abs(p) / np.maximum(rho, 1e-300)[:, None]
            assert np.all(rel[mism] <= 1e-6), "a sign bit differs away from zero"
    return int((~same).sum())


def _f32(x):
    return x.detach().float().cpu().numpy()


# ------------------------------------------------------------------ compress --------------
@pytest.mark.parametrize("name,tokens,batch", [
    ("single_head_1k", None, None), ("tinyllama_layer", None, None), ("llama8b_decode_32k", None, 2),
    ("sparse_128k_top2048", 16384, 1), ("bulk_64k_scan", None, None), ("vector_search_d200", 20000, None)])
def test_compress_against_the_scalar_oracle(name, tokens, batch):
    w = W.WORKLOADS[name]
    _case(f"compress {name} tokens={tokens or w.tokens} batch={batch or w.batch}")
    K, V = W.make_kv(w, "cuda", tokens=tokens, batch=batch)
    h = GP._handle(w)
    rec = GP._compress(w, h, K, V).cpu().numpy()
    Kn, Vn = _f32(K), _f32(V)
    c = _codec(w)
    B, T, H, d = K.shape
    jobs = [(b, hh) for b in range(B) for hh in range(H)]
    diffs = _pmap(lambda u: check_compress(c, Kn[u[0], :, u[1]], Vn[u[0], :, u[1]], rec[u[0], u[1]]), jobs)
    print(f"[compress] {name}: {sum(diffs)} of {B * H * T} records differ at a boundary", flush=True)


# ------------------------------------------------------------------ decode ----------------
def _decode_against_c(w, seq_lens, hot=False, sample_heads=None):
    h = GP._handle(w)
    c = _codec(w)
    K, V = W.make_kv(w, "cuda")
    rec = h.new_cache(w.batch, w.kv_heads, w.tokens, "cuda")
    h.compress_kv(K, V, rec)
    del K, V
    q = W.make_queries(w, "cuda")
    B, Hq, d, N = w.batch, w.q_heads, w.head_dim, w.tokens
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    hk = hv = hl = None
    nh = 0
    if hot:
        hk, hv = W.make_hot(w, "cuda")
        nh = hk.shape[2]
        hl = torch.full((B,), nh, dtype=torch.int32, device="cuda")
    ws = torch.empty(h.decode_workspace_size(B, Hq, w.kv_heads, N), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    logits = torch.full((B, Hq, N + nh), float("nan"), device="cuda")
    h.decode_attention(q, rec, sl, hot_k=hk, hot_v=hv, hot_lens=hl, out=out, lse=lse, workspace=ws)
    out2 = torch.full((B, Hq, d), float("nan"), device="cuda")
    h.decode_attention(q, rec, sl, hot_k=hk, hot_v=hv, hot_lens=hl, out=out2, logits=logits, workspace=ws)
    torch.cuda.synchronize()
    r, qn = rec.cpu().numpy(), _f32(q)
    hkn = _f32(hk) if hot else None
    hvn = _f32(hv) if hot else None
    G = Hq // w.kv_heads
    units = [(b, hq) for b in range(B) for hq in range(Hq)] if sample_heads is None else sample_heads

    def one(u):
        b, hq = u
        g = hq // G
        return c.decode_head(qn[b, hq], r[b, g], seq_lens[b], None,
                             None if not hot else hkn[b, g], None if not hot else hvn[b, g],
                             0.0, want_logits=True)

    _case(f"{w.name}: scalar oracle over {len(units)} heads")
    res = _pmap(one, units)
    o, L, o2, lg = out.cpu().numpy(), lse.cpu().numpy(), out2.cpu().numpy(), logits.cpu().numpy()
    ref_o = np.stack([x[0] for x in res])
    ref_l = np.array([x[1] for x in res])
    sel_o = np.stack([o[b, hq] for b, hq in units])
    GP._close(sel_o, ref_o, f"{w.name}: out, {len(units)} heads")
    GP._close(np.stack([o2[b, hq] for b, hq in units]), ref_o, f"{w.name}: out (logits run)")
    GP._close(np.array([L[b, hq] for b, hq in units]), ref_l, f"{w.name}: lse")
    ref_lg = np.concatenate([x[2] for x in res])
    got_lg = np.concatenate([np.concatenate([lg[b, hq, :seq_lens[b]], lg[b, hq, N:N + nh]]) for b, hq in units])
    GP._close(got_lg, ref_lg, f"{w.name}: all {got_lg.size} logits (cold, then exact)")


def test_decode_single_head_1k_against_the_scalar_oracle():
    _decode_against_c(W.WORKLOADS["single_head_1k"], [1024])


def test_decode_tinyllama_layer_with_exact_tokens_against_the_scalar_oracle():
    _decode_against_c(W.WORKLOADS["tinyllama_layer"], [1024], hot=True)


def test_decode_llama8b_full_size_every_head_against_the_scalar_oracle():
    w = W.WORKLOADS["llama8b_decode_32k"]
    _decode_against_c(w, [w.tokens] * w.batch)


# ------------------------------------------------------------------ sparse ----------------
def test_sparse_128k_full_size_against_the_scalar_oracle():
    w = W.WORKLOADS["sparse_128k_top2048"]
    _case("sparse_128k_top2048 at full size: sign index, select, one-call sparse attention")
    h = GP._handle(w)
    c = _codec(w)
    K, V = W.make_kv(w, "cuda")
    B, T, H, d = K.shape
    G, k = w.q_heads // H, w.top_k
    index = torch.full((B, H, T, d // 8), 0xEE, dtype=torch.uint8, device="cuda")
    book = torch.full((B, H, d // 4, 16, 4), float("nan"), device="cuda")
    mean = torch.full((B, H, d), float("nan"), device="cuda")
    h.build_sign_index(K, index, book, mean)
    rec = h.new_cache(B, H, T, "cuda")
    h.compress_kv(K, V, rec)
    Kn = _f32(K)
    del K, V
    q = W.make_queries(w, "cuda")
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    pws = torch.empty(h.sparse_workspace_size(B, w.q_heads, H, T), dtype=torch.uint8, device="cuda")
    out = torch.full((B, w.q_heads, d), float("nan"), device="cuda")
    lse = torch.full((B, w.q_heads), float("nan"), device="cuda")
    h.sparse_attention(q, index, book, rec, sl, k, out=out, lse=lse, workspace=pws)
    sel = torch.full((B, H, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
    scs = torch.full((B, H, k), -7, dtype=torch.int32, device="cuda")
    h.select_topk(q, index, book, sl, k, out_idx=sel, out_count=cnt, out_scores=scs)
    torch.cuda.synchronize()
    gi, gb, mu = index.cpu().numpy(), book.cpu().numpy(), mean.cpu().numpy()
    qn, r = _f32(q), rec.cpu().numpy()
    si, sc, cn = sel.cpu().numpy(), scs.cpu().numpy(), cnt.cpu().numpy()
    units = [(b, hh) for b in range(B) for hh in range(H)]

    def one(u):
        b, hh = u
        kf = np.ascontiguousarray(Kn[b, :, hh])
        rmu = S.channel_mean(kf)
        ulp = np.spacing(np.abs(rmu)).astype(np.float64)
        assert np.all(np.abs(mu[b, hh].astype(np.float64) - rmu) <= ulp), f"unit {u}: channel mean"
        ri, rb = S.sign_index(kf, mu[b, hh])                 # the oracle's steps at the GPU's mean
        assert np.array_equal(gi[b, hh], ri), f"unit {u}: index at the GPU's mean"
        np.testing.assert_allclose(gb[b, hh], rb, rtol=2.4e-7, atol=1e-12, err_msg=f"unit {u}: codebook")
        idx, n_sel, scores = S.select_unit(qn[b, hh * G:(hh + 1) * G], gi[b, hh], gb[b, hh], T, k)
        outs = [c.decode_head(qn[b, hh * G + j], r[b, hh], n_sel, idx[:n_sel]) for j in range(G)]
        return idx, n_sel, scores, outs

    res = _pmap(one, units)
    o, L = out.cpu().numpy(), lse.cpu().numpy()
    ref_o = np.zeros_like(o, dtype=np.float64)
    ref_l = np.zeros_like(L, dtype=np.float64)
    for (b, hh), (ri, rc, rs, outs) in zip(units, res):
        assert rc == k and cn[b, hh] == k, f"unit {(b, hh)}: count"
        assert np.array_equal(si[b, hh], ri), f"unit {(b, hh)}: selected set"
        assert np.array_equal(sc[b, hh], rs), f"unit {(b, hh)}: selected scores"
        for j, (oo, ll, _) in enumerate(outs):
            ref_o[b, hh * G + j], ref_l[b, hh * G + j] = oo, ll
    GP._close(o, ref_o, "sparse attention (one call), all 32 units")
    GP._close(L, ref_l, "sparse attention lse, all 32 units")


# ------------------------------------------------------------------ bulk scan -------------
def test_bulk_scan_full_size_rows_against_the_scalar_oracle():
    w = W.WORKLOADS["bulk_64k_scan"]
    _case("bulk_64k_scan at full size: 16 query rows per KV head")
    h = GP._handle(w)
    c = _codec(w)
    K, V = W.make_kv(w, "cuda")
    rec = h.new_cache(1, w.kv_heads, w.tokens, "cuda")
    h.compress_kv(K, V, rec)
    del K, V
    q = W.make_queries(w, "cuda")
    sc = h.score_scan(q, rec, w.tokens)
    torch.cuda.synchronize()
    r, qn = rec.cpu().numpy(), _f32(q)
    rows = np.r_[0:8, 248:256]
    res = _pmap(lambda hh: c.score_scan(qn[:, hh:hh + 1, rows], r[:, hh:hh + 1], w.tokens), range(w.kv_heads))
    got = sc[0][:, rows].cpu().numpy()
    GP._close(got, np.concatenate([x[0] for x in res]), "bulk scan rows, all tokens")
