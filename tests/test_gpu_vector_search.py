"""GPU parity of compression and the bulk scan at head_dim 200 (the GloVe d=200 shape of the
TurboQuant page's vector-search section) and of the 1@k recall they give.

* compress end to end: the scalar codec's rule (norms within 1e-6 relative, codes and QJL
  bits exact except at a boundary / zero), through the generic (non-matrix-core) kernel;
* scan: every estimate within 1e-4 + 1e-3 |oracle|;
* recall: 1@k recall from the GPU scores equals the recall from the oracle's scores up to
  queries whose exact best sits on a near-tie of the approximate ranking (at most 1 of 64).
"""
import numpy as np
import pytest
import torch

import test_gpu_parity as GP
from compressed_key_attention_amd import workloads as W
from oracle import tq_oracle as O

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["vector_search_d200"]


def _wl(kb=2, m=192, vb=2, tokens=3000, nq=64, d=200, dt="f32"):
    return W.Workload("vector_search_d200", 1, 1, 1, d, tokens, 0, kb, m, vb, dt, dt,
                      scan_queries=nq, seed=BASE.seed)


@pytest.mark.parametrize("kb,m,vb,dt,d", [(2, 192, 2, "f32", 200), (3, 0, 4, "bf16", 200), (4, 32, 3, "f16", 200),
                                           (3, 256, 2, "f32", 200), (3, 32, 4, "f32", 40), (4, 256, 4, "bf16", 256)])
def test_compress_head_dim_200(kb, m, vb, dt, d):
    print(f"[case] d={d} compress kb={kb} m={m} vb={vb} {dt}", flush=True)
    w = _wl(kb, m, vb, tokens=77, dt=dt, d=d)
    h = GP._handle(w)
    codec = GP._codec(h)
    assert h.record_bytes == codec.record_bytes
    K, V = W.make_kv(w, "cuda")
    rec = GP._compress(w, h, K, V).cpu().numpy()
    stats = GP.check_compress(codec, GP._np(K[0, :, 0]), GP._np(V[0, :, 0]), rec[0, 0])
    print(f"[compress] exempt mismatches {stats}", flush=True)


def _scan(w, h, rec, q, n_tokens):
    scores = torch.full((w.batch, w.kv_heads, w.scan_queries, n_tokens), float("nan"), device="cuda")
    h.score_scan(q, rec, n_tokens, scores)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


@pytest.mark.parametrize("kb,m,vb,d", [(2, 192, 2, 200), (3, 0, 4, 200), (4, 32, 3, 200), (3, 256, 4, 128),
                                        (3, 32, 4, 40), (4, 256, 4, 256)])
def test_scan_head_dim_200_and_long_contractions(kb, m, vb, d):
    print(f"[case] scan d={d} kb={kb} m={m}", flush=True)
    w = _wl(kb, m, vb, tokens=1000, nq=70, d=d)
    h = GP._handle(w)
    codec = GP._codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = GP._compress(w, h, K, V)
    q = W.make_queries(w, "cuda")
    got = _scan(w, h, rec, q, 997)
    ref = O.score_scan(codec, GP._np(q), rec.cpu().numpy(), 997)
    GP._close(got, ref, "scan estimates")


def test_recall_from_gpu_scan_matches_oracle():
    print("[case] recall d=200", flush=True)
    w = _wl(tokens=4096, nq=64)
    h = GP._handle(w)
    codec = GP._codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = GP._compress(w, h, K, V)
    q = W.make_queries(w, "cuda")
    got = _scan(w, h, rec, q, w.tokens)[0, 0]
    ref = O.score_scan(codec, GP._np(q), rec.cpu().numpy(), w.tokens)[0, 0]
    exact = GP._np(q)[0, 0].astype(np.float64) @ GP._np(K)[0, :, 0].astype(np.float64).T
    ks = [1, 2, 4, 8, 16, 32, 64]
    rg = O.recall_1_at_k(got, exact, ks)
    rr = O.recall_1_at_k(ref, exact, ks)
    print(f"[recall] gpu {rg} oracle {rr}", flush=True)
    for k in ks:
        assert abs(rg[k] - rr[k]) <= 1 / 64 + 1e-12, (k, rg[k], rr[k])
    assert rg[64] >= rg[1] and rr[64] > 0.5


def test_head_dim_200_rejected_where_not_built():
    """The hot/cold step is built for head_dim 64 and 128 only."""
    tq = GP._tq()
    h = GP._handle(_wl(tokens=16))
    with pytest.raises(tq.TqError) as e:
        tq.monarch_workspace_size(h, 1, 1, 1, 8, 8)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED


def test_vector_search_full_size_sampled():
    """The benchmark's workload at full size (100,000 vectors, 1,000 queries, the launch the
    benchmark times): sampled compress records and sampled scores against the oracle, and
    the recall of every query against exact inner products on a sampled block."""
    print("[case] vector search full size", flush=True)
    w = BASE
    h = GP._handle(w)
    codec = GP._codec(h)
    K, V = W.make_kv(w, "cuda")
    rec = GP._compress(w, h, K, V)
    toks = np.r_[0:64, 49_980:50_020, 99_936:100_000]
    r = rec[0, 0].cpu().numpy()
    GP.check_compress(codec, GP._np(K[0, toks, 0]), GP._np(V[0, toks, 0]), r[toks])
    q = W.make_queries(w, "cuda")
    scores = torch.full((1, 1, w.scan_queries, w.tokens), float("nan"), device="cuda")
    h.score_scan(q, rec, w.tokens, scores)
    torch.cuda.synchronize()
    qs = [0, 1, 499, 998, 999]
    blk = np.r_[0:2048, 97_952:100_000]
    ref = O.score_scan(codec, GP._np(q[:, :, qs]), r[None, None, blk], len(blk))[0, 0]
    GP._close(scores[0, 0, qs][:, blk].cpu().numpy(), ref, "sampled scan estimates")
    assert not torch.isnan(scores).any()
