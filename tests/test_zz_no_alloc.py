"""tq_decode_attention_noalloc (the decode with the library's fixed device scratch instead of a
workspace) against tq_decode_attention on the same inputs: two calls in a row, the second
smaller, then a call on another handle with an exact segment; outputs, lse and logits must be
identical (the two share their kernels, and nothing in the scratch carries over between
calls).  A decode whose workspace exceeds the fixed scratch is rejected with nothing written."""
import ctypes

import numpy as np
import pytest
import torch

from compressed_key_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20


def _tq():
    import compressed_key_attention_amd as tq
    return tq


def _handle(w):
    return _tq().Handle(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2)


def _same(a, b, what):
    a, b = a.cpu().numpy(), b.cpu().numpy()
    assert np.array_equal(a, b, equal_nan=True), f"{what}: allocation-free decode differs"


def _both(h, q, rec, lens, hot=None):
    B, Hq, d = q.shape
    N = rec.shape[2] + (0 if hot is None else hot["hot_k"].shape[2])
    res = []
    for noalloc in (False, True):
        out = torch.full((B, Hq, d), float("nan"), device="cuda")
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        logits = torch.full((B, Hq, N), float("nan"), device="cuda")
        if noalloc:
            h.decode_attention_noalloc(q, rec, lens, out, lse=lse, logits=logits, **(hot or {}))
        else:
            h.decode_attention(q, rec, lens, out=out, lse=lse, logits=logits, **(hot or {}))
        torch.cuda.synchronize()
        res.append((out, lse, logits))
    for (a, b, what) in zip(res[0], res[1], ("out", "lse", "logits")):
        _same(a, b, what)
    assert torch.isfinite(res[1][0]).all()


def test_noalloc_decode_matches_the_workspace_decode():
    print("[case] allocation-free decode: llama8b shape, 4 x 6,000 tokens then 2 x 1,500", flush=True)
    w = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=6000, batch=4)
    h = _handle(w)
    assert h.decode_workspace_size(w.batch, w.q_heads, w.kv_heads, w.tokens) <= SCRATCH
    K, V = W.make_kv(w, "cuda")
    rec = h.new_cache(w.batch, w.kv_heads, w.tokens, "cuda")
    h.compress_kv(K, V, rec)
    q = W.make_queries(w, "cuda")
    _both(h, q, rec, torch.tensor([6000, 5999, 4097, 1], dtype=torch.int32, device="cuda"))
    # a smaller second call: the scratch still holds the first call's partials
    rec2 = rec[:2, :, :1500].contiguous()
    _both(h, q[:2].contiguous(), rec2, torch.tensor([1500, 333], dtype=torch.int32, device="cuda"))

    print("[case] allocation-free decode: tinyllama shape with an exact segment", flush=True)
    w3 = W.small(W.WORKLOADS["tinyllama_layer"], tokens=700, batch=2, hot_tokens=100)
    h3 = _handle(w3)
    K3, V3 = W.make_kv(w3, "cuda")
    rec3 = h3.new_cache(w3.batch, w3.kv_heads, w3.tokens, "cuda")
    h3.compress_kv(K3, V3, rec3)
    hk, hv = W.make_hot(w3, "cuda")
    hot = dict(hot_k=hk, hot_v=hv, hot_lens=torch.tensor([100, 37], dtype=torch.int32, device="cuda"))
    _both(h3, W.make_queries(w3, "cuda"), rec3, torch.tensor([700, 512], dtype=torch.int32, device="cuda"), hot)


def test_noalloc_decode_rejects_a_workspace_beyond_the_fixed_scratch():
    tq = _tq()
    w = W.WORKLOADS["llama8b_decode_32k"]
    h = _handle(w)
    B, cap = 256, 1 << 20
    need = h.decode_workspace_size(B, w.q_heads, w.kv_heads, cap)
    assert need > SCRATCH
    q = torch.zeros((B, w.q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    rec = torch.zeros((1, 1, 1, h.record_bytes), dtype=torch.uint8, device="cuda")   # never read
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.full((B, w.q_heads, w.head_dim), float("nan"), device="cuda")
    st = tq._decode_noalloc(h._h, q.data_ptr(), tq.TQ_BF16, B, w.q_heads, w.kv_heads, rec.data_ptr(), cap,
                            lens.data_ptr(), None, None, tq.TQ_F32, None, 0, None, 0, 0.0, out.data_ptr(), None,
                            None, None)
    assert st == tq.TQ_ERR_WORKSPACE_TOO_SMALL, st
    assert "fixed device scratch" in tq.last_error()
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "a rejected call wrote its output"
