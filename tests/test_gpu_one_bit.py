"""1-bit stage-1 codes (TurboQuant page, "Funktionsweise von TurboQuant", step 1 at its smallest
width: the two-level Lloyd-Max code +-sqrt(2/pi) for N(0, 1)) through every entry point, against
the oracle with the rules of test_gpu_parity: records bit-exact from given rotated inputs,
compress end to end with the boundary exemption, decode / sparse attention / bulk scan within
1e-4 + 1e-3 |oracle|, selection bit-exact."""
import numpy as np
import pytest
import torch

import test_gpu_parity as GP
from compressed_key_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [(64, 1, 64, 1), (128, 1, 0, 4), (128, 4, 32, 1), (128, 1, 128, 1)])
def test_one_bit_packing_is_bit_exact(cfg):
    GP.test_debug_quantize_is_bit_exact(cfg)


@pytest.mark.parametrize("name,kb,vb,tokens,batch", [("llama8b_decode_32k", 1, 1, 1000, 2),
                                                     ("tinyllama_layer", 1, 2, 700, 1),
                                                     ("single_head_1k", 4, 1, 1024, 1)])
def test_one_bit_compress_end_to_end(name, kb, vb, tokens, batch):
    base = W.small(W.WORKLOADS[name], tokens=tokens, batch=batch)
    w = W.Workload(**{**base.__dict__, "key_bits": kb, "value_bits": vb})
    h = GP._handle(w)
    codec = GP._codec(h)
    K, V = W.make_kv(w, "cpu")
    rec = GP._compress(w, h, K.cuda(), V.cuda()).cpu().numpy()
    Kn, Vn = GP._np(K), GP._np(V)
    for b in range(w.batch):
        for hh in range(w.kv_heads):
            GP.check_compress(codec, Kn[b, :, hh], Vn[b, :, hh], rec[b, hh])


@pytest.mark.parametrize("d,kb,vb,m,hq,tokens,lens", [
    (64, 1, 1, 64, 32, 900, [900, 333]),       # short cache, 8 query heads per KV head: direct kernel
    (128, 1, 4, 128, 8, 2000, [2000, 1999]),   # one query head per KV head: LUT kernel, code-pair tables
    (128, 1, 1, 0, 32, 5000, [5000, 4097]),    # 4 query heads per KV head, long cache: LUT kernel, 4 heads per lane
    (128, 4, 1, 128, 64, 600, [600, 1]),       # 1-bit values only
])
def test_one_bit_decode(d, kb, vb, m, hq, tokens, lens):
    base = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=tokens, batch=len(lens))
    w = W.Workload(**{**base.__dict__, "head_dim": d, "key_bits": kb, "value_bits": vb, "qjl_dim": m,
                      "q_heads": hq})
    GP._decode_case(w, lens)


def test_one_bit_decode_with_exact_segment_and_gather():
    base = W.small(W.WORKLOADS["tinyllama_layer"], tokens=800, batch=2, hot_tokens=64)
    w = W.Workload(**{**base.__dict__, "key_bits": 1, "value_bits": 1})
    GP._decode_case(w, [800, 500], hot_lens=[64, 3])
    rng = np.random.default_rng(11)
    sel = np.full((2, w.kv_heads, 100), -1, np.int32)
    for b in range(2):
        for hh in range(w.kv_heads):
            k = rng.integers(1, 100)
            sel[b, hh, :k] = np.sort(rng.choice(800, size=k, replace=False))
    GP._decode_case(w, [800, 800], sel=torch.from_numpy(sel).cuda())


@pytest.mark.parametrize("kb,vb,m,hq,k,lens,sinks", [(1, 1, 0, 8, 300, [5000, 4097], 0),
                                                     (1, 4, 64, 16, 200, [3000, 2000], 16)])
def test_one_bit_sparse_attention(kb, vb, m, hq, k, lens, sinks):
    GP.test_sparse_attention_one_call(kb, vb, m, hq, k, lens, sinks, 0, 128)


@pytest.mark.parametrize("kb,m,d,nq,T,n_tok", [(1, 128, 128, 20, 700, 700), (1, 0, 64, 9, 300, 257)])
def test_one_bit_bulk_scan(kb, m, d, nq, T, n_tok):
    GP.test_score_scan_variants(kb, m, d, nq, T, n_tok)
