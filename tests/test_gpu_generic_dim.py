"""GPU parity of tq_debug_quantize, decode attention, the sign index, top-k selection and sparse
attention at head dims other than 64 and 128 (any multiple of 8 up to 256: the TurboQuant page's vector-search
section uses d = 200), through the direct kernels that read d at run time, against the oracle
with the rules of test_gpu_parity: outputs, lse and every logit within 1e-4 + 1e-3 |oracle|;
sign index bit-exact at the GPU's channel mean; selected sets and scores bit-exact."""
import numpy as np
import pytest
import torch

import test_gpu_parity as GP
from compressed_key_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _wl(d, kb, m, vb, hq, hkv, tokens, batch, hot=0):
    base = W.small(W.WORKLOADS["llama8b_decode_32k"], tokens=tokens, batch=batch, hot_tokens=hot)
    return W.Workload(**{**base.__dict__, "head_dim": d, "key_bits": kb, "qjl_dim": m, "value_bits": vb,
                         "q_heads": hq, "kv_heads": hkv})


@pytest.mark.parametrize("cfg", [(200, 3, 192, 2), (200, 2, 96, 3), (40, 3, 32, 4), (200, 1, 64, 1), (104, 4, 0, 3)])
def test_debug_quantize_generic_head_dim(cfg):
    """Records from given rotated coordinates, byte for byte: the partial 3-bit group of d = 200
    and 40, the zero pad of fields that are not whole words (d = 200 at 2 bits: 50 + 2 bytes)."""
    GP.test_debug_quantize_is_bit_exact(cfg)


@pytest.mark.parametrize("d,kb,m,vb,hq,hkv,lens,hot", [
    (200, 2, 192, 2, 4, 4, [3000, 1234], None),       # the vector-search codec, one head per KV head
    (200, 3, 0, 4, 16, 4, [700, 65], [37, 0]),        # 3-bit keys (partial 3-bit group), exact tokens
    (40, 3, 32, 4, 8, 1, [1000, 999], None),          # d = 40: one whole 3-bit group + 8 codes
    (256, 4, 256, 4, 4, 2, [5000, 4097], [3, 2100]),  # the largest d and sketch; exact segment > 2048
    (96, 1, 64, 1, 2, 2, [300, 0], None),             # 1-bit codes; an empty sequence
])
def test_decode_generic_head_dim(d, kb, m, vb, hq, hkv, lens, hot):
    w = _wl(d, kb, m, vb, hq, hkv, max(lens), len(lens), hot=max(hot) if hot else 0)
    GP._decode_case(w, lens, hot_lens=hot)


def test_decode_generic_head_dim_gather():
    w = _wl(200, 3, 64, 4, 8, 2, 900, 2)
    rng = np.random.default_rng(5)
    sel = np.full((2, 2, 130), -1, np.int32)
    for b in range(2):
        for h in range(2):
            k = int(rng.integers(1, 130))
            sel[b, h, :k] = np.sort(rng.choice(900, size=k, replace=False))
    GP._decode_case(w, [900, 900], sel=torch.from_numpy(sel).cuda())


@pytest.mark.parametrize("d,hq,lens,k", [(200, 8, [9000, 4097], 700), (40, 16, [3000, 2999], 64),
                                         (256, 8, [5000, 100], 5000)])
def test_sign_index_and_topk_generic_head_dim(d, hq, lens, k):
    base = W.small(W.WORKLOADS["sparse_128k_top2048"], tokens=max(lens), batch=len(lens))
    w = W.Workload(**{**base.__dict__, "head_dim": d})
    GP._index_case(w, lens, k, q_heads=hq)


@pytest.mark.parametrize("kb,vb,m,hq,k,lens,sinks,d", [
    (4, 4, 0, 8, 300, [5000, 4097], 0, 200),
    (2, 2, 192, 16, 900, [9000, 123], 64, 200),
    (3, 4, 32, 8, 2000, [2500, 2500], 16, 40),
])
def test_sparse_attention_generic_head_dim(kb, vb, m, hq, k, lens, sinks, d):
    GP.test_sparse_attention_one_call(kb, vb, m, hq, k, lens, sinks, 0, d)
