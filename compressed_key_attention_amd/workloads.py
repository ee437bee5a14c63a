"""Seeded synthetic workloads shared by the tests, the benchmark and smoke().

This module only draws random tensors: it holds none of the codec's arithmetic
(no rotation, quantizer, estimator or attention).  Both the HIP path and the
oracle are fed the very same tensors produced here.

Shapes and value distributions follow the workloads the pages describe:

* ``single_head_1k`` - one head, head_dim 128, 1,024 cached tokens, fp32 keys,
  values and query drawn i.i.d. N(0, 1).
* ``tinyllama_layer`` - a TinyLlama-1.1B-shaped decode layer (32 query heads,
  4 KV heads, head_dim 64, batch 1) with 1,024 compressed (cold) tokens and 512
  exact fp16 (hot) tokens, as in the Monarch v3 benchmark set-up (Monarch v3
  page, "Benchmark-Ergebnisse").  K/V are N(0, 1) with two seeded outlier
  channels scaled by 8 (the same two channels for every head, token, K and V).
* ``llama8b_decode_32k`` - Llama-3-8B-shaped decode: 32 query heads, 8 KV heads,
  head_dim 128, batch 16, 32,768 cached tokens per sequence; K/V i.i.d.
  Student-t with 4 degrees of freedom rounded to bf16; bf16 N(0, 1) queries.
  It stands in for the long-context LLM evaluations the TurboQuant and
  Self-Indexing pages report (no dataset or weights are used).
* ``sparse_128k_top2048`` - 8 KV heads (= 8 query heads), head_dim 128, batch 4,
  131,072 tokens, top-2048 selection; bf16 N(0, 1) K, V and queries.
* ``llama8b_decode_32k_polar`` - the llama8b_decode_32k shapes and distributions with
  polar key codes (4-bit level-1 angles, 2-bit higher angles: 48 key bytes, as 3-bit
  scalar codes) - the PolarQuant variant of stage 1 on the TurboQuant page.
* ``vector_search_d200`` - 100,000 database vectors and 1,000 queries of dimension 200
  (the GloVe d=200 shape of the TurboQuant page's vector-search section; GloVe itself is not
  used): every vector and query is mu + sigma * N(0, I) with seeded per-channel mean
  mu_i ~ 0.3 N(0, 1) and scale sigma_i = exp(0.4 N(0, 1)), i.e. dense embeddings with a
  shared offset and uneven channel energy.  2-bit codes plus a 192-bit QJL sketch (about 3
  bits per coordinate); the bulk scan scores every query against every vector.
* ``bulk_64k_scan`` - 65,536 tokens x 8 KV heads x head_dim 128 in bf16, N(0, 1)
  except 10 seeded (head, channel) pairs whose entries are 20 * t4; 256 bf16
  N(0, 1) queries per KV head score the whole compressed cache.  It stands in
  for the vector-search workload of the TurboQuant page (GloVe is not used).

Student-t(4) is drawn as Z / sqrt(C / 4) with C = -2 (ln U1 + ln U2), which is
chi-square with 4 degrees of freedom (sum of two exponentials of mean 2).
"""
from __future__ import annotations

import dataclasses

import torch

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int            # sequences
    q_heads: int
    kv_heads: int
    head_dim: int
    tokens: int           # compressed (cold) tokens per sequence
    hot_tokens: int       # exact tokens per sequence (0 = none)
    key_bits: int
    qjl_dim: int
    value_bits: int
    kv_dtype: str
    q_dtype: str
    top_k: int = 0        # > 0: sparse decode over the top-k tokens
    scan_queries: int = 0  # > 0: bulk scan with this many queries per KV head
    seed: int = 0
    polar_upper_bits: int = 0  # > 0: polar key codes (key_bits = level-1 angle bits)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


WORKLOADS = {
    "single_head_1k": Workload("single_head_1k", 1, 1, 1, 128, 1024, 0, 3, 128, 4,
                               "f32", "f32", seed=101),
    "tinyllama_layer": Workload("tinyllama_layer", 1, 32, 4, 64, 1024, 512, 3, 64, 4,
                                "f16", "f16", seed=202),
    "llama8b_decode_32k": Workload("llama8b_decode_32k", 16, 32, 8, 128, 32768, 0, 3, 128, 4,
                                   "bf16", "bf16", seed=303),
    "sparse_128k_top2048": Workload("sparse_128k_top2048", 4, 8, 8, 128, 131072, 0, 4, 0, 4,
                                    "bf16", "bf16", top_k=2048, seed=404),
    "bulk_64k_scan": Workload("bulk_64k_scan", 1, 8, 8, 128, 65536, 0, 3, 128, 4,
                              "bf16", "bf16", scan_queries=256, seed=505),
    "vector_search_d200": Workload("vector_search_d200", 1, 1, 1, 200, 100000, 0, 2, 192, 2,
                                   "f32", "f32", scan_queries=1000, seed=707),
    "llama8b_decode_32k_polar": Workload("llama8b_decode_32k_polar", 16, 32, 8, 128, 32768, 0, 4, 128, 4,
                                         "bf16", "bf16", seed=606, polar_upper_bits=2),
}


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def student_t4(shape, gen, device) -> torch.Tensor:
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    u1 = 1.0 - torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    u2 = 1.0 - torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    chi2 = -2.0 * (torch.log(u1) + torch.log(u2))
    return z / torch.sqrt(chi2 / 4.0)


def make_kv(w: Workload, device="cpu", tokens: int | None = None, batch: int | None = None,
            seed_offset: int = 0):
    """Keys and values ``[batch, tokens, kv_heads, head_dim]`` in the workload dtype.

    Generated one sequence at a time so that large caches need little scratch memory.
    """
    T = w.tokens if tokens is None else tokens
    B = w.batch if batch is None else batch
    dt = _DT[w.kv_dtype]
    shape = (T, w.kv_heads, w.head_dim)
    gsel = generator(w.seed * 7919 + 17 + seed_offset, "cpu")
    if w.name == "vector_search_d200":
        mu, sigma = embedding_channels(w)
    if w.name == "tinyllama_layer":
        outlier = torch.randperm(w.head_dim, generator=gsel)[:2]
    elif w.name == "bulk_64k_scan":
        outlier = torch.randperm(w.kv_heads * w.head_dim, generator=gsel)[:10]
    else:
        outlier = None
    K = torch.empty((B,) + shape, dtype=dt, device=device)
    V = torch.empty((B,) + shape, dtype=dt, device=device)
    for b in range(B):
        for X, which in ((K, 0), (V, 1)):
            g = generator(w.seed * 1_000_003 + 2 * b + which + seed_offset, device)
            if w.name in ("llama8b_decode_32k", "llama8b_decode_32k_polar"):
                x = student_t4(shape, g, device)
            elif w.name == "vector_search_d200":
                x = mu.to(device) + sigma.to(device) * normal(shape, g, device)
            elif w.name == "bulk_64k_scan":
                x = normal(shape, g, device)
                t = 20.0 * student_t4((T, len(outlier)), g, device)
                flat = x.view(T, -1)
                flat[:, outlier.to(device)] = t
            else:
                x = normal(shape, g, device)
                if outlier is not None:
                    x[..., outlier.to(device)] *= 8.0
            X[b].copy_(x.to(dt))
    return K, V


def embedding_channels(w: Workload):
    """Per-channel mean and scale of the embedding-like vectors (CPU float32 [head_dim])."""
    g = generator(w.seed * 104729 + 3, "cpu")
    z = torch.randn((2, w.head_dim), generator=g, dtype=torch.float32)
    return 0.3 * z[0], torch.exp(0.4 * z[1])


def make_hot(w: Workload, device="cpu", seed_offset: int = 0):
    """Exact (hot) keys/values ``[batch, kv_heads, hot_tokens, head_dim]`` in fp16/bf16/fp32."""
    dt = _DT[w.kv_dtype]
    g = generator(w.seed * 31337 + 5 + seed_offset, device)
    shape = (w.batch, w.kv_heads, w.hot_tokens, w.head_dim)
    hk = normal(shape, g, device)
    hv = normal(shape, g, device)
    if w.name == "tinyllama_layer":
        gsel = generator(w.seed * 7919 + 17 + seed_offset, "cpu")
        outlier = torch.randperm(w.head_dim, generator=gsel)[:2].to(device)
        hk[..., outlier] *= 8.0
        hv[..., outlier] *= 8.0
    return hk.to(dt), hv.to(dt)


def make_queries(w: Workload, device="cpu", seed_offset: int = 0) -> torch.Tensor:
    """Decode queries ``[batch, q_heads, head_dim]``; for a bulk scan
    ``[batch, kv_heads, scan_queries, head_dim]``."""
    g = generator(w.seed * 65537 + 11 + seed_offset, device)
    if w.scan_queries:
        shape = (w.batch, w.kv_heads, w.scan_queries, w.head_dim)
    else:
        shape = (w.batch, w.q_heads, w.head_dim)
    x = normal(shape, g, device)
    if w.name == "vector_search_d200":        # queries from the database's distribution
        mu, sigma = embedding_channels(w)
        x = mu.to(device) + sigma.to(device) * x
    return x.to(_DT[w.q_dtype])


def small(w: Workload, tokens: int, batch: int | None = None, hot_tokens: int | None = None,
          top_k: int | None = None, scan_queries: int | None = None) -> Workload:
    """The same workload family at a reduced size (for oracle-sized parity cases)."""
    return dataclasses.replace(
        w, tokens=tokens, batch=w.batch if batch is None else batch,
        hot_tokens=w.hot_tokens if hot_tokens is None else hot_tokens,
        top_k=w.top_k if top_k is None else top_k,
        scan_queries=w.scan_queries if scan_queries is None else scan_queries)
