"""Oracle work for the full-size parity tests, spread over spawned worker processes.

Test infrastructure: the workers import numpy and the oracle only (never torch, never the
HIP library), so they hold no GPU context.  Each job is one independent unit of the oracle's
own functions - a sequence of a decode, a (sequence, KV head) unit of a selection - called
exactly as a single-process test would call them; the pool only runs several at once.
"""
from __future__ import annotations

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

_CODECS = {}


def workers() -> int:
    """At most 16 processes: the CPU share of one GPU on the test machines."""
    return max(1, min(16, os.cpu_count() or 1))


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:
        pass


def run(fn, jobs):
    """fn(job) for every job, in job order."""
    jobs = list(jobs)
    if len(jobs) <= 1:
        return [fn(j) for j in jobs]
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=min(workers(), len(jobs)), mp_context=ctx,
                             initializer=_init_worker) as ex:
        return list(ex.map(fn, jobs))


def codec(args):
    """args = (head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed, polar_upper_bits)."""
    if args not in _CODECS:
        from oracle import polar as P
        from oracle import tq_oracle as O
        *base, ub = args
        _CODECS[args] = P.PolarCodec(*base, upper_bits=ub) if ub else O.Codec(*base)
    return _CODECS[args]


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(u16, np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ jobs ----------------
def decode_job(job):
    """One sequence of tq_decode_attention: job = (codec args, q [1, Hq, d], records
    [1, Hkv, cap, R], n_tokens, want_logits).  Returns (out [Hq, d], lse [Hq], cold logits
    [Hq, n] float32 or None)."""
    from oracle import tq_oracle as O
    args, q, rec, n, want_logits = job
    c = codec(args)
    out, lse, lg = O.decode_attention(c, q, rec, [n])
    logits = None
    if want_logits:
        logits = np.stack([lg[(0, h)][0] for h in range(q.shape[1])]).astype(np.float32)
    return out[0], lse[0], logits


def sparse_unit_job(job):
    """One (sequence, KV head) unit of Self-Indexing sparse decode: the oracle's select_topk on
    the given index and codebook, then its decode over the selected records.  job = (codec
    args, q [1, G, d], index [1, 1, cap, d/8], codebook [1, 1, d/4, 16, 4], records
    [1, 1, cap, R], n_tokens, k).  Returns (idx [k], count, scores [k], out [G, d], lse [G])."""
    from oracle import tq_oracle as O
    args, q, index, book, rec, n, k = job
    c = codec(args)
    idx, cnt, scs = O.select_topk(c, q, index, book, [n], k)
    out, lse, _ = O.decode_attention(c, q, rec, [n], sel_idx=idx)
    return idx[0, 0], int(cnt[0, 0]), scs[0, 0], out[0], lse[0]


def sign_index_unit_job(job):
    """Sign index of one (sequence, KV head) unit.  job = (keys [n, d] as bfloat16 bits,
    the GPU's mean [d], the GPU's patterns [n, d/4]).  Returns the oracle's own (mean,
    patterns, codebook) and its patterns and codebook taken with the GPU's mean and
    patterns: (mu, pat, book, pat_at_gpu_mu, book_at_gpu_patterns)."""
    from oracle import tq_oracle as O
    ku16, mu_gpu, pat_gpu = job
    k = bf16_bits_to_f32(ku16)
    ref_index, ref_book, ref_mu = O.build_sign_index(None, k[None, :, None, :], k.shape[0])
    ng = k.shape[1] // 4
    pat = O._unpack_stream(ref_index[0, 0], ng, 4)
    return (ref_mu[0, 0], pat, ref_book[0, 0], O.sign_patterns(k, mu_gpu),
            O.pattern_centroids(k, mu_gpu, pat_gpu))
