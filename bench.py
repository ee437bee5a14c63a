#!/usr/bin/env python3
"""Benchmark of the compressed-KV hot path on one MI355X.

Default workload (the configuration the metric is quoted on): the Llama-3-8B-shaped 32K-context
decode - batch 16, 32 query heads, 8 KV heads, head_dim 128, 3-bit keys + 128-bit QJL sketch,
4-bit values, Student-t(4) K/V in bf16.  A step is one decode pass of the hot path over the
resident compressed cache: query preparation, the split-K scan over every packed record (score
estimates from the codes, online softmax, rotated-domain value aggregation) and the merge
(log-sum-exp combine, exact segment, un-rotation).  The cache is compressed once before the
timed region; that compress is timed on its own and reported beside the step.

Other workloads (``--workload``), each with its own step:
  * ``sparse_128k_top2048``: Self-Indexing top-k over the 1-bit sign index (integer LUT scores
    of every token, radix selection of 2,048 per KV head) followed by attention over the
    selected tokens' records (gather mode); the index and the records are built once.
  * ``bulk_64k_scan``: the score scan of 256 queries per KV head against all 65,536 compressed
    tokens of 8 heads (score matrix written to HBM).
  * ``tinyllama_layer``, ``single_head_1k``: small decode steps (latency-bound).

Prints ONE JSON line.  `roofline` describes the step's dominant kernel: algorithmic bytes per
launch over its average duration, timed with HIP events the library records on the kernel's own
stream around every launch of the timed steps.  `cpu_baseline` times the scalar C oracle (one
thread per host core, at most 16) on a bounded sample of the same workload, with the numpy oracle
beside it (polar keys and the hot/cold step: the numpy oracle alone).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "compressed_key_attention_amd", "csrc", "tq_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")
DECODE_WORKLOADS = ["llama8b_decode_32k", "tinyllama_layer", "single_head_1k", "llama8b_decode_32k_polar"]


class HipEvents:
    """hipEvent_t handles through the HIP runtime (the library records them on its stream).
    Created with hipEventDisableSystemFence: they only time work (their results are read after a
    device synchronisation), so recording them needs no system-scope cache write-back, which
    would otherwise add to every timed step."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if it was
    taken from the current kernel source (else null)."""
    try:
        with open(os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256_16") != kernel_source_hash() or s.get("workload") != workload:
        return None
    return s.get("hbm_bytes_per_launch")


def decode_kernel_name(w) -> str:
    """The scan kernel the library picks for this shape (matrix-core path for head_dim 128,
    4 query heads per KV head, 2/3-bit keys, 4-bit values, m in {0, 128})."""
    if w.polar_upper_bits:   # polar keys: 4-bit level-1 / 2-bit higher angles on the same shape
        mfma = (w.head_dim == 128 and w.q_heads == 4 * w.kv_heads and w.value_bits == 4
                and w.key_bits == 4 and w.polar_upper_bits == 2 and w.qjl_dim in (0, 128))
    else:
        mfma = (w.head_dim == 128 and w.q_heads == 4 * w.kv_heads and w.value_bits == 4
                and w.key_bits in (2, 3) and w.qjl_dim in (0, 128))
    if mfma:
        return "decode_mfma_kernel"
    G = w.q_heads // w.kv_heads
    small = (not w.polar_upper_bits and w.tokens <= 4096 and 4 <= G <= 16 and w.qjl_dim <= 128
             and w.qjl_dim % 32 == 0 and w.head_dim in (64, 128))
    return "decode_small_kernel" if small else "decode_scan_kernel"


def record_payload_bytes(w) -> int:
    kbytes = w.head_dim * w.key_bits // 8
    if w.polar_upper_bits:   # level-1 angle stream + upper-level stream in whole 32-bit words
        kbytes = w.head_dim // 2 * w.key_bits // 8 + 4 * (((w.head_dim // 2 - 1) * w.polar_upper_bits + 31) // 32)
    return kbytes + w.qjl_dim // 8 + w.head_dim * w.value_bits // 8 + 12


KERNEL_STATS = {}   # median / min of the last time_steps' dominant-kernel durations


def time_steps(ev, tq, step, steps, warmup):
    """Runs warmup + steps; events around the dominant kernel of every timed step."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in pairs:
        tq.set_profile_events(a, b)
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = sorted(ev.elapsed_ms(a, b) for a, b in pairs)
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    KERNEL_STATS["median_ms"] = times[len(times) // 2]
    KERNEL_STATS["min_ms"] = times[0]
    return wall * 1000.0 / steps, sum(times) / len(times)


def read_ceiling_gbps(tq, ev, nbytes: int = 2 << 30, reps: int = 10) -> float:
    """The library's own streaming read over a 2 GiB buffer (HIP-event timed): the practical
    HBM read ceiling the roofline fractions are also quoted against."""
    import torch
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(64 * torch.cuda.get_device_properties(0).multi_processor_count, dtype=torch.int32,
                       device="cuda")
    for _ in range(3):
        tq.stream_read(buf, sink)
    torch.cuda.synchronize()
    tot = 0.0
    for _ in range(reps):
        a, b = ev.create(), ev.create()
        tq.set_profile_events(a, b)
        tq.stream_read(buf, sink)
        torch.cuda.synchronize()
        tot += ev.elapsed_ms(a, b)
        ev.destroy(a)
        ev.destroy(b)
    del buf
    return nbytes / (tot / reps * 1e-3) / 1e9


def flushed_kernel_ms(tq, ev, step, reps: int = 20) -> float:
    """Mean duration of the step's dominant kernel when a 1 GiB streaming read replaces the
    256 MB MALL's contents before every step (clean lines, so the eviction writes nothing
    back), i.e. the step's inputs come from HBM, not the cache."""
    import torch
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(7)
    sink = torch.empty(64 * torch.cuda.get_device_properties(0).multi_processor_count, dtype=torch.int32,
                       device="cuda")
    torch.cuda.synchronize()
    tot = 0.0
    for _ in range(reps):
        tq.stream_read(scratch, sink)
        a, b = ev.create(), ev.create()
        tq.set_profile_events(a, b)
        step()
        torch.cuda.synchronize()
        tot += ev.elapsed_ms(a, b)
        ev.destroy(a)
        ev.destroy(b)
    del scratch
    return tot / reps


def roofline(kernel, workload, alg_bytes, kernel_ms, extra=None, flushed_ms=None, ceiling=None):
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    r = {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_from_profile(kernel, workload),
         "algorithmic_bytes_per_launch": alg_bytes, "kernel_ms": kernel_ms,
         "kernel_ms_median": KERNEL_STATS.get("median_ms"), "kernel_ms_min": KERNEL_STATS.get("min_ms")}
    if flushed_ms:
        fa = alg_bytes / (flushed_ms * 1e-3) / 1e9
        r.update({"kernel_ms_mall_flushed": flushed_ms, "achieved_mall_flushed": fa,
                  "frac_mall_flushed": fa / HBM_PEAK_GBPS})
    if ceiling:
        r.update({"read_ceiling_gbps": ceiling, "frac_of_read_ceiling": achieved / ceiling})
    if extra:
        r.update(extra)
    return r


def compress_once(ev, tq, h, K, V, records):
    """One-time compress of the whole cache (warm-up call first), timed on its own."""
    import torch
    h.compress_kv(K, V, records)
    torch.cuda.synchronize()
    c0, c1 = ev.create(), ev.create()
    tq.set_profile_events(c0, c1)
    h.compress_kv(K, V, records)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(c0, c1)
    ev.destroy(c0)
    ev.destroy(c1)
    return ms


_CODECS = {}


def codec_args_of(w):
    """The oracle codec's constructor arguments for a workload (last: polar upper-level bits)."""
    return (w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2,
            w.polar_upper_bits)


def _codec(codec_args):
    """The oracle's handle constants, built once per process (outside any timed region)."""
    if codec_args not in _CODECS:
        from oracle import polar as P
        from oracle import tq_oracle as O
        *base, ub = codec_args
        _CODECS[codec_args] = P.PolarCodec(*base, upper_bits=ub) if ub else O.Codec(*base)
    return _CODECS[codec_args]


def _oracle_job(job):
    """One unit of oracle work (runs in this process or in a spawned worker)."""
    from threadpoolctl import threadpool_limits
    from oracle import tq_oracle as O
    kind, codec_args, arrays, extra = job
    codec = _codec(codec_args)
    with threadpool_limits(limits=1):
        if kind == "decode":
            q, rec, hk, hv = arrays
            if hk is None:
                O.decode_attention(codec, q, rec, [extra["tokens"]])
            else:
                O.decode_attention(codec, q, rec, [extra["tokens"]], hk, hv, [extra["hot"]])
        elif kind == "sparse":
            q, idx, book, rec = arrays
            ri, _, _ = O.select_topk(codec, q, idx, book, [extra["tokens"]], extra["k"])
            O.decode_attention(codec, q, rec, [extra["tokens"]], sel_idx=ri)
        else:
            q, rec = arrays
            O.score_scan(codec, q, rec, extra["tokens"])
    return 0


def _warm_job(codec_args):
    import threadpoolctl  # noqa: F401
    _codec(codec_args)
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_baseline(units, make_job, tokens_per_unit, total_units, unit_name, budget_s=12.0, max_workers=16):
    """The oracle as it is, single-threaded on units in order until ~budget_s of CPU time, then
    over a pool of worker processes (one per host core, at most max_workers) on a batch sized to
    about the same wall time.  Inputs are copied to host memory before each timer starts."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    done, elapsed = 0, 0.0
    _codec(make_job(units[0])[1])
    for u in units:
        job = make_job(u)
        t0 = time.perf_counter()
        _oracle_job(job)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= budget_s:
            break
    rate1 = done * tokens_per_unit / elapsed
    workers = max(1, min(max_workers, os.cpu_count() or 1))
    per_unit = elapsed / done
    # at least one unit per worker (units repeated when the workload has fewer)
    n_multi = workers * max(1, int(budget_s / per_unit / 2))
    if len(units) >= workers:
        n_multi = min(len(units), n_multi)
    jobs = [make_job(units[i % len(units)]) for i in range(n_multi)]
    with ProcessPoolExecutor(max_workers=workers, mp_context=multiprocessing.get_context("spawn")) as ex:
        list(ex.map(_warm_job, [jobs[0][1]] * workers))
        t0 = time.perf_counter()
        list(ex.map(_oracle_job, jobs))
        wall = time.perf_counter() - t0
    rate_w = n_multi * tokens_per_unit / wall
    host = os.cpu_count() or 1
    return {"value": rate_w, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "host_cores": host,
            "core_cap": (f"at most {max_workers} worker processes: the CPU share of one GPU on the "
                         f"benchmark machines ({host} host cores visible)") if host > workers else None,
            "sample": f"{n_multi} (of {total_units}, repeated when fewer than the workers) {unit_name} over {workers} worker processes "
                      f"(numpy float64 oracle, BLAS 1 thread each), {wall:.1f} s wall",
            "single_thread": {"value": rate1, "cores": 1,
                              "sample": f"{done} {unit_name}, {elapsed:.1f} s"},
            "cpu_model": cpu_model()}


def _scalar_codec(w):
    from oracle import scalar as SC
    key = ("scalar",) + codec_args_of(w)[:6]
    if key not in _CODECS:
        _CODECS[key] = SC.ScalarCodec(*codec_args_of(w)[:6])
    return _CODECS[key]


def scalar_baseline(units, run_unit, tokens_per_unit, total_units, unit_name, budget_s=6.0, max_threads=16):
    """The scalar C oracle (oracle/tq_scalar.c) as it is: one thread on units in order until
    ~budget_s, then one thread per host core (at most max_threads; the library's calls release
    the GIL) on a batch sized to about the same wall time.  Inputs are host arrays prepared
    before the timers start."""
    from concurrent.futures import ThreadPoolExecutor
    done, elapsed = 0, 0.0
    for u in units:
        t0 = time.perf_counter()
        run_unit(u)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= budget_s:
            break
    rate1 = done * tokens_per_unit / elapsed
    threads = max(1, min(max_threads, os.cpu_count() or 1))
    per_unit = elapsed / done
    # a batch of at least one unit per thread (the units repeated when the workload has fewer),
    # sized to about half the single-thread budget of wall time
    n_multi = threads * max(1, int(budget_s / per_unit / 2))
    if len(units) >= threads:
        n_multi = min(len(units), n_multi)
    batch = [units[i % len(units)] for i in range(n_multi)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(run_unit, batch))
        wall = time.perf_counter() - t0
    host = os.cpu_count() or 1
    return {"value": n_multi * tokens_per_unit / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cores": host,
            "core_cap": (f"at most {max_threads} threads: the CPU share of one GPU on the benchmark "
                         f"machines ({host} host cores visible)") if host > threads else None,
            "sample": f"{n_multi} (of {total_units}, repeated when fewer than the threads) {unit_name} over {threads} threads (scalar C oracle, "
                      f"oracle/tq_scalar.c at -O2, double accumulation), {wall:.1f} s wall",
            "single_thread": {"value": rate1, "cores": 1, "sample": f"{done} {unit_name}, {elapsed:.1f} s"},
            "cpu_model": cpu_model()}


def compute_dtype(w) -> str:
    """Arithmetic of the step's scan: int8 matrix-core key products (exact in int32) and bf16
    matrix-core value products accumulated in fp32 on the matrix-core paths (decode at head_dim
    128 with 4 query heads per KV head; the bulk scan's int8 products), fp32 elsewhere."""
    if w.name == "bulk_64k_scan" and w.head_dim == 128 and w.key_bits in (2, 3) and w.qjl_dim in (0, 128):
        return "i8 (int32 accumulate)"
    if w.scan_queries:
        return "f16 hi/lo matrix-core products (fp32 accumulate)"
    if w.name == "sparse_128k_top2048":
        return "i32 (selection scores) + f32 (attention)"
    if decode_kernel_name(w) == "decode_mfma_kernel" and w.polar_upper_bits:
        return "f16 hi/lo key products + i8 sketch + bf16 values (fp32 / int32 accumulate)"
    if decode_kernel_name(w) == "decode_mfma_kernel":
        return "i8 + bf16 (int32 / fp32 accumulate)"
    return "f32"


def base_line(args, w, ms_per_step, tokens_per_step):
    return {
        "metric": "compressed KV tokens attended/sec per GPU + % of HBM roofline (GB/s)",
        "value": tokens_per_step / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(w),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "context": w.tokens, "key_bits": w.key_bits,
                   "qjl_dim": w.qjl_dim, "value_bits": w.value_bits, "kv_dtype": w.kv_dtype,
                   "q_dtype": w.q_dtype, "seed": w.seed,
                   "key_codec": "polar" if w.polar_upper_bits else "scalar",
                   "polar_upper_bits": w.polar_upper_bits},
    }


# ---------------------------------------------------------------------------------------------
def run_decode(args, tq, W, ev):
    import torch
    w = W.WORKLOADS[args.workload]
    dev = "cuda"
    h = tq.Handle(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2,
                  polar_upper_bits=w.polar_upper_bits)
    K, V = W.make_kv(w, dev)
    q = W.make_queries(w, dev)
    records = h.new_cache(w.batch, w.kv_heads, w.tokens, dev)
    compress_ms = compress_once(ev, tq, h, K, V, records)
    del K, V
    token_heads = w.batch * w.kv_heads * w.tokens
    flops_th = 2 * (2 * w.head_dim * w.head_dim + w.qjl_dim * w.head_dim)
    hot = {}
    if w.hot_tokens:
        hk, hv = W.make_hot(w, dev)
        hot = dict(hot_k=hk, hot_v=hv,
                   hot_lens=torch.full((w.batch,), w.hot_tokens, dtype=torch.int32, device=dev))
    seq_lens = torch.full((w.batch,), w.tokens, dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(h.decode_workspace_size(w.batch, w.q_heads, w.kv_heads, w.tokens), dtype=torch.uint8,
                     device=dev)

    def step():
        h.decode_attention(q, records, seq_lens, out=out, workspace=ws, **hot)

    ms_per_step, scan_ms = time_steps(ev, tq, step, args.steps, args.warmup)
    fl_ms = flushed_kernel_ms(tq, ev, step)
    ceiling = read_ceiling_gbps(tq, ev)
    alg_bytes = record_payload_bytes(w) * token_heads
    line = base_line(args, w, ms_per_step, w.batch * (w.tokens + w.hot_tokens))
    line["config"].update({"hot_tokens": w.hot_tokens, "record_bytes": h.record_bytes})
    line["roofline"] = roofline(decode_kernel_name(w), w.name, alg_bytes, scan_ms, {"scan_ms": scan_ms}, fl_ms,
                                ceiling)
    line["token_heads_per_s"] = token_heads / (ms_per_step * 1e-3)
    line["compress"] = {"ms": compress_ms, "token_heads_per_s": token_heads / (compress_ms * 1e-3),
                        "mfma_f64_tflops": flops_th * token_heads / (compress_ms * 1e-3) / 1e12,
                        "mfma_f64_peak_tflops": 78.6}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(w, h, q, records, hot)
        line["compress"]["cpu_baseline"] = cpu_baseline_compress(w)
    return line


def cpu_baseline_decode(w, h, q, records, hot, budget_s: float = 6.0):
    """Oracle decode of the same cache: the scalar C oracle per (sequence, query head) - a unit
    attends (tokens + hot tokens) / q_heads tokens of the metric - and, where it covers the
    codec (not polar keys), the numpy oracle over whole sequences beside it."""
    qn = q.float().cpu().numpy()
    hk = hot["hot_k"].float().cpu().numpy() if hot else None
    hv = hot["hot_v"].float().cpu().numpy() if hot else None
    codec_args = codec_args_of(w)

    def make_job(b):
        return ("decode", codec_args,
                (qn[b:b + 1], records[b:b + 1].cpu().numpy(), None if hk is None else hk[b:b + 1],
                 None if hv is None else hv[b:b + 1]), {"tokens": w.tokens, "hot": w.hot_tokens})

    numpy_leg = oracle_baseline(list(range(w.batch)), make_job, w.tokens + w.hot_tokens, w.batch, "sequences",
                                budget_s)
    if w.polar_upper_bits:
        return numpy_leg
    c = _scalar_codec(w)
    r = records.cpu().numpy()
    G = w.q_heads // w.kv_heads
    units = [(b, hq) for b in range(w.batch) for hq in range(w.q_heads)]

    def run_unit(u):
        b, hq = u
        c.decode_head(qn[b, hq], r[b, hq // G], w.tokens, None, None if hk is None else hk[b, hq // G],
                      None if hv is None else hv[b, hq // G])

    line = scalar_baseline(units, run_unit, (w.tokens + w.hot_tokens) / w.q_heads, len(units),
                           "(sequence, query head) units", budget_s)
    line["numpy_oracle"] = numpy_leg
    return line


def cpu_baseline_compress(w, budget_s: float = 4.0):
    """Oracle compress (one core) of 4096-token blocks of one head of the same synthetic K/V: the
    scalar C oracle and, beside it, the numpy oracle."""
    from threadpoolctl import threadpool_limits
    from compressed_key_attention_amd import workloads as W
    codec = _codec(codec_args_of(w))
    K, V = W.make_kv(w, "cpu", tokens=4096, batch=1)
    blocks = [(K[0, :, hh].float().numpy(), V[0, :, hh].float().numpy()) for hh in range(w.kv_heads)]

    def leg(fn, what):
        done, elapsed = 0, 0.0
        for k, v in blocks:
            t0 = time.perf_counter()
            fn(k, v)
            elapsed += time.perf_counter() - t0
            done += 1
            if elapsed >= budget_s:
                break
        return {"value": done * 4096 / elapsed, "unit": "token-heads/s", "cores": 1, "kind": "oracle",
                "sample": f"{done} blocks of 4096 token-heads, {elapsed:.2f} s ({what})"}

    with threadpool_limits(limits=1):
        numpy_leg = leg(codec.compress_fields, "numpy oracle")
    if w.polar_upper_bits:
        return numpy_leg
    c = _scalar_codec(w)
    line = leg(c.compress, "scalar C oracle")
    line["numpy_oracle"] = numpy_leg
    return line


# ---------------------------------------------------------------------------------------------
def run_sparse(args, tq, W, ev):
    import torch
    w = W.WORKLOADS["sparse_128k_top2048"]
    dev = "cuda"
    h = tq.Handle(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2,
                  polar_upper_bits=w.polar_upper_bits)
    K, V = W.make_kv(w, dev)
    B, T, H, d = K.shape
    index = torch.empty((B, H, T, d // 8), dtype=torch.uint8, device=dev)
    book = torch.empty((B, H, d // 4, 16, 4), dtype=torch.float32, device=dev)
    h.build_sign_index(K, index, book)
    # sign-index build (one-time): a warm call timed with events on the library's stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    h.build_sign_index(K, index, book)
    e1.record()
    torch.cuda.synchronize()
    index_ms = e0.elapsed_time(e1)
    records = h.new_cache(B, H, T, dev)
    compress_ms = compress_once(ev, tq, h, K, V, records)
    del K, V
    q = W.make_queries(w, dev)
    seq_lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    sel = torch.empty((B, H, w.top_k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
    sws = torch.empty(h.select_workspace_size(B, H, T), dtype=torch.uint8, device=dev)
    out = torch.empty((B, w.q_heads, d), dtype=torch.float32, device=dev)
    dws = torch.empty(h.decode_workspace_size(B, w.q_heads, H, T, k_sel=w.top_k), dtype=torch.uint8,
                      device=dev)

    pws = torch.empty(h.sparse_workspace_size(B, w.q_heads, H, T), dtype=torch.uint8, device=dev)

    def step():
        # selection and attention over the selected compressed tokens in one call
        h.sparse_attention(q, index, book, records, seq_lens, w.top_k, out=out, workspace=pws)

    def step_two_calls():
        h.select_topk(q, index, book, seq_lens, w.top_k, out_idx=sel, out_count=cnt, workspace=sws)
        h.decode_attention(q, records, seq_lens, sel_idx=sel, out=out, workspace=dws)

    two_call_ms, _ = time_steps(ev, tq, step_two_calls, args.steps, args.warmup)
    ms_per_step, score_ms = time_steps(ev, tq, step, args.steps, args.warmup)
    fl_ms = flushed_kernel_ms(tq, ev, step)
    ceiling = read_ceiling_gbps(tq, ev)
    token_heads = B * H * T
    alg_bytes = token_heads * (d // 8)            # 1-bit sign index: d/8 bytes per token-head
    line = base_line(args, w, ms_per_step, B * T)
    line["metric"] = "tokens scored per second (sign-index top-k + sparse attention) + % of HBM roofline"
    line["config"].update({"top_k": w.top_k, "index_bytes_per_token_head": d // 8})
    line["roofline"] = roofline("select_score_kernel", w.name, alg_bytes, score_ms, None, fl_ms, ceiling)
    line["tokens_attended_per_s"] = B * H * w.top_k / (ms_per_step * 1e-3)
    line["step"] = "tq_sparse_attention (one call)"
    line["two_call_ms_per_step"] = two_call_ms        # tq_select_topk + tq_decode_attention(sel_idx)
    line["compress"] = {"ms": compress_ms}
    key_bytes = B * T * H * d * 2
    line["sign_index_build"] = {"ms": index_ms, "key_bytes": key_bytes,
                                "key_read_gbps": key_bytes / (index_ms * 1e-3) / 1e9,
                                "note": "two passes over the bf16 keys (channel mean, then patterns and centroids)"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_sparse(w, q, index, book, records)
    return line


def cpu_baseline_sparse(w, q, index, book, records, budget_s: float = 6.0):
    """Oracle select + gathered attention per (sequence, KV head) unit; a unit scores T tokens
    of one KV head, so T / kv_heads tokens of the workload.  The scalar C oracle, and the numpy
    oracle beside it."""
    from oracle import scalar as SC
    codec_args = codec_args_of(w)
    qn = q.float().cpu().numpy()
    T, G = w.tokens, w.q_heads // w.kv_heads
    units = [(b, hh) for b in range(w.batch) for hh in range(w.kv_heads)]

    def make_job(u):
        b, hh = u
        return ("sparse", codec_args,
                (qn[b:b + 1, hh * G:(hh + 1) * G], index[b:b + 1, hh:hh + 1].cpu().numpy(),
                 book[b:b + 1, hh:hh + 1].cpu().numpy(), records[b:b + 1, hh:hh + 1].cpu().numpy()),
                {"tokens": T, "k": w.top_k})

    numpy_leg = oracle_baseline(units, make_job, T / w.kv_heads, len(units), "(sequence, KV head) units",
                                budget_s)
    c = _scalar_codec(w)
    gi, gb, r = index.cpu().numpy(), book.cpu().numpy(), records.cpu().numpy()

    def run_unit(u):
        b, hh = u
        idx, n, _ = SC.select_unit(qn[b, hh * G:(hh + 1) * G], gi[b, hh], gb[b, hh], T, w.top_k)
        for j in range(G):
            c.decode_head(qn[b, hh * G + j], r[b, hh], n, idx[:n])

    line = scalar_baseline(units, run_unit, T / w.kv_heads, len(units), "(sequence, KV head) units", budget_s)
    line["numpy_oracle"] = numpy_leg
    return line


# ---------------------------------------------------------------------------------------------
def recall_1_at_k(approx, exact, ks):
    """Measurement only: share of queries whose exact best inner product is among the k best
    approximate scores (ties to the lower index), for approx / exact [queries, vectors]."""
    import numpy as np
    best = np.argmax(exact, axis=1)
    a = approx[np.arange(len(best)), best][:, None]
    idx = np.arange(approx.shape[1])[None, :]
    rank = np.sum(approx > a, axis=1) + np.sum((approx == a) & (idx < best[:, None]), axis=1)
    return {str(k): float(np.mean(rank < k)) for k in ks}


def run_bulk_scan(args, tq, W, ev):
    import torch
    w = W.WORKLOADS[args.workload]
    dev = "cuda"
    h = tq.Handle(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2,
                  polar_upper_bits=w.polar_upper_bits)
    K, V = W.make_kv(w, dev)
    B, T, H, d = K.shape
    records = h.new_cache(B, H, T, dev)
    compress_ms = compress_once(ev, tq, h, K, V, records)
    k_host = K[0, :, 0].double().cpu().numpy() if w.name == "vector_search_d200" else None
    del K, V
    q = W.make_queries(w, dev)                     # [B, H, n_queries, d]
    nq = w.scan_queries
    scores = torch.empty((B, H, nq, T), dtype=torch.float32, device=dev)
    ws = torch.empty(h.scan_workspace_size(B, H, nq), dtype=torch.uint8, device=dev)

    def step():
        h.score_scan(q, records, T, scores=scores, workspace=ws)

    ms_per_step, scan_ms = time_steps(ev, tq, step, args.steps, args.warmup)
    fl_ms = flushed_kernel_ms(tq, ev, step)
    ceiling = read_ceiling_gbps(tq, ev)
    key_bytes = d * w.key_bits // 8 + w.qjl_dim // 8 + 8      # codes + sketch + r_k, rho
    alg_bytes = B * H * T * key_bytes + B * H * nq * T * 4     # key records read + scores written
    line = base_line(args, w, ms_per_step, B * T)
    line["metric"] = (f"compressed tokens scanned per second ({nq} queries per KV head) + % of "
                      + ("HBM" if w.name == "bulk_64k_scan" else "fp16 matrix-core") + " roofline")
    line["config"].update({"scan_queries": nq})
    mfma = w.head_dim == 128 and w.key_bits in (2, 3) and w.qjl_dim in (0, 128)
    kname = "scan_mfma_kernel" if mfma else "scan_mfma16_kernel"
    extra = None
    if mfma:
        # int8 matrix-core work the kernel executes: 22 (16 without the sketch) 16x16x64 MFMAs
        # per tile of 16 tokens x 16 queries
        n_mfma = (22 if w.qjl_dim else 16) * (B * H * T / 16) * (nq / 16)
        tops = n_mfma * 2 * 16 * 16 * 64 / (scan_ms * 1e-3) / 1e12
        extra = {"mfma_int8_executed_tops": tops, "mfma_int8_peak_tops": 5000.0,
                 "mfma_int8_frac": tops / 5000.0}
    line["roofline"] = roofline(kname, w.name, alg_bytes, scan_ms, extra, fl_ms, ceiling)
    if not mfma:
        # a dense contraction over the d + m operands of every (query, vector) pair, run as three
        # fp16 matrix-core products (hi.hi, hi.lo, lo.hi) of operands padded to 32-multiples
        flops = 2.0 * (d + w.qjl_dim) * B * H * nq * T
        kp = (d + w.qjl_dim + 31) // 32 * 32
        executed = 3 * 2.0 * kp * B * H * (((nq + 127) // 128) * 128) * (((T + 127) // 128) * 128)
        tf = flops / (scan_ms * 1e-3) / 1e12
        tx = executed / (scan_ms * 1e-3) / 1e12
        hbm = line["roofline"]
        line["roofline"] = {"bound": "mfma", "kernel": kname, "achieved": tf, "peak": 2500.0, "unit": "TFLOP/s",
                            "frac": tf / 2500.0, "traffic": hbm["traffic"], "algorithmic_flops_per_launch": flops,
                            "mfma_f16_executed_tflops": tx, "mfma_f16_executed_frac": tx / 2500.0,
                            "kernel_ms": scan_ms, "kernel_ms_median": hbm["kernel_ms_median"],
                            "kernel_ms_min": hbm["kernel_ms_min"], "hbm_gbps": hbm["achieved"],
                            "hbm_frac": hbm["frac"], "algorithmic_bytes_per_launch": alg_bytes}
    line["scores_per_s"] = B * H * nq * T / (ms_per_step * 1e-3)
    if k_host is not None:
        exact = q[0, 0].double().cpu().numpy() @ k_host.T
        line["recall_1_at_k"] = recall_1_at_k(scores[0, 0].double().cpu().numpy(), exact,
                                              [1, 2, 4, 8, 16, 32, 64])
    line["compress"] = {"ms": compress_ms, "token_heads_per_s": B * H * T / (compress_ms * 1e-3)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_scan(w, q, records)
    return line


def cpu_baseline_scan(w, q, records, budget_s: float = 6.0):
    """Oracle bulk scan on 4096-token blocks of one KV head (all its queries); a block is
    4096 / kv_heads tokens of the workload.  The scalar C oracle, and the numpy oracle beside it."""
    codec_args = codec_args_of(w)
    qn = q.float().cpu().numpy()
    chunk = 4096
    units = [(hh, t0) for hh in range(w.kv_heads) for t0 in range(0, w.tokens - chunk + 1, chunk)]

    def make_job(u):
        hh, t0 = u
        return ("scan", codec_args, (qn[0:1, hh:hh + 1], records[0:1, hh:hh + 1, t0:t0 + chunk].cpu().numpy()),
                {"tokens": chunk})

    unit_name = f"4096-token blocks x {w.scan_queries} queries"
    numpy_leg = oracle_baseline(units, make_job, chunk / w.kv_heads, len(units), unit_name, budget_s)
    c = _scalar_codec(w)
    r = records.cpu().numpy()

    def run_unit(u):
        hh, t0 = u
        c.score_scan(qn[0:1, hh:hh + 1], r[0:1, hh:hh + 1, t0:t0 + chunk], chunk)

    line = scalar_baseline(units, run_unit, chunk / w.kv_heads, len(units), unit_name, budget_s)
    line["numpy_oracle"] = numpy_leg
    return line


# ---------------------------------------------------------------------------------------------
def run_monarch(args, tq, W, ev):
    """Hot/cold decode steps on the TinyLlama-shaped layer: 512 exact fp16 tokens in the ring,
    1,024 compressed cold tokens, one new token per step (so one eviction per step)."""
    import torch
    w = W.WORKLOADS["tinyllama_layer"]
    dev = "cuda"
    h = tq.Handle(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2,
                  polar_upper_bits=w.polar_upper_bits)
    n_steps = args.warmup + args.steps + 20
    window, Hq, H, d = w.hot_tokens, w.q_heads, w.kv_heads, w.head_dim
    hot_cap = window + 1 + 6 * Hq
    cold_cap = w.tokens + n_steps + 32
    st = tq.HotCold(h, w.batch, H, hot_cap, cold_cap, torch.float16, dev)
    K, V = W.make_kv(w, dev)
    h.compress_kv(K, V, st.records)
    hk, hv = W.make_hot(w, dev)
    st.hot_k[:, :, :window].copy_(hk)
    st.hot_v[:, :, :window].copy_(hv)
    st.hot_len.fill_(window)
    st.cold_len.fill_(w.tokens)
    g = torch.Generator(device=dev).manual_seed(w.seed * 977 + 3)
    qs = torch.randn((n_steps, w.batch, Hq, d), generator=g, device=dev).to(torch.float16)
    ks = torch.randn((n_steps, w.batch, H, d), generator=g, device=dev).to(torch.float16)
    vs = torch.randn((n_steps, w.batch, H, d), generator=g, device=dev).to(torch.float16)
    out = torch.empty((w.batch, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.monarch_workspace_size(h, w.batch, Hq, H, hot_cap, cold_cap), dtype=torch.uint8, device=dev)
    state = {"i": 0}
    snapshot = None
    if not args.no_cpu_baseline:
        snapshot = (st.records.cpu().numpy(), hk.float().cpu().numpy(), hv.float().cpu().numpy())

    def step():
        i = state["i"]
        state["i"] += 1
        tq.monarch_step(h, st, qs[i], ks[i], vs[i], window, out=out, workspace=ws)

    ms_per_step, scan_ms = time_steps(ev, tq, step, args.steps, args.warmup)
    torch.cuda.synchronize()
    tokens = window + w.tokens
    line = base_line(args, w, ms_per_step, w.batch * tokens)
    line["metric"] = "hot/cold decode steps: tokens attended/sec (512 exact + ~1,024 compressed per step)"
    line["config"].update({"window": window, "hot_capacity": hot_cap, "cold_gate": "inf",
                           "promote_weight": 0.15, "promote_steps": 3, "ring_dtype": "f16"})
    rec_alg = record_payload_bytes(w)
    alg = rec_alg * w.batch * H * (w.tokens + args.warmup + args.steps // 2)
    line["roofline"] = roofline(decode_kernel_name(w), "monarch_tinyllama", alg, scan_ms,
                                {"note": "latency-bound: the step is ~7 small launches; report us/step"})
    line["us_per_step"] = ms_per_step * 1e3
    line["state_after"] = {"hot_len": int(st.hot_len[0]), "cold_len": int(st.cold_len[0]),
                           "overflow": int(st.overflow[0])}
    if snapshot is not None:
        line["cpu_baseline"] = cpu_baseline_monarch(w, h, snapshot, qs, ks, vs, window)
    return line


def cpu_baseline_monarch(w, h, snapshot, qs, ks, vs, window, budget_s: float = 8.0):
    """The hot/cold oracle stepping the same initial state on one core."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import monarch as MO
    codec = _codec(codec_args_of(w))
    rec, hk, hv = snapshot
    o = MO.HotColdOracle(codec, w.batch, w.kv_heads, "float16", rec.shape[2])
    for b in range(w.batch):
        o.hot_k[b], o.hot_v[b] = hk[b].astype(np.float64), hv[b].astype(np.float64)
        o.cold[b] = rec[b][:, :w.tokens].copy()
        o.hits[b] = np.zeros(w.tokens, np.int64)
    qn, kn, vn = qs.float().cpu().numpy(), ks.float().cpu().numpy(), vs.float().cpu().numpy()
    done, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        for i in range(qn.shape[0]):
            t0 = time.perf_counter()
            o.step(qn[i], kn[i], vn[i], window)
            elapsed += time.perf_counter() - t0
            done += 1
            if elapsed >= budget_s:
                break
    tokens = done * (window + w.tokens)
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} hot/cold steps from the same initial state, {elapsed:.1f} s",
            "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama8b_decode_32k",
                    choices=DECODE_WORKLOADS + ["sparse_128k_top2048", "bulk_64k_scan", "monarch_tinyllama",
                                                "vector_search_d200"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device-to-device copies of 1 GiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "copies": 5}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus above 1 is not "
                                   "supported (sequences and KV heads would shard over GPUs with no "
                                   "exchange, so one GPU's share is what is measured)"}))
        sys.exit(2)

    import torch
    import compressed_key_attention_amd as tq
    from compressed_key_attention_amd import workloads as W

    torch.cuda.set_device(0)
    ev = HipEvents()
    if args.workload in DECODE_WORKLOADS:
        line = run_decode(args, tq, W, ev)
    elif args.workload == "sparse_128k_top2048":
        line = run_sparse(args, tq, W, ev)
    elif args.workload == "monarch_tinyllama":
        line = run_monarch(args, tq, W, ev)
    else:
        line = run_bulk_scan(args, tq, W, ev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
