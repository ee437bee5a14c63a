#!/usr/bin/env python3
"""Benchmark of the compressed-KV decode path on one MI355X.

A step is one decode pass of the hot path over the resident compressed cache: query
preparation (q_x = Pi q, q_s = S q_x), the split-K scan over every packed record (score
estimates from the codes, online softmax, rotated-domain value aggregation) and the merge
(log-sum-exp combine, exact segment, un-rotation).  The cache is compressed once before the timed region
(that compress is timed separately and reported beside the step).  The default workload is
the Llama-3-8B-shaped 32K-context decode (batch 16, 32 query heads, 8 KV heads, head_dim
128, 3-bit keys + 128-bit QJL sketch, 4-bit values, Student-t(4) K/V in bf16).

Prints ONE JSON line.  `roofline` describes the decode scan kernel: algorithmic bytes per
launch (140 B per token-head x token-heads) over its average duration, timed with HIP
events recorded on the kernel's own stream around every scan launch of the timed steps.
`cpu_baseline` times the oracle (single thread) on a bounded sample of the same workload.
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
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_scan_llama8b_decode_32k_traffic.json")


class HipEvents:
    """hipEvent_t handles through the HIP runtime (the library records them on its stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
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


def traffic_from_profile(workload: str, launches_bytes: float):
    """HBM bytes per scan launch from the committed rocprofv3 counter summary, if it was
    taken from the current kernel source (else null)."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256_16") != kernel_source_hash() or s.get("workload") != workload:
        return None
    return s.get("hbm_bytes_per_launch")


def scan_kernel_name(w) -> str:
    """The scan kernel the library picks for this shape (matrix-core path for head_dim 128,
    4 query heads per KV head, 2/3-bit keys, 4-bit values, m in {0, 128})."""
    mfma = (w.head_dim == 128 and w.q_heads == 4 * w.kv_heads and w.value_bits == 4
            and w.key_bits in (2, 3) and w.qjl_dim in (0, 128))
    return "decode_mfma_kernel" if mfma else "decode_scan_kernel"


def cpu_baseline(w, h, q, records, budget_s: float = 12.0):
    """The oracle, as it is, on whole sequences of the same cache until ~budget_s of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import tq_oracle as O
    codec = O.Codec(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, h.rotation_seed, h.qjl_seed)
    qn = q.float().cpu().numpy()
    done, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        for b in range(w.batch):
            rec = records[b:b + 1].cpu().numpy()
            t0 = time.perf_counter()
            O.decode_attention(codec, qn[b:b + 1], rec, [w.tokens])
            elapsed += time.perf_counter() - t0
            done += 1
            if elapsed >= budget_s:
                break
    return {"value": done * w.tokens / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {w.batch} sequences ({done * w.tokens} tokens x {w.q_heads} query heads), "
                      f"numpy float64 oracle, BLAS limited to 1 thread, {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_decode_32k",
                    choices=["llama8b_decode_32k", "tinyllama_layer", "single_head_1k"])
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
                                   "supported (the decode shards with no exchange, see the design notes)"}))
        sys.exit(2)

    import torch
    import compressed_key_attention_amd as tq
    from compressed_key_attention_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    h = tq.Handle(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, w.seed * 3 + 1, w.seed * 3 + 2)
    K, V = W.make_kv(w, dev)
    q = W.make_queries(w, dev)
    records = h.new_cache(w.batch, w.kv_heads, w.tokens, dev)
    ev = HipEvents()

    # ---- one-time compress of the whole cache (timed on its own) ----
    h.compress_kv(K, V, records)                 # warm-up (module load, LDS attribute)
    torch.cuda.synchronize()
    c0, c1 = ev.create(), ev.create()
    tq.set_profile_events(c0, c1)
    h.compress_kv(K, V, records)
    torch.cuda.synchronize()
    compress_ms = ev.elapsed_ms(c0, c1)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in pairs:
        tq.set_profile_events(a, b)
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    scan_ms = sum(ev.elapsed_ms(a, b) for a, b in pairs) / len(pairs)
    ms_per_step = wall * 1000.0 / args.steps

    tokens_per_step = w.batch * (w.tokens + w.hot_tokens)
    rec_alg = w.head_dim * w.key_bits // 8 + w.qjl_dim // 8 + w.head_dim * w.value_bits // 8 + 12
    alg_bytes = rec_alg * token_heads
    achieved = alg_bytes / (scan_ms * 1e-3) / 1e9
    line = {
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "context": w.tokens, "hot_tokens": w.hot_tokens,
                   "key_bits": w.key_bits, "qjl_dim": w.qjl_dim, "value_bits": w.value_bits,
                   "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype, "record_bytes": h.record_bytes,
                   "seed": w.seed},
        "roofline": {"bound": "hbm", "kernel": scan_kernel_name(w), "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic_from_profile(w.name, alg_bytes),
                     "algorithmic_bytes_per_launch": alg_bytes, "scan_ms": scan_ms},
        "token_heads_per_s": token_heads / (ms_per_step * 1e-3),
        "compress": {"ms": compress_ms, "token_heads_per_s": token_heads / (compress_ms * 1e-3),
                     "mfma_f64_tflops": flops_th * token_heads / (compress_ms * 1e-3) / 1e12,
                     "mfma_f64_peak_tflops": 78.6},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, h, q, records)
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
