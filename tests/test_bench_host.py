"""Host-side checks of bench.py (no GPU): the single-GPU guard, the payload byte counts and
the recall measurement, against the oracle's definition."""
import json
import subprocess
import sys
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_payload_bytes_match_the_oracle_record_fields():
    sys.path.insert(0, ROOT)
    import bench
    from compressed_key_attention_amd import workloads as W
    from oracle import polar as P
    from oracle import tq_oracle as O
    for name, w in W.WORKLOADS.items():
        if w.polar_upper_bits:
            codec = P.PolarCodec(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, 1, 2,
                                 upper_bits=w.polar_upper_bits)
        else:
            codec = O.Codec(w.head_dim, w.key_bits, w.qjl_dim, w.value_bits, 1, 2)
        # algorithmic payload: the code bits themselves, without the word padding of the fields
        key = codec.kbytes if w.polar_upper_bits else w.head_dim * w.key_bits // 8
        want = key + codec.sbytes + w.head_dim * w.value_bits // 8 + 12
        assert bench.record_payload_bytes(w) == want, name
        assert 0 <= codec.kbytes + codec.sbytes + codec.vbytes + 12 - want < 8, name


def test_bench_recall_equals_the_oracle_definition():
    sys.path.insert(0, ROOT)
    import bench
    from oracle import tq_oracle as O
    rng = np.random.default_rng(11)
    exact = rng.standard_normal((40, 500))
    approx = exact + 0.5 * rng.standard_normal((40, 500))
    approx[3, :] = approx[3, 7]                       # a query with every approximate score tied
    ks = [1, 2, 4, 16, 64]
    got = bench.recall_1_at_k(approx, exact, ks)
    want = O.recall_1_at_k(approx, exact, ks)
    assert {int(k): v for k, v in got.items()} == want
