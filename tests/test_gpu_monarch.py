"""GPU parity of the hot/cold step (tq_monarch_step) against oracle/monarch.py, step by step:
gates exact, outputs and lse within 1e-4 + 1e-3 |oracle|, and the whole state - ring
contents in ring order, cold records bytewise, sticky counts, lengths, overflow - equal.

The inputs keep every decision away from its threshold (checked on the oracle's values), so
float32 and float64 take the same decisions: background queries are small (near-uniform
weights, far below 0.15), a planted query points at one cold token for several steps (weight
near 1, promoted at the third), and a planted hot token closes the gate of its KV-head group
(best hot logit far above the gate)."""
import math

import numpy as np
import pytest
import torch

from compressed_key_attention_amd import workloads as W  # noqa: F401  (same seeded helpers)
from oracle import monarch as MO
from oracle import tq_oracle as O

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 1e-3
_DT = {"float16": torch.float16, "bfloat16": torch.bfloat16, "float32": torch.float32}


def _close(gpu, ref, what):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    bad = np.abs(gpu - ref) > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tolerance, worst {np.max(np.abs(gpu - ref)):.3e}"


@pytest.mark.parametrize("d,m,dtype,gate,ub,kb,vb", [
    (64, 64, "float16", math.inf, 0, 3, 4), (128, 128, "bfloat16", 6.0, 0, 3, 4),
    (64, 64, "float32", 6.0, 0, 3, 4), (128, 0, "float16", 6.0, 0, 3, 4),
    (128, 128, "bfloat16", 6.0, 2, 4, 4), (64, 64, "float16", math.inf, 2, 4, 4),
    (64, 32, "float32", 6.0, 4, 4, 4), (128, 0, "float16", 6.0, 1, 4, 4),
    (64, 64, "float16", math.inf, 0, 1, 1), (128, 128, "bfloat16", 6.0, 0, 1, 4),
    (64, 64, "float16", 6.0, 0, 2, 2)])
def test_hot_cold_steps_match_the_oracle(d, m, dtype, gate, ub, kb, vb):
    """ub > 0: polar key codes (4-bit level-1 angles, ub bits per higher angle), the Monarch
    page's polar cold tier: eviction runs the polar transform, promotion rebuilds r_k u.
    kb, vb: scalar key / value code widths (1-bit codes included)."""
    import compressed_key_attention_amd as tq
    from oracle import polar as P
    B, Hq, Hkv, Wn, cold_cap, steps = 2, 8, 2, 16, 40, 64
    G = Hq // Hkv
    h = tq.Handle(d, kb, m, vb, 31, 32, polar_upper_bits=ub)
    codec = P.PolarCodec(d, kb, m, vb, 31, 32, upper_bits=ub) if ub else O.Codec(d, kb, m, vb, 31, 32)
    hot_cap = Wn + 1 + 6 * Hq
    st = tq.HotCold(h, B, Hkv, hot_cap, cold_cap, _DT[dtype])
    ora = MO.HotColdOracle(codec, B, Hkv, dtype, cold_cap)
    rng = np.random.default_rng(d + m)
    keys = MO.round_to(rng.standard_normal((steps, B, Hkv, d)), dtype)
    vals = MO.round_to(rng.standard_normal((steps, B, Hkv, d)), dtype)
    sc = 1.0 / math.sqrt(d)
    out = torch.empty((B, Hq, d), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    gts = torch.empty((B, Hq), dtype=torch.int32, device="cuda")
    promoted_seen = closed_seen = False
    for s in range(steps):
        q = 0.1 * rng.standard_normal((B, Hq, d))
        k_new = keys[s].copy()
        if 40 <= s < 46:      # sequence 0, group 0: logit ~8 on token 3 (cold since step 19)
            q[0, :G] = (8.0 / math.sqrt(d)) * keys[3, 0, 0]
        if 25 <= s < 28 and math.isfinite(gate):
            # sequence 1, group 0: the step's token has norm 40 along u and the group's queries
            # are 5 u (logit 200 / sqrt(d), far above the gate); later random queries give it
            # logits of about 0.5 / sqrt(d / 64) standard deviations
            u = rng.standard_normal(d)
            u /= np.linalg.norm(u)
            k_new[1, 0] = MO.round_to(40.0 * u, dtype)
            q[1, :G] = 5.0 * u
        qt = torch.tensor(q, dtype=torch.float32, device="cuda")
        kt = torch.tensor(k_new, dtype=_DT[dtype], device="cuda")
        vt = torch.tensor(vals[s], dtype=_DT[dtype], device="cuda")
        # oracle first (its values check the margins), then the GPU step
        hot_before = [x.copy() for x in ora.hot_k]
        ro, rl, rg, w = ora.step(q, k_new, vals[s], Wn, gate, 0.15, 3)
        for b in range(B):
            assert np.all(np.abs(w[b] - 0.15) > 0.02), f"step {s}: a cold weight is near the threshold"
            hk = np.concatenate([hot_before[b], k_new[b][:, None]], axis=1)
            for hq in range(Hq):
                mx = np.max(sc * (hk[hq // G] @ q[b, hq]))
                assert not math.isfinite(gate) or abs(mx - gate) > 0.5, f"step {s}: a gate is near its threshold"
        tq.monarch_step(h, st, qt, kt, vt, Wn, cold_gate=gate, promote_weight=0.15, promote_steps=3,
                        out=out, lse=lse, gate_out=gts)
        torch.cuda.synchronize()
        assert np.array_equal(gts.cpu().numpy() != 0, rg), f"step {s}: gates"
        _close(out.cpu().numpy(), ro, f"step {s} out")
        _close(lse.cpu().numpy(), rl, f"step {s} lse")
        hs, hl = st.hot_start.cpu().numpy(), st.hot_len.cpu().numpy()
        cl, hits = st.cold_len.cpu().numpy(), st.hits.cpu().numpy()
        hkg, hvg, rec = st.hot_k.float().cpu().numpy(), st.hot_v.float().cpu().numpy(), st.records.cpu().numpy()
        for b in range(B):
            assert hl[b] == ora.hot_k[b].shape[1] and cl[b] == ora.cold[b].shape[1], f"step {s}: lengths"
            ring = (hs[b] + np.arange(hl[b])) % hot_cap
            assert np.array_equal(hkg[b][:, ring], ora.hot_k[b]), f"step {s}: hot keys"
            assert np.array_equal(hvg[b][:, ring], ora.hot_v[b]), f"step {s}: hot values"
            assert np.array_equal(rec[b][:, :cl[b]], ora.cold[b]), f"step {s}: cold records"
            assert np.array_equal(hits[b][:cl[b]], ora.hits[b]), f"step {s}: sticky counts"
        promoted_seen = promoted_seen or any(len(x) and np.max(x) > 0.5 for x in w)
        closed_seen = closed_seen or not rg.all()
    assert promoted_seen, "the planted token never drew the attention"
    assert closed_seen or not math.isfinite(gate), "no gate ever closed"
    assert np.array_equal(st.overflow.cpu().numpy() != 0, np.array(ora.overflow))
