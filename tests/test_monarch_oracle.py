"""Pins of the hot/cold step oracle (oracle/monarch.py) against facts fixed outside it:
brute-force attention when every head is gated to the hot region, window and eviction
invariants against the already pinned compress, the promotion rule on a planted token, the
swap-remove order, the overflow rule, and bfloat16 rounding against torch."""
import math

import numpy as np
import torch

from oracle import monarch as M
from oracle import tq_oracle as O

D = 64


def _codec():
    return O.Codec(D, 3, 64, 4, 11, 12)


def _tok(rng, n, H=1):
    return M.round_to(rng.standard_normal((n, H, D)), "float16")


def test_bf16_rounding_matches_torch_on_float32_inputs():
    x = np.random.default_rng(0).standard_normal(4096).astype(np.float32) * 10.0
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(M.round_to_bf16(x.astype(np.float64)), ref)
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)])
    assert np.array_equal(M.round_to_bf16(ties), np.array([1.0, 1.0 + 2.0 ** -6, -1.0]))


def test_window_and_eviction_follow_compress():
    c, rng = _codec(), np.random.default_rng(1)
    o = M.HotColdOracle(c, 1, 1, "float16", 100)
    ks, vs = _tok(rng, 12), _tok(rng, 12)
    q = rng.standard_normal((1, 2, D))
    for s in range(12):
        o.step(q, ks[s:s + 1], vs[s:s + 1], window=4, promote_steps=0)
        nh = o.hot_k[0].shape[1]
        assert nh == min(s + 1, 4)                                   # at most `window` hot tokens
        assert np.array_equal(o.hot_k[0][0], ks[s + 1 - nh:s + 1, 0])   # the most recent ones, exact
        ne = s + 1 - nh
        assert o.cold[0].shape[1] == ne
        if ne:                                                       # the evicted ones, compressed in order
            ref = O.pack_records(c, O.compress(c, ks[:ne, 0].astype(np.float32)[None],
                                               vs[:ne, 0].astype(np.float32)[None]))
            assert np.array_equal(o.cold[0], ref)


def test_closed_gate_is_exact_attention_over_the_hot_tokens():
    c, rng = _codec(), np.random.default_rng(2)
    o = M.HotColdOracle(c, 1, 1, "float32", 100)
    ks, vs = _tok(rng, 10), _tok(rng, 10)
    q = rng.standard_normal((1, 1, D))
    for s in range(9):
        o.step(q, ks[s:s + 1], vs[s:s + 1], window=3, promote_steps=0)
    # the last token points along q: its logit exceeds the gate, the head skips the cold tokens
    k_last = (5.0 * q[0] / np.linalg.norm(q[0]) * math.sqrt(D))[None]
    out, lse, gate, _ = o.step(q, k_last, vs[9:10], window=3, cold_gate=4.0, promote_steps=0)
    assert not gate[0, 0]
    hk = np.concatenate([ks[7:9, 0], k_last[:, 0]])
    hv = vs[7:10, 0]
    lg = (hk @ q[0, 0]) / math.sqrt(D)
    p = np.exp(lg - lg.max())
    assert np.allclose(out[0, 0], (p @ hv) / p.sum(), rtol=1e-12, atol=1e-12)
    assert math.isclose(lse[0, 0], lg.max() + math.log(p.sum()), rel_tol=1e-12)


def test_planted_token_is_promoted_after_three_steps():
    c, rng = _codec(), np.random.default_rng(3)
    o = M.HotColdOracle(c, 1, 1, "float16", 100)
    ks, vs = _tok(rng, 30), _tok(rng, 30)
    q0 = rng.standard_normal((1, 1, D))
    for s in range(10):                          # no promotion yet: cold slot t holds token t
        o.step(q0, ks[s:s + 1], vs[s:s + 1], window=4, promote_steps=0)
    target = 2
    rec = o.cold[0][0, target].copy()
    q = (6.0 * ks[target, 0] / np.linalg.norm(ks[target, 0]) * math.sqrt(D) / 8.0)[None, None]
    n_cold = o.cold[0].shape[1]
    for s in range(10, 13):
        _, _, gate, w = o.step(q, ks[s:s + 1], vs[s:s + 1], window=4)
        assert gate[0, 0] and w[0][target] > 0.5 and np.all(np.delete(w[0], target) < 0.15)
        if s < 12:
            assert o.hits[0][target] == s - 9 and np.all(np.delete(o.hits[0], target) == 0)
    # promoted at the third step: one cold token fewer (plus the step's eviction), the newest
    # hot token before eviction is the decompressed record, norm r_k |gamma[c]| / sqrt(d)
    f = O.unpack_records(c, rec[None])
    xk = f["r_k"][0] / math.sqrt(D) * c.key_levels.astype(np.float64)[f["kc"][0]]
    k_prom = M.round_to(c.Pi64.T @ xk, "float16")
    assert any(np.array_equal(k_prom, o.hot_k[0][0, j]) for j in range(o.hot_k[0].shape[1]))
    assert abs(np.linalg.norm(c.Pi64.T @ xk) / np.linalg.norm(xk) - 1.0) < 1e-6   # float32 Pi
    assert np.dot(k_prom, ks[target, 0]) / (np.linalg.norm(k_prom) * np.linalg.norm(ks[target, 0])) > 0.9
    assert o.cold[0].shape[1] == n_cold - 1 + 4      # one eviction per step, two with the promotion
    assert not any(np.array_equal(rec, o.cold[0][0, t]) for t in range(o.cold[0].shape[1]))


def test_swap_remove_order_and_overflow():
    c, rng = _codec(), np.random.default_rng(4)
    o = M.HotColdOracle(c, 1, 1, "float16", 8)
    ks, vs = _tok(rng, 40), _tok(rng, 40)
    q = rng.standard_normal((1, 1, D))
    for s in range(10):
        o.step(q, ks[s:s + 1], vs[s:s + 1], window=2, promote_steps=0)
    assert o.cold[0].shape[1] == 8 and not o.overflow[0]            # 10 - 2 = 8 evicted: just full
    before = o.cold[0].copy()
    o.hits[0] = np.array([0, 2, 0, 0, 2, 0, 0, 0])
    # a query that puts its weight on cold tokens 1 and 4, which then reach the third step
    f = O.unpack_records(c, before[0])
    sd = math.sqrt(D)
    khat = ((f["r_k"][:, None] / sd) * c.key_levels.astype(np.float64)[f["kc"]]) @ c.Pi64
    qv = 3.0 * sd * (khat[1] / np.linalg.norm(khat[1]) + khat[4] / np.linalg.norm(khat[4]))
    _, _, gate, w = o.step(qv[None, None], ks[10:11], vs[10:11], window=2, promote_steps=3)
    assert gate[0, 0] and w[0][1] > 0.15 and w[0][4] > 0.15 and np.all(np.delete(w[0], [1, 4]) < 0.15)
    # slots handled from the highest: 4 <- 7, then 1 <- 6; the hot region then holds
    # 2 + 1 + 2 tokens, 3 are evicted but only 2 fit: the last is dropped (overflow)
    assert np.array_equal(o.cold[0][:, 4], before[:, 7]) and np.array_equal(o.cold[0][:, 1], before[:, 6])
    assert np.array_equal(o.cold[0][:, [0, 2, 3, 5]], before[:, [0, 2, 3, 5]])
    assert o.cold[0].shape[1] == 8 and o.hot_k[0].shape[1] == 2 and o.overflow[0]
    assert np.array_equal(o.hits[0], [0, 0, 0, 0, 0, 0, 0, 0])


def _polar_codec():
    from oracle import polar as P
    return P.PolarCodec(D, 4, 64, 4, 11, 12, upper_bits=2)


def test_polar_keys_evict_through_the_polar_compress():
    """With polar key codes (the Monarch page's cold tier) eviction writes exactly the polar
    codec's records of the evicted tokens, in order."""
    c, rng = _polar_codec(), np.random.default_rng(5)
    o = M.HotColdOracle(c, 1, 2, "float16", 100)
    ks, vs = _tok(rng, 9, 2), _tok(rng, 9, 2)
    q = rng.standard_normal((1, 4, D))
    for s in range(9):
        o.step(q, ks[s:s + 1], vs[s:s + 1], window=3, promote_steps=0)
    ref = c.pack(c.compress_fields(np.transpose(ks[:6], (1, 0, 2)).astype(np.float32),
                                   np.transpose(vs[:6], (1, 0, 2)).astype(np.float32)))
    assert np.array_equal(o.cold[0], ref)


def test_polar_promoted_key_is_the_rotated_back_polar_reconstruction():
    """A promoted polar key is Pi^T (r_k u): its norm is the stored radius (u has unit norm and
    Pi is orthogonal to float32 rounding), it points along the original key, and the step's
    ring holds exactly that vector rounded to the hot dtype."""
    from oracle import polar as P
    c, rng = _polar_codec(), np.random.default_rng(6)
    o = M.HotColdOracle(c, 1, 1, "float32", 100)
    ks, vs = _tok(rng, 20), _tok(rng, 20)
    q0 = rng.standard_normal((1, 1, D))
    for s in range(8):
        o.step(q0, ks[s:s + 1], vs[s:s + 1], window=4, promote_steps=0)
    target = 1
    rec = o.cold[0][0, target].copy()
    q = (6.0 * ks[target, 0] / np.linalg.norm(ks[target, 0]) * math.sqrt(D) / 8.0)[None, None]
    for s in range(8, 11):
        _, _, gate, w = o.step(q, ks[s:s + 1], vs[s:s + 1], window=4)
        assert gate[0, 0] and w[0][target] > 0.5
    f = c.unpack(rec[None])
    ang = [c.angle_levels[l].astype(np.float64)[f["kc"][l][0]] for l in range(c.L)]
    u = P.polar_inverse(np.ones(()), ang)
    assert abs(np.linalg.norm(u) - 1.0) < 1e-14
    k_prom = M.round_to(c.Pi64.T @ (float(f["r_k"][0]) * u), "float32")
    assert any(np.array_equal(k_prom, o.hot_k[0][0, j]) for j in range(o.hot_k[0].shape[1]))
    assert abs(np.linalg.norm(k_prom) / f["r_k"][0] - 1.0) < 1e-6
    assert np.dot(k_prom, ks[target, 0]) / (np.linalg.norm(k_prom) * np.linalg.norm(ks[target, 0])) > 0.9
