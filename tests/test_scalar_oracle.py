"""Pins of the scalar C oracle (oracle/tq_scalar.c) against facts fixed outside it, and its
agreement with the numpy oracle written separately from the same definitions.

The pins are the ones the C oracle must meet on its own: published generator outputs and a
hand-worked Box-Muller pair, an orthogonal rotation that keeps norms to 1e-6, Max's (1960)
Gaussian quantizer tables and the 1-bit closed form, distortion falling with every added
bit, hand-worked packed bytes, QJL estimates unbiased over 10^4 seeded sketches within 3
standard errors, brute-force softmax attention on tiny inputs, textbook attention for exact
tokens, and brute-force top-k with ties.  The agreement tests then hold the two oracles to
each other: records byte for byte, attention within 1e-12, sign index and top-k bit-exact.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import scalar as S
from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- generator ----------
def test_splitmix64_reference_vector():
    g = _golden("splitmix64_seed0.json")
    assert [f"{int(x):016x}" for x in S.splitmix64(g["seed"], 3)] == g["first_outputs_hex"]


def test_box_muller_first_pair_worked_by_hand():
    g = _golden("box_muller_seed0_pair0.json")
    w = S.splitmix64(g["seed"], 2)
    assert [int(w[0]), int(w[1])] == [int(g["w0_hex"], 16), int(g["w1_hex"], 16)]
    got = S.gaussians(g["seed"], 2)
    want = np.array([float(g["g0_cos"]), float(g["g1_sin"])])
    assert np.all(np.abs(got - want) <= 4e-16 * np.abs(want)), (got, want)
    assert np.array_equal(S.gaussians(9, 5), S.gaussians(9, 6)[:5])


def test_gaussians_are_standard_normal():
    n = 200_000
    x = S.gaussians(12345, n)
    assert abs(x.mean()) < 4.0 / math.sqrt(n)
    assert abs(x.var() - 1.0) < 4.0 * math.sqrt(2.0 / n)
    assert stats.kstest(x, "norm").pvalue > 1e-4


# ---------------------------------------------------------------- rotation -----------
@pytest.mark.parametrize("d", [1, 8, 64, 128, 200])
def test_rotation_is_orthogonal_keeps_norms_and_has_positive_r_diagonal(d):
    Pi = S.rotation(77, d).astype(np.float64)
    assert np.abs(Pi.T @ Pi - np.eye(d)).max() <= 1e-6
    G = S.gaussians(77, d * d).reshape(d, d)
    R = Pi.T @ G                       # G = Pi R, R upper triangular with a positive diagonal
    assert np.all(np.diag(R) > 0)
    assert np.abs(np.tril(R, -1)).max(initial=0.0) <= 1e-5 * np.abs(R).max()
    x = np.random.default_rng(d).standard_normal((100, d))
    ratio = np.linalg.norm(x @ Pi.T, axis=1) / np.linalg.norm(x, axis=1)
    assert np.abs(ratio - 1.0).max() <= 1e-6


def test_qjl_matrix_is_the_gaussian_stream():
    Sm = S.qjl_matrix(5, 16, 8)
    assert np.array_equal(Sm, S.gaussians(5, 128).reshape(16, 8).astype(np.float32))


# ---------------------------------------------------------------- codebooks ----------
def test_lloyd_max_one_bit_closed_form():
    lev, bnd = S.lloyd_max(1)
    assert np.allclose(lev, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=0, atol=1e-14)
    assert bnd[0] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960_table_and_lloyds_conditions(bits):
    t = _golden("lloyd_max_gaussian_max1960.json")["tables"][str(bits)]
    lev, bnd = S.lloyd_max(bits)
    half = len(lev) // 2
    assert np.allclose(lev[half:], t["levels"], rtol=0, atol=6e-4)
    assert np.allclose(bnd[half - 1:], t["bounds"], rtol=0, atol=6e-4)
    assert np.array_equal(lev, -lev[::-1])
    edges = [-np.inf] + list(bnd) + [np.inf]
    pdf = stats.norm.pdf
    for k in range(len(lev)):
        mass = integrate.quad(pdf, edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-13)[0]
        mom = integrate.quad(lambda x: x * pdf(x), edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(mom / mass - lev[k]) < 1e-9


def _stage1_distortion(bits, d=128, n=3000):
    """Relative distortion |k - Pi^T x_hat|^2 / |k|^2 of the codes read back from records."""
    c = S.ScalarCodec(d, bits, 0, bits, 3, 4)
    t = c.tables()
    k = np.random.default_rng(bits).standard_normal((n, d)).astype(np.float32)
    f = c.unpack(c.compress(k, k))
    xhat = (f["r_k"].astype(np.float64) / math.sqrt(d))[:, None] * t["key_levels"].astype(np.float64)[f["kc"]]
    khat = xhat @ t["Pi"].astype(np.float64)
    kk = k.astype(np.float64)
    return float(np.mean(np.sum((kk - khat) ** 2, 1) / np.sum(kk * kk, 1)))


def test_quantization_distortion_falls_with_every_bit_and_sits_at_the_gaussian_table():
    table = _golden("lloyd_max_gaussian_max1960.json")["tables"]
    rel = [_stage1_distortion(b) for b in (1, 2, 3, 4)]
    assert all(a > b for a, b in zip(rel, rel[1:])), rel
    for b, r in zip((1, 2, 3, 4), rel):
        assert 0.93 * table[str(b)]["mse"] <= r <= 1.0 * table[str(b)]["mse"], (b, r)


# ---------------------------------------------------------------- packing ------------
def test_pack_matches_hand_worked_bytes():
    """Codes placed through quantize_from_rotated (z at a level lies inside that level's cell)."""
    for case in _golden("pack_example.json")["cases"]:
        b, codes = case["bits"], np.array(case["codes"])
        c = S.ScalarCodec(32, b, 0, 4, 1, 2)
        lev = c.tables()["key_levels"]
        z = np.zeros((1, 32), np.float32)
        z[0, :len(codes)] = lev[codes]
        z[0, len(codes):] = lev[0]
        rec = c.quantize_from_rotated(z, np.zeros((1, 0)), [1.0], [0.0], np.zeros((1, 32)), [1.0])
        nbytes = len(case["bytes_hex"]) // 2
        assert rec[0, :nbytes].tobytes().hex() == case["bytes_hex"], case


@pytest.mark.parametrize("cfg,size", [((128, 3, 128, 4), 144), ((64, 3, 64, 4), 80),
                                      ((128, 4, 0, 4), 144), ((128, 2, 128, 2), 96), ((200, 3, 192, 2), 176)])
def test_record_layout(cfg, size):
    c = S.ScalarCodec(*cfg, 1, 2)
    assert c.record_bytes == size
    d = cfg[0]
    rng = np.random.default_rng(0)
    k, v = rng.standard_normal((5, d)).astype(np.float32), rng.standard_normal((5, d)).astype(np.float32)
    rec = c.compress(k, v)
    f = c.unpack(rec)
    assert np.array_equal(f["r_k"], np.linalg.norm(k.astype(np.float64), axis=1).astype(np.float32))
    assert np.array_equal(f["r_v"], np.linalg.norm(v.astype(np.float64), axis=1).astype(np.float32))
    kb = (d * cfg[1] // 8 + 3) // 4 * 4
    vb = (d * cfg[3] // 8 + 3) // 4 * 4
    assert np.all(rec[:, kb + cfg[2] // 8 + vb + 12:] == 0)


def test_zero_vector_reading_and_boundary_goes_up():
    c = S.ScalarCodec(64, 3, 64, 4, 1, 2)
    f = c.unpack(c.compress(np.zeros((1, 64)), np.zeros((1, 64))))
    assert np.all(f["kc"] == 4) and np.all(f["vc"] == 8) and np.all(f["bits"] == 1)
    assert f["r_k"][0] == 0 and f["rho"][0] == 0 and f["r_v"][0] == 0
    t = c.tables()["key_bounds"]
    z = np.full((1, 64), 0.0, np.float32)
    z[0, :7] = [t[0], np.nextafter(t[0], np.float32(-10)), 0.0, -0.0, t[-1], 100, -100]
    f = c.unpack(c.quantize_from_rotated(z, np.zeros((1, 64)), [1.0], [0.0], z, [1.0]))
    assert f["kc"][0, :7].tolist() == [1, 0, 4, 4, 7, 7, 0]


# ---------------------------------------------------------------- QJL ----------------
def test_qjl_estimate_is_unbiased_over_ten_thousand_sketches():
    """TurboQuant explainer, "Stufe 2": the 1-bit residual sketch gives an unbiased inner
    product.  10^4 codecs share the rotation and differ in the QJL seed only; the mean of
    the estimate minus <q, k> lies within 3 standard errors of 0."""
    d = 32
    rng = np.random.default_rng(2024)
    k = rng.standard_normal((1, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    exact = float(q.astype(np.float64) @ k[0].astype(np.float64))
    errs = np.empty(10_000)
    for s in range(len(errs)):
        c = S.ScalarCodec(d, 2, d, 2, 11, 1000 + s)
        rec = c.compress(k, k)
        _, _, lg = c.decode_head(q, rec, 1, scale=1.0, want_logits=True)
        errs[s] = lg[0] - exact
    se = errs.std(ddof=1) / math.sqrt(len(errs))
    assert abs(errs.mean()) <= 3 * se, (errs.mean(), se)
    assert errs.std() > 0.01                    # the sketch does vary


# ---------------------------------------------------------------- attention ----------
@pytest.mark.parametrize("d,T,Hq", [(8, 5, 2), (16, 3, 1), (8, 1, 4)])
def test_decode_equals_brute_force_attention_on_effective_keys(d, T, Hq):
    """k~ = Pi^T [x_hat + (sqrt(pi/2) rho / m) S^T (2 bit - 1)], v^ = Pi^T x_hat_v, then plain
    softmax attention, exact tokens in the same softmax."""
    rng = np.random.default_rng(d * 10 + T)
    c = S.ScalarCodec(d, 3, d, 2, 21, 22)
    t = c.tables()
    Pi, Sm = t["Pi"].astype(np.float64), t["S"].astype(np.float64)
    B, Hkv, nh = 2, 1, 2
    K = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    hk = rng.standard_normal((B, Hkv, nh, d)).astype(np.float32)
    hv = rng.standard_normal((B, Hkv, nh, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    rec = c.compress_cache(K, V)
    out, lse, _ = c.decode_attention(q, rec, [T, T], hk, hv, [nh, nh - 1])
    for b in range(B):
        f = c.unpack(rec[b, 0])
        xk = (f["r_k"].astype(np.float64) / math.sqrt(d))[:, None] * t["key_levels"].astype(np.float64)[f["kc"]]
        xk += (math.sqrt(math.pi / 2) * f["rho"].astype(np.float64) / d)[:, None] * ((2.0 * f["bits"] - 1.0) @ Sm)
        xv = (f["r_v"].astype(np.float64) / math.sqrt(d))[:, None] * t["val_levels"].astype(np.float64)[f["vc"]]
        n_hot = [nh, nh - 1][b]
        kall = np.concatenate([xk @ Pi, hk[b, 0, :n_hot].astype(np.float64)])
        vall = np.concatenate([xv @ Pi, hv[b, 0, :n_hot].astype(np.float64)])
        for h in range(Hq):
            lg = kall @ q[b, h].astype(np.float64) / math.sqrt(d)
            p = np.exp(lg - lg.max())
            assert np.allclose(out[b, h], p @ vall / p.sum(), rtol=1e-12, atol=1e-13)
            assert abs(lse[b, h] - (lg.max() + math.log(p.sum()))) < 1e-12


def test_exact_segment_alone_is_textbook_attention_and_empty_is_zero():
    import torch
    rng = np.random.default_rng(3)
    c = S.ScalarCodec(64, 3, 64, 4, 1, 2)
    B, Hq, Hkv, n = 2, 8, 2, 37
    hk = rng.standard_normal((B, Hkv, n, 64)).astype(np.float32)
    hv = rng.standard_normal((B, Hkv, n, 64)).astype(np.float32)
    q = rng.standard_normal((B, Hq, 64)).astype(np.float32)
    rec = np.zeros((B, Hkv, 4, c.record_bytes), np.uint8)
    out, _, _ = c.decode_attention(q, rec, [0, 0], hk, hv, [n, n])
    kk = torch.from_numpy(hk.astype(np.float64)).repeat_interleave(Hq // Hkv, dim=1)
    vv = torch.from_numpy(hv.astype(np.float64)).repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[:, :, None], kk, vv)[:, :, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    out, lse, _ = c.decode_attention(q, rec, [0, 0])
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_gather_equals_full_and_subset_equals_its_own_cache():
    rng = np.random.default_rng(8)
    c = S.ScalarCodec(64, 3, 64, 4, 5, 6)
    K = rng.standard_normal((1, 40, 1, 64)).astype(np.float32)
    V = rng.standard_normal((1, 40, 1, 64)).astype(np.float32)
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    rec = c.compress_cache(K, V)
    full, lse, _ = c.decode_attention(q, rec, [40])
    gat, lse2, _ = c.decode_attention(q, rec, [40], sel_idx=np.arange(40)[None, None])
    assert np.allclose(full, gat, rtol=1e-13, atol=0) and np.allclose(lse, lse2, rtol=1e-13)
    sub = np.array([3, 9, 10, 31])
    g2, _, _ = c.decode_attention(q, rec, [40], sel_idx=np.concatenate([sub, [-1, -1]])[None, None])
    s2, _, _ = c.decode_attention(q, c.compress_cache(K[:, sub], V[:, sub]), [4])
    assert np.allclose(g2, s2, rtol=1e-13, atol=1e-15)


def test_score_scan_matches_decode_logits():
    rng = np.random.default_rng(4)
    c = S.ScalarCodec(64, 3, 64, 4, 5, 6)
    K = rng.standard_normal((1, 30, 2, 64)).astype(np.float32)
    rec = c.compress_cache(K, K)
    q = rng.standard_normal((1, 2, 3, 64)).astype(np.float32)
    sc = c.score_scan(q, rec, 30)
    for h in range(2):
        for i in range(3):
            _, _, lg = c.decode_attention(q[:, h, i:i + 1], rec[:, h:h + 1], [30], scale=1.0)
            assert np.allclose(sc[0, h, i], lg[(0, 0)][0], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- sign index ---------
def test_sign_index_bits_centroids_and_shift_invariance():
    rng = np.random.default_rng(5)
    T, d = 3000, 32
    k = (rng.standard_normal((T, d)) + 0.7).astype(np.float32)
    mu = S.channel_mean(k)
    assert np.allclose(mu, k.astype(np.float64).mean(0), atol=1e-6)
    idx, book = S.sign_index(k, mu)
    bits = np.unpackbits(idx, axis=1, bitorder="little")[:, :d]
    assert np.array_equal(bits.astype(bool), k >= mu)
    assert np.all(np.abs(bits.mean(0) - 0.5) < 0.05)
    pat = (bits.reshape(T, d // 4, 4) << np.arange(4)).sum(-1)
    for g in range(d // 4):
        for p in range(16):
            m = pat[:, g] == p
            if not m.any():
                assert np.all(book[g, p] == 0)
                continue
            mean = (k[m, 4 * g:4 * g + 4].astype(np.float64) - mu[4 * g:4 * g + 4]).mean(0)
            assert np.allclose(book[g, p], mean, rtol=1e-6, atol=1e-7)
    ki = rng.integers(-8, 9, size=(200, 16)).astype(np.float32)
    a = S.sign_index(ki, S.channel_mean(ki))
    b = S.sign_index(ki + 3.0, S.channel_mean(ki + 3.0))
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1], atol=1e-6)


def test_topk_equals_brute_force_sort_with_ties():
    rng = np.random.default_rng(7)
    B, T, H, d, G = 2, 60, 2, 16, 2
    K = rng.standard_normal((B, T, H, d)).astype(np.float32)
    K[:, 20:30] = K[:, 0:10]        # duplicated tokens: tied scores
    idx, book, _ = S.build_sign_index(K, T)
    q = rng.standard_normal((B, H * G, d)).astype(np.float32)
    lens = [T, 45]
    for k in (0, 1, 7, 25, 45, 80):
        sel, cnt, scs = S.select_topk(q, idx, book, lens, k)
        for b in range(B):
            for h in range(H):
                n = lens[b]
                bits = np.unpackbits(idx[b, h, :n], axis=1, bitorder="little")[:, :d]
                pat = (bits.reshape(n, d // 4, 4) << np.arange(4)).sum(-1)
                luts = []
                for j in range(G):
                    qg = q[b, h * G + j].astype(np.float64).reshape(d // 4, 1, 4)
                    cb = book[b, h].astype(np.float64)
                    luts.append(((qg[..., 0] * cb[..., 0] + qg[..., 1] * cb[..., 1]) + qg[..., 2] * cb[..., 2])
                                + qg[..., 3] * cb[..., 3])
                mx = max(np.abs(t).max() for t in luts)
                e = math.frexp(G * (d // 4) * mx)
                s = 30 - e[1] + (1 if e[0] == 0.5 else 0)
                assert G * (d // 4) * mx * 2.0 ** s <= 2 ** 30 < G * (d // 4) * mx * 2.0 ** (s + 1)
                lut = sum(np.rint(t * 2.0 ** s).astype(np.int64) for t in luts)
                ints = lut[np.arange(d // 4)[None, :], pat].sum(1)
                ranked = sorted(range(n), key=lambda t: (-ints[t], t))[:min(k, n)]
                assert cnt[b, h] == min(k, n)
                assert sel[b, h, :cnt[b, h]].tolist() == sorted(ranked)
                assert np.all(sel[b, h, cnt[b, h]:] == -1)
                assert scs[b, h, :cnt[b, h]].tolist() == [int(ints[t]) for t in sorted(ranked)]


# ---------------------------------------------------------------- agreement ----------
@pytest.mark.parametrize("cfg", [(128, 3, 128, 4), (64, 3, 64, 4), (128, 4, 0, 4), (128, 1, 128, 1),
                                 (200, 2, 192, 2), (64, 2, 32, 3), (40, 3, 0, 3)])
def test_agrees_with_the_numpy_oracle(cfg):
    """Two statements of one definition, written apart: the init tables equal (Pi to 1 ulp of
    float, the codebooks exactly), records byte for byte, logits and outputs to 1e-12."""
    d = cfg[0]
    c, o = S.ScalarCodec(*cfg, 31, 32), O.Codec(*cfg, 31, 32)
    t = c.tables()
    assert np.abs(t["Pi"].astype(np.float64) - o.Pi).max() <= 2.0 ** -24
    assert np.array_equal(t["S"], o.S)
    for a, b in (("key_levels", o.key_levels), ("key_bounds", o.key_bounds), ("val_levels", o.val_levels),
                 ("val_bounds", o.val_bounds)):
        assert np.array_equal(t[a], b), a
    rng = np.random.default_rng(d)
    k = rng.standard_normal((400, d)).astype(np.float32)
    v = (3.0 * rng.standard_t(4, (400, d))).astype(np.float32)
    k[7] = 0.0
    rec = c.compress(k, v)
    assert np.array_equal(rec, o.pack(o.compress_fields(k, v)))
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    recs = np.stack([rec, rec[::-1]])[:, None]
    hk = rng.standard_normal((2, 1, 9, d)).astype(np.float32)
    hv = rng.standard_normal((2, 1, 9, d)).astype(np.float32)
    sel = np.full((2, 1, 50), -1, np.int32)
    sel[0, 0, :40] = np.sort(rng.choice(400, 40, replace=False))
    sel[1, 0, :3] = [0, 5, 399]
    for kw in (dict(seq_lens=[400, 123]), dict(seq_lens=[400, 400], sel_idx=sel),
               dict(seq_lens=[17, 0], hot_k=hk, hot_v=hv, hot_lens=[9, 4])):
        a = c.decode_attention(q, recs, **kw)
        b = O.decode_attention(o, q, recs, **kw)
        assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
        assert np.allclose(a[1], b[1], rtol=1e-12, atol=1e-14)
        for key in b[2]:
            for x, y in zip(a[2][key], b[2][key]):
                assert np.allclose(x, y, rtol=1e-12, atol=1e-13)


def test_sign_index_and_topk_agree_with_the_numpy_oracle():
    rng = np.random.default_rng(1)
    B, T, H, d, G = 2, 3000, 2, 128, 3
    K = rng.standard_normal((B, T, H, d)).astype(np.float32)
    K[0, :, 0, 5] += 3.0
    ic, bc, mc = S.build_sign_index(K, 2500)
    io, bo, mo = O.build_sign_index(None, K, 2500)
    assert np.array_equal(mc, mo) and np.array_equal(ic, io) and np.array_equal(bc, bo)
    q = rng.standard_normal((B, H * G, d)).astype(np.float32)
    for qq in (q, np.round(2 * q) / 2):
        for k in (0, 1, 100, 2500, 4000):
            a = S.select_topk(qq, io, bo, [2500, 1700], k)
            b = O.select_topk(None, qq, io, bo, [2500, 1700], k)
            assert all(np.array_equal(x, y) for x, y in zip(a, b)), k
