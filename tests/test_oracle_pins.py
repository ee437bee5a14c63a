"""Pins of the oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, a published table, a library routine, a
statistical property the pages state, or a brute-force construction on tiny inputs, so
that a dropped term, a wrong sign or index, or a transposed operand fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- generator ----------
def test_splitmix64_reference_vector():
    g = _golden("splitmix64_seed0.json")
    got = [f"{x:016x}" for x in O.splitmix64(g["seed"], 3)]
    assert got == g["first_outputs_hex"]


def test_box_muller_first_pair_worked_by_hand():
    """The first two normals of seed 0 equal the pair worked by hand from the SplitMix64
    reference words (golden file): pins the word-to-uniform mapping (>> 11, the + 1 of u1,
    2^-53), which word feeds the radius, and the cos-then-sin order."""
    g = _golden("box_muller_seed0_pair0.json")
    w0, w1 = int(g["w0_hex"], 16), int(g["w1_hex"], 16)
    assert [w0, w1] == O.splitmix64(g["seed"], 2)
    assert (w0 >> 11) + 1 == g["u1_numerator"] and w1 >> 11 == g["u2_numerator"]
    got = O.gaussians(g["seed"], 2)
    want = np.array([float(g["g0_cos"]), float(g["g1_sin"])])
    assert np.all(np.abs(got - want) <= 4e-16 * np.abs(want)), (got, want)


def test_box_muller_gaussians_are_standard_normal():
    n = 200_000
    x = O.gaussians(12345, n)
    assert abs(x.mean()) < 4.0 / math.sqrt(n)
    assert abs(x.var() - 1.0) < 4.0 * math.sqrt(2.0 / n)
    assert stats.kstest(x, "norm").pvalue > 1e-4
    # odd n uses the first value of the last pair
    assert np.array_equal(O.gaussians(9, 5), O.gaussians(9, 6)[:5])


# ---------------------------------------------------------------- rotation -----------
@pytest.mark.parametrize("d", [1, 8, 64, 128])
def test_rotation_is_orthogonal_with_positive_r_diagonal(d):
    Pi = O.rotation(77, d).astype(np.float64)
    assert np.abs(Pi.T @ Pi - np.eye(d)).max() <= 1e-6
    G = O.gaussians(77, d * d).reshape(d, d)
    R = Pi.T @ G                       # G = Pi R with R upper triangular, diag(R) > 0
    assert np.all(np.diag(R) > 0)
    assert np.abs(np.tril(R, -1)).max(initial=0.0) <= 1e-5 * np.abs(R).max()
    x = np.random.default_rng(d).standard_normal((100, d))
    ratio = np.linalg.norm(x @ Pi.T, axis=1) / np.linalg.norm(x, axis=1)
    assert np.abs(ratio - 1.0).max() <= 1e-6
    assert np.array_equal(O.rotation(77, d), O.rotation(77, d))
    if d > 1:
        assert not np.array_equal(O.rotation(77, d), O.rotation(78, d))


def test_qjl_matrix_is_the_gaussian_stream():
    S = O.qjl_matrix(5, 16, 8)
    assert S.shape == (16, 8) and S.dtype == np.float32
    assert np.array_equal(S, O.gaussians(5, 128).reshape(16, 8).astype(np.float32))


# ---------------------------------------------------------------- codebooks ----------
def test_lloyd_max_one_bit_closed_form():
    lev, bnd = O.lloyd_max(1)
    assert np.allclose(lev, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=0, atol=1e-14)
    assert bnd[0] == 0.0
    assert abs(O.quantizer_mse(lev, bnd) - (1 - 2 / math.pi)) < 1e-14


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960_table(bits):
    t = _golden("lloyd_max_gaussian_max1960.json")["tables"][str(bits)]
    lev, bnd = O.lloyd_max(bits)
    half = len(lev) // 2
    assert np.allclose(lev[half:], t["levels"], rtol=0, atol=6e-4)
    assert np.allclose(bnd[half - 1:], t["bounds"], rtol=0, atol=6e-4)
    assert abs(O.quantizer_mse(lev, bnd) - t["mse"]) <= 1e-3 * t["mse"]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_conditions_by_quadrature(bits):
    lev, bnd = O.lloyd_max(bits)
    assert np.array_equal(lev, -lev[::-1])          # odd symmetry, exact
    assert bnd[len(bnd) // 2] == 0.0
    assert np.allclose(bnd, 0.5 * (lev[:-1] + lev[1:]), rtol=0, atol=1e-15)
    edges = [-np.inf] + list(bnd) + [np.inf]
    pdf = stats.norm.pdf
    mse = 0.0
    for k in range(len(lev)):
        mass = integrate.quad(pdf, edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-13)[0]
        mom = integrate.quad(lambda x: x * pdf(x), edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(mom / mass - lev[k]) < 1e-9       # level = conditional mean of its cell
        mse += integrate.quad(lambda x: (x - lev[k]) ** 2 * pdf(x), edges[k], edges[k + 1],
                              epsabs=1e-14, epsrel=1e-12)[0]
    assert abs(mse - O.quantizer_mse(lev, bnd)) < 1e-10


def test_quantizer_mse_strictly_decreases_with_bits():
    mses = [O.quantizer_mse(*O.lloyd_max(b, tol=1e-10, max_iter=3000)) for b in range(1, 9)]
    assert all(a > b for a, b in zip(mses, mses[1:])), mses


def _dequantize_keys(codec, f):
    """k_hat = Pi^T x_hat with x_hat = (r / sqrt(d)) gamma[c] (codes only)."""
    d = codec.head_dim
    xhat = (f["r_k"].astype(np.float64) / math.sqrt(d))[:, None] * codec.key_levels.astype(np.float64)[f["kc"]]
    return xhat @ codec.Pi64


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_rotated_quantizer_distortion_matches_gaussian_table(bits):
    """Rotated unit-vector coordinates are close to N(0, 1/d), so the relative distortion
    of rotate+quantize at d = 128 sits just under the N(0, 1) table value."""
    codec = O.Codec(128, bits, 0, bits, 3, 4)
    k = np.random.default_rng(bits).standard_normal((4000, 128))
    f = O.compress(codec, k, k)
    khat = _dequantize_keys(codec, f)
    rel = np.mean(np.sum((k - khat) ** 2, 1) / np.sum(k * k, 1))
    table = O.quantizer_mse(*O.lloyd_max(bits))
    assert 0.93 * table <= rel <= 1.0 * table, (rel, table)


def test_code_on_a_boundary_goes_up():
    _, bnd = O.lloyd_max(3)
    b32 = bnd.astype(np.float32)
    z = np.array([b32[0], np.nextafter(b32[0], np.float32(-10)), 0.0, -0.0, b32[-1], 100, -100],
                 np.float32)
    assert O.quantize(z, b32).tolist() == [1, 0, 4, 4, 7, 7, 0]


# ---------------------------------------------------------------- packing ------------
def test_pack_matches_hand_worked_bytes():
    for case in _golden("pack_example.json")["cases"]:
        got = O._pack_stream(np.array([case["codes"]]), case["bits"])[0]
        assert got.tobytes().hex() == case["bytes_hex"], case


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_unpack_roundtrip(bits):
    c = np.random.default_rng(bits).integers(0, 1 << bits, size=(7, 128))
    assert np.array_equal(O._unpack_stream(O._pack_stream(c, bits), 128, bits), c)


@pytest.mark.parametrize("n", [8, 16, 72])
def test_pack_unpack_roundtrip_partial_3bit_group(n):
    c = np.random.default_rng(n).integers(0, 8, size=(5, n))
    buf = O._pack_stream(c, 3)
    assert buf.shape[-1] == 3 * n // 8
    assert np.array_equal(O._unpack_stream(buf, n, 3), c)


def test_3bit_group_bytes_are_selectors():
    """The property the 3-bit grouped layout exists for: read as words, (W_p >> 3s) masked by
    0x07070707 holds codes 8p + 4s + k in byte k, and the top two bits of the three words
    assemble codes 24..31 the same way."""
    c = np.random.default_rng(7).integers(0, 8, size=(32,))
    w = O._pack_stream(c[None], 3)[0].view("<u4").astype(np.int64)
    def bytes_of(x):
        return [(x >> (8 * k)) & 0xFF for k in range(4)]
    for p in range(3):
        for s in range(2):
            assert bytes_of((w[p] >> (3 * s)) & 0x07070707) == list(c[8 * p + 4 * s: 8 * p + 4 * s + 4])
    t = ((w[0] >> 6) & 0x03030303) | ((w[1] >> 4) & 0x0C0C0C0C) | ((w[2] >> 2) & 0x30303030)
    assert bytes_of(t & 0x07070707) == list(c[24:28])
    assert bytes_of((t >> 3) & 0x07070707) == list(c[28:32])


@pytest.mark.parametrize("cfg,size", [((128, 3, 128, 4), 144), ((64, 3, 64, 4), 80),
                                      ((128, 4, 0, 4), 144), ((128, 2, 128, 2), 96)])
def test_record_layout(cfg, size):
    codec = O.Codec(*cfg, 1, 2)
    assert codec.record_bytes == size
    rng = np.random.default_rng(0)
    k, v = rng.standard_normal((5, cfg[0])), rng.standard_normal((5, cfg[0]))
    f = O.compress(codec, k, v)
    rec = O.pack_records(codec, f)
    off = codec.kbytes + codec.sbytes + codec.vbytes
    norms = np.frombuffer(rec[:, off:off + 12].tobytes(), "<f4").reshape(5, 3)
    assert np.array_equal(norms[:, 0], np.linalg.norm(k, axis=1).astype(np.float32))
    assert np.array_equal(norms[:, 2], np.linalg.norm(v, axis=1).astype(np.float32))
    assert np.all(rec[:, off + 12:] == 0)
    g = O.unpack_records(codec, rec)
    for key in f:
        assert np.array_equal(f[key], g[key]), key


def test_zero_vector_reading():
    codec = O.Codec(64, 3, 64, 4, 1, 2)
    f = O.compress(codec, np.zeros((1, 64)), np.zeros((1, 64)))
    assert np.all(f["kc"] == 4) and np.all(f["vc"] == 8)
    assert f["r_k"][0] == 0 and f["rho"][0] == 0 and f["r_v"][0] == 0
    assert np.all(f["bits"] == 1)


# ---------------------------------------------------------------- QJL ----------------
def test_qjl_estimator_is_unbiased_with_closed_form_variance():
    """TurboQuant explainer, "Stufe 2": the 1-bit residual sketch is an unbiased estimator.
    Over 10^4 independent Gaussian sketches S (the codes do not depend on S) the mean of
    s_hat - <q, k> lies within 3 standard errors of 0, and its variance is
    (rho^2/m) (pi/2 |q_x|^2 - (q_x . e / rho)^2)."""
    d = m = 128
    codec = O.Codec(d, 3, m, 4, 11, 12)
    rng = np.random.default_rng(2024)
    k = rng.standard_normal(d)
    q = rng.standard_normal(d)
    exact = float(q @ k)
    qx = codec.Pi64 @ q
    # residual (independent of S)
    r = np.linalg.norm(k)
    x = codec.Pi64 @ k
    c = O.quantize((x * (math.sqrt(d) / r)).astype(np.float32), codec.key_bounds)
    e = x - (np.float64(np.float32(r)) / math.sqrt(d)) * codec.key_levels.astype(np.float64)[c]
    rho = np.linalg.norm(e)
    errs = []
    for t in range(10_000):
        codec.S = rng.standard_normal((m, d)).astype(np.float32)
        codec.S64 = codec.S.astype(np.float64)
        f = O.compress(codec, k[None], k[None])
        qx_, qs = O.prepare_query(codec, q)
        errs.append(O.score_estimates(codec, qx_, qs, f)[0] - exact)
    errs = np.array(errs)
    se = errs.std(ddof=1) / math.sqrt(len(errs))
    assert abs(errs.mean()) <= 3 * se, (errs.mean(), se)
    var_cf = rho ** 2 / m * (math.pi / 2 * (qx @ qx) - (qx @ e / rho) ** 2)
    assert abs(errs.var(ddof=1) / var_cf - 1) <= 0.06, (errs.var(), var_cf)


# ---------------------------------------------------------------- attention ----------
@pytest.mark.parametrize("d,T,H", [(8, 5, 2), (16, 3, 1), (8, 1, 4)])
def test_decode_equals_brute_force_attention_on_effective_keys(d, T, H):
    """Tiny inputs: build explicit effective keys
    k~ = Pi^T [x_hat + (sqrt(pi/2) rho / m) S^T (2 bit - 1)] and values v^ = Pi^T x_hat_v,
    then plain softmax attention (with exact hot tokens in the same softmax)."""
    rng = np.random.default_rng(d * 10 + T)
    codec = O.Codec(d, 3, d, 2, 21, 22)
    B, Hkv, nh = 2, 1, 2
    Hq = H
    K = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    hk = rng.standard_normal((B, Hkv, nh, d)).astype(np.float32)
    hv = rng.standard_normal((B, Hkv, nh, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    rec = O.compress_cache(codec, K, V)
    out, lse, _ = O.decode_attention(codec, q, rec, [T, T], hk, hv, [nh, nh - 1])
    for b in range(B):
        f = O.unpack_records(codec, rec[b, 0])
        xk = (f["r_k"].astype(np.float64) / math.sqrt(d))[:, None] * codec.key_levels.astype(np.float64)[f["kc"]]
        xk += (math.sqrt(math.pi / 2) * f["rho"].astype(np.float64) / d)[:, None] * \
            ((2.0 * f["bits"] - 1.0) @ codec.S64)
        keff = xk @ codec.Pi64
        xv = (f["r_v"].astype(np.float64) / math.sqrt(d))[:, None] * codec.val_levels.astype(np.float64)[f["vc"]]
        veff = xv @ codec.Pi64
        n_hot = [nh, nh - 1][b]
        kall = np.concatenate([keff, hk[b, 0, :n_hot].astype(np.float64)])
        vall = np.concatenate([veff, hv[b, 0, :n_hot].astype(np.float64)])
        for h in range(Hq):
            lg = kall @ q[b, h].astype(np.float64) / math.sqrt(d)
            p = np.exp(lg - lg.max())
            ref = p @ vall / p.sum()
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)
            assert abs(lse[b, h] - (lg.max() + math.log(p.sum()))) < 1e-12


def test_exact_segment_alone_is_textbook_attention():
    import torch
    rng = np.random.default_rng(3)
    codec = O.Codec(64, 3, 64, 4, 1, 2)
    B, Hq, Hkv, n = 2, 8, 2, 37
    hk = rng.standard_normal((B, Hkv, n, 64))
    hv = rng.standard_normal((B, Hkv, n, 64))
    q = rng.standard_normal((B, Hq, 64))
    rec = np.zeros((B, Hkv, 4, codec.record_bytes), np.uint8)
    out, _, _ = O.decode_attention(codec, q, rec, [0, 0], hk, hv, [n, n])
    kk = torch.from_numpy(hk).repeat_interleave(Hq // Hkv, dim=1)
    vv = torch.from_numpy(hv).repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], kk, vv)[:, :, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_empty_cache_gives_zero_output_and_minus_inf_lse():
    codec = O.Codec(64, 3, 64, 4, 1, 2)
    rec = np.zeros((1, 1, 4, codec.record_bytes), np.uint8)
    out, lse, _ = O.decode_attention(codec, np.ones((1, 2, 64)), rec, [0])
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_logit_shift_invariance_and_gather_equals_full():
    rng = np.random.default_rng(8)
    codec = O.Codec(64, 3, 64, 4, 5, 6)
    K = rng.standard_normal((1, 40, 1, 64))
    V = rng.standard_normal((1, 40, 1, 64))
    q = rng.standard_normal((1, 2, 64))
    rec = O.compress_cache(codec, K, V)
    full, lse, _ = O.decode_attention(codec, q, rec, [40])
    sel = np.arange(40)[None, None]
    gat, lse2, _ = O.decode_attention(codec, q, rec, [40], sel_idx=sel)
    assert np.allclose(full, gat, rtol=1e-13, atol=0) and np.allclose(lse, lse2, rtol=1e-13)
    # a gather of a subset equals attention over a cache holding only that subset
    sub = np.array([3, 9, 10, 31])
    g2, _, _ = O.decode_attention(codec, q, rec, [40], sel_idx=np.concatenate([sub, [-1, -1]])[None, None])
    r2 = O.compress_cache(codec, K[:, sub], V[:, sub])
    s2, _, _ = O.decode_attention(codec, q, r2, [4])
    assert np.allclose(g2, s2, rtol=1e-13, atol=1e-15)
    # a larger logit scale sharpens the distribution toward the arg-max token
    o_sharp, _, lg = O.decode_attention(codec, q, rec, [40], scale=50.0)
    t = int(np.argmax(lg[(0, 0)][0]))
    vhat = O.value_sum_rotated(codec, O.unpack_records(codec, rec[0, 0, t:t + 1]), np.ones(1))
    assert np.allclose(o_sharp[0, 0], codec.Pi64.T @ vhat, atol=1e-3)


def test_score_scan_matches_decode_logits():
    rng = np.random.default_rng(4)
    codec = O.Codec(64, 3, 64, 4, 5, 6)
    K = rng.standard_normal((1, 30, 2, 64))
    rec = O.compress_cache(codec, K, K)
    q = rng.standard_normal((1, 2, 3, 64))
    sc = O.score_scan(codec, q, rec, 30)
    for h in range(2):
        for i in range(3):
            _, _, lg = O.decode_attention(codec, q[:, h, i:i + 1], rec[:, h:h + 1], [30], scale=1.0)
            assert np.allclose(sc[0, h, i], lg[(0, 0)][0], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- sign index ---------
def test_sign_index_centroids_and_balance():
    rng = np.random.default_rng(5)
    B, T, H, d = 1, 3000, 2, 32
    K = (rng.standard_normal((B, T, H, d)) + 0.7).astype(np.float32)   # offset: centring matters
    codec = O.Codec(d, 3, 0, 4, 1, 2)
    idx, book, mu = O.build_sign_index(codec, K, T)
    for h in range(H):
        k = K[0, :, h].astype(np.float64)
        assert np.allclose(mu[0, h], k.mean(0), atol=1e-6)
        pat = O._unpack_stream(idx[0, h], d // 4, 4)
        bits = ((pat[:, :, None] >> np.arange(4)) & 1).reshape(T, d)
        assert np.all(bits == (K[0, :, h] >= mu[0, h]))
        assert np.all(np.abs(bits.mean(0) - 0.5) < 0.05)   # ~ half the signs positive
        for g in range(d // 4):
            for p in range(16):
                m = pat[:, g] == p
                resid = (k[m, 4 * g:4 * g + 4] - mu[0, h, 4 * g:4 * g + 4]) - book[0, h, g, p]
                assert np.all(np.abs(resid.sum(0)) <= 1e-5 * max(1, m.sum()))
                if not m.any():
                    assert np.all(book[0, h, g, p] == 0)
                else:   # each member's sub-vector signs agree with its pattern
                    assert np.all(((book[0, h, g, p] >= 0) == ((p >> np.arange(4)) & 1).astype(bool))
                                  | (np.abs(book[0, h, g, p]) < 1e-6))


def test_sign_index_is_invariant_to_a_constant_shift():
    """Self-Indexing page, "Methodologie" 2: centring by the channel mean does not change the
    index (softmax invariance makes the shift irrelevant to attention)."""
    rng = np.random.default_rng(6)
    K = rng.integers(-8, 9, size=(1, 200, 1, 16)).astype(np.float32)
    codec = O.Codec(16, 3, 0, 4, 1, 2)
    a = O.build_sign_index(codec, K, 200)
    b = O.build_sign_index(codec, K + 3.0, 200)
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1], atol=1e-6)


def test_topk_equals_brute_force_sort_with_ties():
    rng = np.random.default_rng(7)
    B, T, H, d, G = 2, 60, 2, 16, 2
    K = rng.standard_normal((B, T, H, d)).astype(np.float32)
    K[:, 20:30] = K[:, 0:10]        # duplicated tokens -> tied scores
    codec = O.Codec(d, 3, 0, 4, 1, 2)
    idx, book, _ = O.build_sign_index(codec, K, T)
    q = rng.standard_normal((B, H * G, d)).astype(np.float32)
    lens = [T, 45]
    for k in (1, 7, 25, 45, 80):
        sel, cnt, scs = O.select_topk(codec, q, idx, book, lens, k)
        for b in range(B):
            for h in range(H):
                n = lens[b]
                pat = O._unpack_stream(idx[b, h, :n], d // 4, 4)
                # direct float scores, to validate the integer table within its rounding
                direct = np.zeros(n)
                for j in range(G):
                    qg = q[b, h * G + j].astype(np.float64).reshape(d // 4, 4)
                    direct += np.array([sum(qg[g] @ book[b, h, g, pat[t, g]] for g in range(d // 4))
                                        for t in range(n)])
                luts = [np.einsum("gk,gpk->gp", q[b, h * G + j].astype(np.float64).reshape(d // 4, 4),
                                  book[b, h].astype(np.float64)) for j in range(G)]
                s = O.lut_scale_exponent(max(np.abs(t).max() for t in luts), G * d // 4)
                ints = np.zeros(n, np.int64)
                for t in range(n):
                    ints[t] = sum(int(np.rint(luts[j][g, pat[t, g]] * 2.0 ** s))
                                  for j in range(G) for g in range(d // 4))
                assert np.all(np.abs(ints - direct * 2.0 ** s) <= 0.5 * G * d // 4 + 1e-6)
                ranked = sorted(range(n), key=lambda t: (-ints[t], t))[:min(k, n)]
                assert cnt[b, h] == min(k, n)
                assert sel[b, h, :cnt[b, h]].tolist() == sorted(ranked)
                assert np.all(sel[b, h, cnt[b, h]:] == -1)
                assert scs[b, h, :cnt[b, h]].tolist() == [int(ints[t]) for t in sorted(ranked)]


def test_lut_scale_exponent_bounds():
    for maxabs, n in [(1.0, 32), (0.37, 64), (1e-9, 256), (123456.0, 8), (0.5, 1), (2.0 ** -3, 64)]:
        s = O.lut_scale_exponent(maxabs, n)
        assert n * maxabs * 2.0 ** s <= 2 ** 30 < n * maxabs * 2.0 ** (s + 1)
    assert O.lut_scale_exponent(0.0, 32) == 0


def test_quantize_from_rotated_packs_given_fields():
    codec = O.Codec(64, 3, 64, 4, 1, 2)
    rng = np.random.default_rng(9)
    k, v = rng.standard_normal((6, 64)), rng.standard_normal((6, 64))
    f = O.compress(codec, k, v)
    r = np.linalg.norm(k, axis=1)
    x = k @ codec.Pi64.T
    z = (x * (8.0 / r)[:, None]).astype(np.float32)
    xh = (f["r_k"].astype(np.float64) / 8.0)[:, None] * codec.key_levels.astype(np.float64)[f["kc"]]
    p = ((x - xh) @ codec.S64.T).astype(np.float32)
    rv = np.linalg.norm(v, axis=1)
    zv = ((v @ codec.Pi64.T) * (8.0 / rv)[:, None]).astype(np.float32)
    rec = O.quantize_from_rotated(codec, z, p, f["r_k"], f["rho"], zv, f["r_v"])
    assert np.array_equal(rec, O.pack_records(codec, f))


# ---------------------------------------------------------------- vector search ------
def test_recall_1_at_k_hand_example():
    """Three queries over four vectors.  Query 0: exact best 2, approximate order 2 first
    -> found at k = 1.  Query 1: exact best 0, approximate scores rank it third -> found
    from k = 3.  Query 2: exact best 3 tied in the approximate scores with index 1, which
    wins the tie -> rank 1, found from k = 2."""
    exact = np.array([[0.1, 0.2, 0.9, 0.3], [0.8, 0.1, 0.2, 0.3], [0.0, 0.5, 0.2, 0.7]])
    approx = np.array([[0.0, 0.1, 0.5, 0.2], [0.3, 0.1, 0.5, 0.4], [0.1, 0.6, 0.2, 0.6]])
    r = O.recall_1_at_k(approx, exact, [1, 2, 3, 4])
    assert r == {1: 1 / 3, 2: 2 / 3, 3: 1.0, 4: 1.0}


def test_recall_equals_sort_based_definition_and_exact_scores_give_one():
    rng = np.random.default_rng(4)
    exact = rng.standard_normal((50, 300))
    approx = exact + 0.3 * rng.standard_normal((50, 300))
    ks = [1, 2, 5, 10, 50]
    got = O.recall_1_at_k(approx, exact, ks)
    order = np.argsort(-approx, axis=1, kind="stable")      # ties: lower index first
    best = np.argmax(exact, axis=1)
    for k in ks:
        want = np.mean([best[i] in order[i, :k] for i in range(50)])
        assert got[k] == pytest.approx(want, abs=0)
    assert O.recall_1_at_k(exact, exact, [1])[1] == 1.0
    assert all(got[a] <= got[b] for a, b in zip(ks, ks[1:]))


@pytest.mark.parametrize("kb,vb,m", [(3, 2, 192), (2, 4, 0), (4, 3, 32)])
def test_head_dim_200_layout(kb, vb, m):
    """head_dim 200: code fields padded to whole words; a 3-bit field is 6 groups of 32
    codes (72 bytes) plus the last 8 codes as a plain 24-bit stream; pack/unpack round trip."""
    codec = O.Codec(200, kb, m, vb, 3, 4)
    assert codec.kbytes == (200 * kb // 8 + 3) // 4 * 4 and codec.kbytes % 4 == 0
    rng = np.random.default_rng(kb)
    f = dict(kc=rng.integers(0, 1 << kb, (5, 200)), bits=rng.integers(0, 2, (5, m)),
             vc=rng.integers(0, 1 << vb, (5, 200)), r_k=np.float32(rng.random(5)),
             rho=np.float32(rng.random(5)), r_v=np.float32(rng.random(5)))
    rec = O.pack_records(codec, f)
    assert rec.shape == (5, codec.record_bytes) and codec.record_bytes % 16 == 0
    g = O.unpack_records(codec, rec)
    for key in ("kc", "bits", "vc", "r_k", "rho", "r_v"):
        assert np.array_equal(g[key], f[key]), key
    if kb == 3:
        # tail: code 192 + i at bits 3 i of the little-endian 24-bit value after byte 72
        tail = rec[:, 72].astype(np.int64) | rec[:, 73].astype(np.int64) << 8 | rec[:, 74].astype(np.int64) << 16
        for i in range(8):
            assert np.array_equal((tail >> (3 * i)) & 7, f["kc"][:, 192 + i])
        assert np.all(rec[:, 75] == 0)


def test_head_dim_200_compress_decodes_exactly_without_quantization_error_terms():
    """With 4-bit codes and QJL (m = 224) at d = 200: the estimator equals
    <q_x, xhat> + coef rho <q_s, signs> recomputed from first principles, and the
    reconstruction error |x - xhat|^2 / |x|^2 sits near the 4-bit Lloyd-Max MSE / 1
    (0.0095 per coordinate)."""
    d = 200
    codec = O.Codec(d, 4, 224, 4, 5, 6)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((300, d))
    f = O.compress(codec, k, k)
    x = k @ codec.Pi64.T
    xhat = (f["r_k"].astype(np.float64) / math.sqrt(d))[:, None] * codec.key_levels.astype(np.float64)[f["kc"]]
    rel = np.mean(np.sum((x - xhat) ** 2, 1) / np.sum(x * x, 1))
    lm, lb = O.lloyd_max(4)
    assert abs(rel - O.quantizer_mse(lm, lb)) < 0.002
    q = rng.standard_normal(d)
    qx, qs = O.prepare_query(codec, q)
    s = O.score_estimates(codec, qx, qs, f)
    ref = xhat @ qx + math.sqrt(math.pi / 2) / 224 * f["rho"].astype(np.float64) * ((2.0 * f["bits"] - 1) @ qs)
    assert np.allclose(s, ref, rtol=1e-12, atol=1e-12)
