"""Pins of the PolarQuant-variant oracle (TurboQuant page, "PolarQuant: Ein neuer Winkel auf
Kompression") against facts fixed outside it: the page's worked example, closed-form
Lloyd-Max levels, the exact law of the angles of a random direction, an explicit
hyperspherical-coordinate formula, a hand-packed record, QJL unbiasedness and brute-force
attention on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import polar as P
from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pages_worked_example_radius_and_angle():
    with open(os.path.join(GOLDEN, "polar_example.json")) as f:
        g = json.load(f)
    R, ang = P.polar_transform(np.array(g["pair"]))
    assert R == pytest.approx(g["radius"], abs=1e-12)
    assert len(ang) == 1 and round(math.degrees(float(ang[0][0]))) == g["angle_degrees_rounded"]


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_transform_inverts_exactly_and_keeps_the_norm(d):
    y = np.random.default_rng(d).standard_normal((50, d))
    R, ang = P.polar_transform(y)
    assert [a.shape[-1] for a in ang] == [d >> l for l in range(1, P.n_levels(d) + 1)]
    assert np.allclose(R, np.linalg.norm(y, axis=1), rtol=1e-14)
    assert np.allclose(P.polar_inverse(R, ang), y, rtol=1e-12, atol=1e-13)
    assert np.all((ang[0] > -math.pi) & (ang[0] <= math.pi))
    for a in ang[1:]:
        assert np.all((a >= 0) & (a <= math.pi / 2))


def test_inverse_equals_explicit_hyperspherical_products():
    """Coordinate j of the unit vector is the product over levels l of cos or sin of the
    angle of node j >> l, sin when bit l-1 of j is set - an index formula, not a recursion."""
    d = 64
    L = P.n_levels(d)
    rng = np.random.default_rng(5)
    ang = [rng.uniform(-math.pi, math.pi, d // 2)] + \
          [rng.uniform(0, math.pi / 2, d >> l) for l in range(2, L + 1)]
    u = P.polar_inverse(np.float64(1.0), ang)
    ref = np.ones(d)
    for j in range(d):
        for l in range(1, L + 1):
            a = ang[l - 1][j >> l]
            ref[j] *= math.sin(a) if (j >> (l - 1)) & 1 else math.cos(a)
    assert np.allclose(u, ref, rtol=1e-14, atol=1e-15)
    assert abs(np.linalg.norm(u) - 1.0) < 1e-14


def test_zero_pairs_have_angle_zero():
    R, ang = P.polar_transform(np.array([0.0, -0.0, -0.0, 0.0, 3.0, 0.0, 0.0, 0.0]))
    assert R == 3.0
    assert list(ang[0]) == [0.0, 0.0, 0.0, 0.0]
    assert list(ang[1]) == [0.0, 0.0] and ang[2][0] == pytest.approx(math.pi / 2)


def test_level1_grid_is_uniform_on_the_circle():
    for b in (2, 4):
        lv, bd = P.level1_grid(b)
        w = 2 * math.pi / (1 << b)
        assert np.allclose(np.diff(lv), w) and np.allclose(np.diff(bd), w)
        assert lv[0] == pytest.approx(-math.pi + w / 2) and bd[0] == pytest.approx(-math.pi + w)
    # level-1 angles of rotated Gaussian vectors fill the 16 cells evenly
    y = np.random.default_rng(1).standard_normal((20000, 64))
    _, ang = P.polar_transform(y)
    _, bd = P.level1_grid(4)
    cnt = np.bincount(np.sum(ang[0].ravel()[:, None] >= bd, axis=1), minlength=16)
    assert stats.chisquare(cnt).pvalue > 1e-4


def test_one_bit_upper_grids_have_closed_forms():
    """Density sin(2 psi) (level 2): E[psi | psi < pi/4] = (1/4) / (1/2) = 1/2.
    Density sin^3(2 psi) (level 3): (7/36) / (1/3) = 7/12 (integration by parts)."""
    lv2, bd2 = P.upper_grid(2, 1)
    lv3, bd3 = P.upper_grid(3, 1)
    assert np.allclose(lv2, [0.5, math.pi / 2 - 0.5], atol=1e-12)
    assert np.allclose(lv3, [7 / 12, math.pi / 2 - 7 / 12], atol=1e-12)
    assert bd2[0] == pytest.approx(math.pi / 4, abs=1e-15) and bd3[0] == pytest.approx(math.pi / 4, abs=1e-15)


@pytest.mark.parametrize("bits", [2, 4])
def test_upper_grids_match_the_empirical_law_of_the_angles(bits):
    """For Gaussian vectors (a uniformly random direction) the level-l angles obey
    sin^2 psi ~ Beta(n/2, n/2), n = 2^(l-1) (Kolmogorov-Smirnov); each Lloyd-Max cell holds
    the mass the law gives it, and the level is the mean of the angles falling in it."""
    d, N = 128, 40000
    y = np.random.default_rng(bits).standard_normal((N, d))
    _, ang = P.polar_transform(y)
    for l in range(2, P.n_levels(d) + 1):
        n = 1 << (l - 1)
        a = ang[l - 1].ravel()
        assert stats.kstest(np.sin(a) ** 2, stats.beta(n / 2, n / 2).cdf).pvalue > 1e-4, l
        lv, bd = P.upper_grid(l, bits)
        cell = np.sum(a[:, None] >= bd, axis=1)
        cdf = stats.beta(n / 2, n / 2).cdf(np.sin(np.concatenate([[0.0], bd, [math.pi / 2]])) ** 2)
        mass = np.diff(cdf)
        for c in range(1 << bits):
            sel = a[cell == c]
            frac = sel.size / a.size
            assert abs(frac - mass[c]) <= 5 * math.sqrt(mass[c] * (1 - mass[c]) / a.size) + 1e-9, (l, c)
            assert abs(sel.mean() - lv[c]) <= 5 * sel.std() / math.sqrt(sel.size) + 1e-9, (l, c)


def test_upper_grid_levels_are_cell_centroids_by_an_independent_rule():
    """Centroid condition rechecked with a composite Simpson rule on a fine grid."""
    for l in (2, 5, 7):
        n = 1 << (l - 1)
        lv, bd = P.upper_grid(l, 2)
        edges = np.concatenate([[0.0], bd, [math.pi / 2]])
        for c in range(4):
            t = np.linspace(edges[c], edges[c + 1], 200001)
            w = np.sin(2 * t) ** (n - 1)
            h = t[1] - t[0]
            simpson = lambda v: h / 3 * (v[0] + v[-1] + 4 * v[1:-1:2].sum() + 2 * v[2:-1:2].sum())
            assert abs(simpson(t * w) / simpson(w) - lv[c]) < 1e-10


def test_record_layout_hand_packed():
    """d = 8, b1 = 4, bh = 2: level-1 codes [1, 2, 3, 4] -> bytes 0x21 0x43; upper codes
    (level 2: [1, 2], level 3: [3]) -> 1 | 2 << 2 | 3 << 4 = 0x39, padded to 4 bytes."""
    codec = P.PolarCodec(8, 4, 0, 2, 1, 2, upper_bits=2)
    assert codec.kbytes == 2 + 4
    f = dict(kc=[np.array([[1, 2, 3, 4]]), np.array([[1, 2]]), np.array([[3]])],
             bits=np.zeros((1, 0), np.int64), vc=np.zeros((1, 8), np.int64),
             r_k=np.float32([1.5]), rho=np.float32([0.25]), r_v=np.float32([2.0]))
    rec = codec.pack(f)
    assert list(rec[0, :6]) == [0x21, 0x43, 0x39, 0, 0, 0]
    assert rec.shape[-1] == codec.record_bytes == 32
    back = codec.unpack(rec)
    for a, b in zip(back["kc"], f["kc"]):
        assert np.array_equal(a, b)
    assert back["r_k"][0] == 1.5 and back["rho"][0] == 0.25 and back["r_v"][0] == 2.0


def test_zero_key_codes():
    codec = P.PolarCodec(16, 4, 32, 2, 3, 4, upper_bits=2)
    f = codec.compress_fields(np.zeros((1, 16)), np.ones((1, 16)))
    assert np.all(f["kc"][0] == 8) and all(np.all(c == 0) for c in f["kc"][1:])
    assert f["r_k"][0] == 0 and f["rho"][0] == 0 and np.all(f["bits"] == 1)


def test_distortion_falls_with_angle_bits():
    """E|y - r u|^2 / r^2 over random keys decreases as the grids get finer."""
    k = np.random.default_rng(0).standard_normal((400, 64))
    errs = []
    for b1, bh in [(2, 1), (2, 2), (4, 2), (4, 4)]:
        codec = P.PolarCodec(64, b1, 0, 2, 7, 8, upper_bits=bh)
        f = codec.compress_fields(k, k)
        y = k @ codec.Pi64.T
        yh = f["r_k"].astype(np.float64)[:, None] * codec.unit_vector(f["kc"])
        errs.append(np.mean(np.sum((y - yh) ** 2, axis=1) / np.sum(y * y, axis=1)))
    assert all(a > b for a, b in zip(errs, errs[1:])), errs
    assert errs[2] < 0.05


def test_polar_estimator_is_unbiased():
    """The QJL term corrects the polar stage-1 estimate: over 4000 independent sketches
    the mean of s_hat - <q, k> lies within 3 standard errors of 0, while the stage-1
    estimate alone r <q_x, u> has a fixed bias."""
    d = m = 64
    codec = P.PolarCodec(d, 4, m, 2, 31, 32, upper_bits=2)
    rng = np.random.default_rng(9)
    k, q = rng.standard_normal(d), rng.standard_normal(d)
    exact = float(q @ k)
    errs = []
    for _ in range(4000):
        codec.S = rng.standard_normal((m, d)).astype(np.float32)
        codec.S64 = codec.S.astype(np.float64)
        f = codec.compress_fields(k[None], k[None])
        qx, qs = O.prepare_query(codec, q)
        errs.append(O.score_estimates(codec, qx, qs, f)[0] - exact)
    errs = np.array(errs)
    se = errs.std(ddof=1) / math.sqrt(len(errs))
    assert abs(errs.mean()) <= 3 * se, (errs.mean(), se)
    stage1 = codec.key_part(codec.Pi64 @ q, f)[0] - exact
    assert abs(stage1) > 5 * se


@pytest.mark.parametrize("d,T,H", [(8, 5, 2), (16, 3, 4)])
def test_polar_decode_equals_brute_force_attention(d, T, H):
    """Tiny inputs: effective keys Pi^T [r u + (sqrt(pi/2) rho / m) S^T (2 bit - 1)], u built
    from the explicit hyperspherical products of the stored codes' grid angles."""
    rng = np.random.default_rng(d + T)
    codec = P.PolarCodec(d, 4, 2 * d, 2, 41, 42, upper_bits=2)
    B, Hkv = 2, 1
    K = rng.standard_normal((B, T, Hkv, d))
    V = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, H, d))
    rec = O.compress_cache(codec, K, V)
    out, lse, _ = O.decode_attention(codec, q, rec, [T, T - 1])
    L = P.n_levels(d)
    for b in range(B):
        n = [T, T - 1][b]
        f = codec.unpack(rec[b, 0, :n])
        u = np.ones((n, d))
        for j in range(d):
            for l in range(1, L + 1):
                a = codec.angle_levels[l - 1].astype(np.float64)[f["kc"][l - 1][:, j >> l]]
                u[:, j] *= np.sin(a) if (j >> (l - 1)) & 1 else np.cos(a)
        xk = f["r_k"].astype(np.float64)[:, None] * u
        xk += (math.sqrt(math.pi / 2) * f["rho"].astype(np.float64) / codec.qjl_dim)[:, None] * \
            ((2.0 * f["bits"] - 1.0) @ codec.S64)
        keff = xk @ codec.Pi64
        xv = (f["r_v"].astype(np.float64) / math.sqrt(d))[:, None] * codec.val_levels.astype(np.float64)[f["vc"]]
        veff = xv @ codec.Pi64
        for h in range(H):
            lg = keff @ q[b, h] / math.sqrt(d)
            p = np.exp(lg - lg.max())
            assert np.allclose(out[b, h], p @ veff / p.sum(), rtol=1e-12, atol=1e-13)
            assert abs(lse[b, h] - (lg.max() + math.log(p.sum()))) < 1e-12
