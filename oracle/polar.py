"""Oracle of the PolarQuant variant of stage 1 (keys): recursive polar codes.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it, and
it shares no code, table or constant generator with the HIP path.

TurboQuant page (de.news.hada.io/topic?id=27867), section "PolarQuant: Ein neuer Winkel
auf Kompression": a vector becomes a radius and angles instead of Cartesian coordinates;
the coordinates of a d-dimensional vector are taken in pairs and turned into polar
coordinates, then the radii are paired and transformed again, recursively, until one
radius and a set of angles remain; the angles follow a known, concentrated pattern, so
they are mapped onto a fixed circular grid whose bounds are known in advance (no
per-block normalisation).  The page's first step (random rotation) and second step
(1-bit QJL on what stage 1 leaves) are unchanged; comments on the same page say the
polar codebook survives in TurboQuant.

Readings taken where the page leaves a step open:

* P1  The polar transform acts on the rotated key y = Pi k, coordinates paired as
      (y_2i, y_2i+1).  Level 1: radius sqrt(a^2 + b^2), angle atan2(b, a) in (-pi, pi].
      Level l >= 2 pairs the level-(l-1) radii (left, right) the same way: radius
      sqrt(left^2 + right^2), angle atan2(right, left) in [0, pi/2].  d = 2^L gives L
      levels with d/2^l angles at level l (d - 1 angles) and one final radius = |y|.
      A pair of two zeros has angle 0 (atan2 of two zeros is otherwise sign-dependent).
* P2  Level-1 angles are uniform on the circle for a rotated vector, so their grid is
      uniform: 2^b1 cells of width 2 pi / 2^b1 from -pi, reconstruction at cell centres
      (the Lloyd-Max quantizer of a uniform density).
* P3  Above level 1 the "known pattern" is the exact law of the angle of a uniformly
      random direction: with n = 2^(l-1) coordinates under each child radius,
      sin^2(psi) ~ Beta(n/2, n/2), density proportional to sin^(n-1)(2 psi) on [0, pi/2],
      concentrated at pi/4.  The fixed grid of level l is the Lloyd-Max quantizer of that
      density with 2^bh cells (boundaries at midpoints, levels at conditional means),
      float64, rounded to float32.
* P4  Bits: b1 per level-1 angle, bh per higher angle (the page gives no allocation;
      the default 4 / 2 makes a 128-dim key field 48 bytes, the size of 3-bit scalar
      codes).
* P5  The radius kept is r = |k| (float32), as in the scalar codec; the key is
      reconstructed as r * u, u the unit vector of the quantized angles.
* P6  QJL sketches the residual e = y - r u exactly as in the scalar codec; the
      estimator's first term becomes r <q_x, u>.
* P7  Values keep the scalar codec (the polar variant is taken for the keys).
* P8  Integer decisions: code = #{j : angle >= bound_j}, the angle in float64 and the
      bounds the float32 grid (the GPU computes the same float64 angles).

Record key field: the level-1 codes as a b1-bit little-endian bitstream, then the codes of
levels 2..L (level 2 first, node order within a level) as a bh-bit bitstream padded to a
multiple of 4 bytes.
"""
from __future__ import annotations

import functools
import math

import numpy as np
from scipy import integrate
from scipy.special import betaincinv

from . import tq_oracle as O

PI = math.pi


def n_levels(d: int) -> int:
    L = int(round(math.log2(d)))
    assert 1 << L == d, "head_dim must be a power of two"
    return L


# ----------------------------------------------------------------------------------------
# The recursive polar transform and its inverse (readings P1)
# ----------------------------------------------------------------------------------------
def _angle(a, b):
    """atan2(b, a), 0 where a = b = 0."""
    both0 = (a == 0) & (b == 0)
    return np.where(both0, 0.0, np.arctan2(b, a))


def polar_transform(y: np.ndarray):
    """y [..., d] -> (final radius [...], [angles of level 1, level 2, ...]); float64."""
    r = np.asarray(y, np.float64)
    angles = []
    while r.shape[-1] > 1:
        a, b = r[..., 0::2], r[..., 1::2]
        angles.append(_angle(a, b))
        r = np.sqrt(a * a + b * b)
    return r[..., 0], angles


def polar_inverse(radius: np.ndarray, angles: list) -> np.ndarray:
    """Top-down inverse: each node's radius splits into (r cos, r sin) of its angle."""
    r = np.asarray(radius, np.float64)[..., None]
    for ang in reversed(angles):
        out = np.empty(r.shape[:-1] + (2 * r.shape[-1],))
        out[..., 0::2] = r * np.cos(ang)
        out[..., 1::2] = r * np.sin(ang)
        r = out
    return r


# ----------------------------------------------------------------------------------------
# Angle grids (readings P2, P3)
# ----------------------------------------------------------------------------------------
def level1_grid(bits: int):
    """Uniform grid on (-pi, pi]: levels -pi + (c + 1/2) w, bounds -pi + j w, w = 2 pi / 2^bits."""
    L = 1 << bits
    w = 2.0 * PI / L
    return -PI + (np.arange(L) + 0.5) * w, -PI + np.arange(1, L) * w


def angle_density(n: int):
    """Unnormalised density of a level-l angle, n = 2^(l-1): sin(2 psi)^(n-1) on [0, pi/2]."""
    return lambda psi: math.sin(2.0 * psi) ** (n - 1)


@functools.lru_cache(maxsize=None)
def upper_grid(level: int, bits: int, tol: float = 1e-13, max_iter: int = 5000):
    """Lloyd-Max quantizer (levels, bounds) of the level-`level` angle law on [0, pi/2].

    Cell mass and first moment by adaptive quadrature (scipy.integrate.quad); start at the
    quantiles (i + 1/2) / 2^bits of the law (sin^2 psi ~ Beta(n/2, n/2)); the law is
    symmetric about pi/4, so the levels are kept exactly mirror-symmetric."""
    n = 1 << (level - 1)
    f = angle_density(n)
    L = 1 << bits
    q = (np.arange(L) + 0.5) / L
    lev = np.arcsin(np.sqrt(betaincinv(n / 2.0, n / 2.0, q)))
    lev = 0.5 * (lev + (PI / 2 - lev[::-1]))
    for _ in range(max_iter):
        edges = np.concatenate([[0.0], 0.5 * (lev[:-1] + lev[1:]), [PI / 2]])
        new = np.empty(L)
        for i in range(L):
            lo, hi = edges[i], edges[i + 1]
            mass = integrate.quad(f, lo, hi, epsabs=0.0, epsrel=1e-13, limit=200)[0]
            mom = integrate.quad(lambda t: t * f(t), lo, hi, epsabs=0.0, epsrel=1e-13, limit=200)[0]
            new[i] = mom / mass
        new = 0.5 * (new + (PI / 2 - new[::-1]))
        delta = float(np.max(np.abs(new - lev)))
        lev = new
        if delta < tol:
            break
    return lev, 0.5 * (lev[:-1] + lev[1:])


# ----------------------------------------------------------------------------------------
# The codec
# ----------------------------------------------------------------------------------------
class PolarCodec(O.Codec):
    """Scalar codec with the key stage 1 replaced by polar codes (key_bits = b1 bits per
    level-1 angle, upper_bits = bh bits per higher angle)."""

    def __init__(self, head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed,
                 upper_bits):
        self.upper_bits = upper_bits
        super().__init__(head_dim, key_bits, qjl_dim, value_bits, rotation_seed, qjl_seed)

    def __post_init__(self):
        d = self.head_dim
        self.L = n_levels(d)
        self.Pi = O.rotation(self.rotation_seed, d)
        self.S = O.qjl_matrix(self.qjl_seed, self.qjl_dim, d)
        gv, tv = O.lloyd_max(self.value_bits)
        self.val_levels, self.val_bounds = gv.astype(np.float32), tv.astype(np.float32)
        self.Pi64 = self.Pi.astype(np.float64)
        self.S64 = self.S.astype(np.float64)
        grids = [level1_grid(self.key_bits)]
        grids += [upper_grid(l, self.upper_bits) for l in range(2, self.L + 1)]
        self.angle_levels = [g[0].astype(np.float32) for g in grids]
        self.angle_bounds = [g[1].astype(np.float32) for g in grids]

    @property
    def l1_bytes(self):
        return self.head_dim // 2 * self.key_bits // 8

    @property
    def upper_bytes(self):
        return 4 * (((self.head_dim // 2 - 1) * self.upper_bits + 31) // 32)

    @property
    def kbytes(self):
        return self.l1_bytes + self.upper_bytes

    # ---- stage 1 + QJL --------------------------------------------------------------
    def unit_vector(self, codes: list) -> np.ndarray:
        """u from per-level codes: the quantized angles (float32 grid values, evaluated in
        float64) through the inverse transform with radius 1."""
        ang = [self.angle_levels[l].astype(np.float64)[c] for l, c in enumerate(codes)]
        return polar_inverse(np.ones(codes[0].shape[:-1]), ang)

    def compress_fields(self, k, v):
        """Keys: r = |k|, y = Pi k, per-level angles and codes (P1-P3, P8), residual
        e = y - r32 u, rho = |e|, QJL bits [(S e)_j >= 0] (float32).  Values: scalar codes."""
        kk = np.asarray(k, np.float64)
        r = np.sqrt(np.sum(kk * kk, axis=-1))
        r32 = r.astype(np.float32)
        y = kk @ self.Pi64.T
        _, angles = polar_transform(y)
        codes = [np.sum(a[..., None] >= self.angle_bounds[l].astype(np.float64), axis=-1)
                 for l, a in enumerate(angles)]
        u = self.unit_vector(codes)
        e = y - r32.astype(np.float64)[..., None] * u
        rho = np.sqrt(np.sum(e * e, axis=-1)).astype(np.float32)
        if self.qjl_dim:
            bits = ((e @ self.S64.T).astype(np.float32) >= 0).astype(np.int64)
        else:
            bits = np.zeros(kk.shape[:-1] + (0,), dtype=np.int64)
        r_v, _, _, cv = O._rotate_and_code(self, v, self.val_bounds)
        return dict(kc=codes, bits=bits, vc=cv, r_k=r32, rho=rho, r_v=r_v)

    # ---- record ---------------------------------------------------------------------
    def pack(self, f):
        codes = f["kc"]
        up = np.concatenate(codes[1:], axis=-1)
        upb = O._pack_stream(up, self.upper_bits)
        upb = np.concatenate([upb, np.zeros(upb.shape[:-1] + (self.upper_bytes - upb.shape[-1],),
                                             np.uint8)], axis=-1)
        parts = [
            O._pack_stream(codes[0], self.key_bits),
            upb,
            O._pack_stream(f["bits"], 1),
            O._pad_to(O._pack_stream(f["vc"], self.value_bits), self.vbytes),
            np.stack([f["r_k"], f["rho"], f["r_v"]], axis=-1).astype("<f4").view(np.uint8),
        ]
        rec = np.concatenate(parts, axis=-1)
        pad = self.record_bytes - rec.shape[-1]
        return np.concatenate([rec, np.zeros(rec.shape[:-1] + (pad,), np.uint8)], axis=-1)

    def unpack(self, rec):
        d, m = self.head_dim, self.qjl_dim
        o1 = self.l1_bytes
        o2 = self.kbytes
        o3 = o2 + self.sbytes
        o4 = o3 + self.vbytes
        c1 = O._unpack_stream(rec[..., :o1], d // 2, self.key_bits)
        up = O._unpack_stream(rec[..., o1:o2], d // 2 - 1, self.upper_bits)
        codes, off = [c1], 0
        for l in range(2, self.L + 1):
            cnt = d >> l
            codes.append(up[..., off:off + cnt])
            off += cnt
        norms = np.ascontiguousarray(rec[..., o4:o4 + 12]).view("<f4")
        return dict(kc=codes, bits=O._unpack_stream(rec[..., o2:o3], m, 1),
                    vc=O._unpack_stream(rec[..., o3:o4], d, self.value_bits),
                    r_k=norms[..., 0], rho=norms[..., 1], r_v=norms[..., 2])

    def key_part(self, qx, f):
        """r_t <q_x, u_t> (reading P6)."""
        return f["r_k"].astype(np.float64) * (self.unit_vector(f["kc"]) @ qx)

    def key_vector(self, f):
        """The stage-1 reconstruction of the keys in the rotated basis, r_k u (reading P5),
        float64."""
        return f["r_k"].astype(np.float64)[..., None] * self.unit_vector(f["kc"])
