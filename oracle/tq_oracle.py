"""Oracle: a plain, slow, fp64 CPU implementation of the compressed-key attention path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path (the HIP
library and its Python binding) never imports, links or calls anything here, and this
module shares no code, table or constant generator with the HIP path.

Every function follows the pages step by step, in their order:

* TurboQuant page (de.news.hada.io/topic?id=27867), section "Funktionsweise von
  TurboQuant": 1. Schritt - rotate the vector at random, then apply a fixed, standard
  quantizer to each coordinate separately; 2. Schritt - spend one more bit on the
  residual with QJL.  Section "QJL: Eine 1-Bit-Methode ohne Overhead": a
  Johnson-Lindenstrauss projection whose outputs keep only their sign, read back with
  an estimator that pairs the full-precision query with the 1-bit data.  Hacker News
  comments on the same page: boundaries and reconstruction values from Lloyd-Max;
  each dimension coded on its own.
* TurboQuant explainer (chatgpz.de, "Die KV-Cache-Optimierung von Google erklaert"),
  "Stufe 1" (random rotation/preconditioning) and "Stufe 2" (1-bit QJL residual,
  an unbiased estimator).
* Self-Indexing KVCache page (gist.science 2603.14224), "Methodologie" items 1-4:
  4-dim sign patterns (0..15) with 16 centroids per group built in one pass,
  channel-mean subtraction before taking signs, LUT-GEMV top-k in the compressed
  domain, token-wise layout.
* Monarch v3 page, "Wie es funktioniert": recent tokens exact, older tokens compressed,
  both in one softmax.

Where the pages leave a step open the reading taken is stated at the function.
Arithmetic is float64 unless a
step says otherwise; decisions that turn a float into an integer (a code, a sign bit, a
sign-index bit) are taken in float32, the precision the GPU kernels take them in.

Pinned by tests/test_oracle_pins.py (closed forms, published Lloyd-Max/Max-1960 tables,
QJL unbiasedness, brute-force attention on tiny inputs, invariants).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.special import ndtr, ndtri

# ----------------------------------------------------------------------------------------
# Counter-based generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
# number generators", OOPSLA 2014).  Output i of stream `seed` is mix(seed + (i+1)*phi).
# ----------------------------------------------------------------------------------------
_M64 = (1 << 64) - 1
_PHI64 = 0x9E3779B97F4A7C15
TWO_PI = 6.283185307179586


def splitmix64(seed: int, n: int) -> list[int]:
    out = []
    for i in range(n):
        z = (seed + (i + 1) * _PHI64) & _M64
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


def gaussians(seed: int, n: int) -> np.ndarray:
    """n standard normals by the Box-Muller transform (Box & Muller 1958) of SplitMix64 words.

    Pair k uses words 2k and 2k+1: u1 = ((w >> 11) + 1) * 2^-53 in (0, 1],
    u2 = (w >> 11) * 2^-53 in [0, 1); g = sqrt(-2 ln u1) * (cos, sin)(2 pi u2).
    """
    pairs = (n + 1) // 2
    w = splitmix64(seed, 2 * pairs)
    g = []
    for k in range(pairs):
        u1 = ((w[2 * k] >> 11) + 1) * 2.0 ** -53
        u2 = (w[2 * k + 1] >> 11) * 2.0 ** -53
        rad = math.sqrt(-2.0 * math.log(u1))
        ang = TWO_PI * u2
        g.append(rad * math.cos(ang))
        g.append(rad * math.sin(ang))
    return np.array(g[:n], dtype=np.float64)


# ----------------------------------------------------------------------------------------
# Init: rotation, QJL matrix, Lloyd-Max codebooks
# ----------------------------------------------------------------------------------------
def rotation(seed: int, d: int) -> np.ndarray:
    """Random rotation Pi (float32, d x d) applied as x = Pi k.

    TurboQuant page, "Funktionsweise", 1. Schritt (random rotation).  Reading: Pi is the
    Q factor of a seeded d x d Gaussian G (row-major from `gaussians(seed, d*d)`),
    normalised so that R = Q^T G has a positive diagonal, then rounded to float32.
    """
    G = gaussians(seed, d * d).reshape(d, d)
    Q, R = np.linalg.qr(G)
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return (Q * s[None, :]).astype(np.float32)


def qjl_matrix(seed: int, m: int, d: int) -> np.ndarray:
    """QJL projection S (float32, m x d) with i.i.d. N(0, 1) entries, row-major from the
    stream of `seed`.  TurboQuant page, "QJL: Eine 1-Bit-Methode ohne Overhead"."""
    if m == 0:
        return np.zeros((0, d), dtype=np.float32)
    return gaussians(seed, m * d).reshape(m, d).astype(np.float32)


def _cell_mass_and_moment(lo: np.ndarray, hi: np.ndarray):
    """P(lo < X < hi) and E[X; lo < X < hi] for X ~ N(0, 1)."""
    return ndtr(hi) - ndtr(lo), _phi(lo) - _phi(hi)


def _phi(t):
    """Standard normal density, 0 at +-inf."""
    t = np.asarray(t, np.float64)
    fin = np.isfinite(t)
    tt = np.where(fin, t, 0.0)
    return np.where(fin, np.exp(-0.5 * tt * tt) / math.sqrt(2.0 * math.pi), 0.0)


def _tphi(t):
    """t * phi(t), 0 at +-inf."""
    t = np.asarray(t, np.float64)
    fin = np.isfinite(t)
    tt = np.where(fin, t, 0.0)
    return tt * _phi(tt) * fin


def lloyd_max(bits: int, tol: float = 1e-14, max_iter: int = 20000):
    """Lloyd-Max quantizer for N(0, 1) with 2^bits levels (float64 levels, boundaries).

    Hacker News comments on the TurboQuant page: boundaries and reconstruction values
    optimised with the Lloyd-Max algorithm.  Lloyd's two conditions are iterated:
    boundaries at the midpoints of adjacent levels; each level the conditional mean of
    its cell.  Start: the Gaussian quantiles at (i + 1/2) / L.  The density is symmetric,
    so after every step the levels are made exactly antisymmetric, gamma[L-1-i] = -gamma[i]
    (the middle boundary is then exactly 0).
    """
    L = 1 << bits
    lev = ndtri((np.arange(L) + 0.5) / L)
    lev = 0.5 * (lev - lev[::-1])
    for _ in range(max_iter):
        b = 0.5 * (lev[:-1] + lev[1:])
        edges = np.concatenate([[-np.inf], b, [np.inf]])
        mass, mom = _cell_mass_and_moment(edges[:-1], edges[1:])
        new = mom / mass
        new = 0.5 * (new - new[::-1])
        delta = np.max(np.abs(new - lev))
        lev = new
        if delta < tol:
            break
    return lev, 0.5 * (lev[:-1] + lev[1:])


def quantizer_mse(levels: np.ndarray, bounds: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0, 1), by the cell identity
    sum_k [ E[X^2; cell] - 2 g_k E[X; cell] + g_k^2 P(cell) ]."""
    edges = np.concatenate([[-np.inf], bounds, [np.inf]])
    lo, hi = edges[:-1], edges[1:]
    mass, mom = _cell_mass_and_moment(lo, hi)
    # E[X^2; lo<X<hi] = mass + lo*phi(lo) - hi*phi(hi)
    m2 = mass + _tphi(lo) - _tphi(hi)
    return float(np.sum(m2 - 2.0 * levels * mom + levels * levels * mass))


@dataclass
class Codec:
    """The constants one handle holds: Pi, S and the two float32 codebooks."""
    head_dim: int
    key_bits: int
    qjl_dim: int
    value_bits: int
    rotation_seed: int
    qjl_seed: int

    def __post_init__(self):
        d, m = self.head_dim, self.qjl_dim
        self.Pi = rotation(self.rotation_seed, d)
        self.S = qjl_matrix(self.qjl_seed, m, d)
        gk, tk = lloyd_max(self.key_bits)
        gv, tv = lloyd_max(self.value_bits)
        self.key_levels, self.key_bounds = gk.astype(np.float32), tk.astype(np.float32)
        self.val_levels, self.val_bounds = gv.astype(np.float32), tv.astype(np.float32)
        self.Pi64 = self.Pi.astype(np.float64)
        self.S64 = self.S.astype(np.float64)

    # record layout ---------------------------------------------------------------------
    @property
    def kbytes(self):
        """Key code field: d * b_k / 8 bytes, padded to a multiple of 4 (every field starts on
        a 32-bit word; no padding at head_dim 64 or 128)."""
        return (self.head_dim * self.key_bits // 8 + 3) // 4 * 4

    @property
    def sbytes(self):
        return self.qjl_dim // 8

    @property
    def vbytes(self):
        return (self.head_dim * self.value_bits // 8 + 3) // 4 * 4

    @property
    def record_bytes(self):
        payload = self.kbytes + self.sbytes + self.vbytes + 12
        return (payload + 15) // 16 * 16

    @property
    def index_bytes(self):
        return self.head_dim // 8

    # per-codec steps (the polar variant of stage 1 replaces these four) ----------------
    def compress_fields(self, k, v):
        return compress(self, k, v)

    def pack(self, f):
        return pack_records(self, f)

    def unpack(self, rec):
        return unpack_records(self, rec)

    def key_part(self, qx, f):
        """First term of the estimator: <q_x, xhat_t> with xhat_t = (r_t/sqrt(d)) gamma[c_t]."""
        gk = self.key_levels.astype(np.float64)
        return (f["r_k"].astype(np.float64) / math.sqrt(self.head_dim)) * (gk[f["kc"]] @ qx)

    def key_vector(self, f):
        """The stage-1 reconstruction of the keys in the rotated basis, xhat = (r_k/sqrt(d))
        gamma[c] (float64) - what a promoted cold key is rebuilt from."""
        gk = self.key_levels.astype(np.float64)
        return (f["r_k"].astype(np.float64) / math.sqrt(self.head_dim))[..., None] * gk[f["kc"]]


# ----------------------------------------------------------------------------------------
# Compression (TurboQuant page, "Funktionsweise" steps 1 and 2)
# ----------------------------------------------------------------------------------------
def quantize(z32: np.ndarray, bounds32: np.ndarray) -> np.ndarray:
    """Code of each float32 coordinate: the number of float32 boundaries it reaches,
    c = #{j : z >= tau_j} (a value exactly on a boundary goes to the upper cell)."""
    return np.sum(z32[..., None] >= bounds32, axis=-1).astype(np.int64)


def _rotate_and_code(codec: Codec, x_in: np.ndarray, bounds32: np.ndarray):
    """Step 1 for vectors [..., d]: r = |k|, x = Pi k, z = x * (sqrt(d) / r) rounded to
    float32, codes from the fixed N(0,1) codebook.  r = 0 gives z = 0 (all codes at the
    middle cell) - a reading, the pages do not treat the zero vector."""
    d = codec.head_dim
    k = x_in.astype(np.float64)
    r = np.sqrt(np.sum(k * k, axis=-1))
    x = k @ codec.Pi64.T
    scale = np.zeros_like(r)
    nz = r > 0
    scale[nz] = math.sqrt(d) / r[nz]
    z32 = (x * scale[..., None]).astype(np.float32)
    return r.astype(np.float32), x, z32, quantize(z32, bounds32)


def compress(codec: Codec, k: np.ndarray, v: np.ndarray):
    """Compress keys and values [..., d] into their record fields.

    Keys: codes c (key_bits each), residual e = x - (r/sqrt(d)) gamma[c] in the rotated
    space (reading: the pages do not say in which basis QJL sees the residual; S Pi^T is
    again an i.i.d. Gaussian matrix, so the rotated basis is statistically the same),
    rho = |e|, QJL signs bit_j = [ (S e)_j >= 0 ] (a float32 comparison, so -0 gives 1).
    Values: codes only (reading: QJL exists to make attention scores precise).
    Returns a dict of arrays; norms are float32 as stored.
    """
    d = codec.head_dim
    r_k, x, _, ck = _rotate_and_code(codec, k, codec.key_bounds)
    xhat = (r_k.astype(np.float64) / math.sqrt(d))[..., None] * codec.key_levels.astype(np.float64)[ck]
    e = x - xhat
    rho = np.sqrt(np.sum(e * e, axis=-1)).astype(np.float32)
    if codec.qjl_dim:
        p32 = (e @ codec.S64.T).astype(np.float32)
        bits = (p32 >= 0).astype(np.int64)
    else:
        bits = np.zeros(k.shape[:-1] + (0,), dtype=np.int64)
    r_v, _, _, cv = _rotate_and_code(codec, v, codec.val_bounds)
    return dict(kc=ck, bits=bits, vc=cv, r_k=r_k, rho=rho, r_v=r_v)


def _pack_stream(codes: np.ndarray, b: int) -> np.ndarray:
    """Pack a field of b-bit codes (last axis) into bytes.

    b = 1, 2, 4: little-endian bitstream - code i occupies stream bits [b*i, b*i + b), stream
    bit n being bit n % 8 of byte n // 8.
    b = 3: groups of 32 codes, each 12 bytes read as little-endian 32-bit words W0, W1, W2.
    Code j < 24 occupies bits [8*(j % 4) + 3*((j % 8) // 4), +3) of W_(j // 8).  Code
    24 + r (r = 0..7) occupies the 6-bit value T_k of byte lane k = r % 4 (bits [3*(r // 4), +3)),
    where bit t of T_k is bit 8k + 6 + (t % 2) of W_(t // 2).  (Four codes of one selector
    byte-lane pattern then come out of a word with one shift and one mask.)  A trailing
    partial group (head_dim 200: codes 192..199) is a plain bitstream as for the other widths,
    starting right after the last whole group.
    """
    if codes.shape[-1] == 0:
        return np.zeros(codes.shape[:-1] + (0,), dtype=np.uint8)
    if b == 3:
        return _pack_groups3(codes)
    return _pack_plain(codes, b)


def _group3_bit_positions() -> np.ndarray:
    """pos[j, t] = bit index within the 96-bit group (32 * word + bit) of bit t of code j."""
    pos = np.zeros((32, 3), dtype=np.int64)
    for j in range(32):
        for t in range(3):
            if j < 24:
                word, bit = j // 8, 8 * (j % 4) + 3 * ((j % 8) // 4) + t
            else:
                r = j - 24
                k, tt = r % 4, 3 * (r // 4) + t          # bit tt of T_k
                word, bit = tt // 2, 8 * k + 6 + tt % 2
            pos[j, t] = 32 * word + bit
    return pos


def _pack_plain(codes: np.ndarray, b: int) -> np.ndarray:
    bitarr = ((codes[..., :, None] >> np.arange(b)) & 1).astype(np.uint8)
    bitarr = bitarr.reshape(codes.shape[:-1] + (codes.shape[-1] * b,))
    return np.packbits(bitarr, axis=-1, bitorder="little")


def _unpack_plain(buf: np.ndarray, n: int, b: int) -> np.ndarray:
    bitarr = np.unpackbits(buf, axis=-1, bitorder="little")[..., : n * b]
    bitarr = bitarr.reshape(buf.shape[:-1] + (n, b)).astype(np.int64)
    return np.sum(bitarr << np.arange(b), axis=-1)


def _pack_groups3(codes: np.ndarray) -> np.ndarray:
    n = codes.shape[-1]
    ng = n // 32
    pos = _group3_bit_positions()
    g = codes[..., : 32 * ng].reshape(codes.shape[:-1] + (ng, 32))
    bits = np.zeros(g.shape[:-1] + (96,), dtype=np.uint8)
    for j in range(32):
        for t in range(3):
            bits[..., pos[j, t]] = (g[..., j] >> t) & 1
    out = np.packbits(bits, axis=-1, bitorder="little")      # word w bit i = stream bit 32w + i
    out = out.reshape(codes.shape[:-1] + (ng * 12,))
    if n % 32:
        out = np.concatenate([out, _pack_plain(codes[..., 32 * ng:], 3)], axis=-1)
    return out


def _unpack_stream(buf: np.ndarray, n: int, b: int) -> np.ndarray:
    if n == 0:
        return np.zeros(buf.shape[:-1] + (0,), dtype=np.int64)
    if b == 3:
        ng = n // 32
        pos = _group3_bit_positions()
        bits = np.unpackbits(buf[..., : ng * 12], axis=-1, bitorder="little")
        bits = bits.reshape(buf.shape[:-1] + (ng, 96)).astype(np.int64)
        codes = np.zeros(buf.shape[:-1] + (ng, 32), dtype=np.int64)
        for j in range(32):
            for t in range(3):
                codes[..., j] |= bits[..., pos[j, t]] << t
        codes = codes.reshape(buf.shape[:-1] + (32 * ng,))
        if n % 32:
            tail = _unpack_plain(buf[..., ng * 12:], n - 32 * ng, 3)
            codes = np.concatenate([codes, tail], axis=-1)
        return codes
    return _unpack_plain(buf, n, b)


def _pad_to(buf: np.ndarray, nbytes: int) -> np.ndarray:
    return np.concatenate([buf, np.zeros(buf.shape[:-1] + (nbytes - buf.shape[-1],), np.uint8)], axis=-1)


def pack_records(codec: Codec, f: dict) -> np.ndarray:
    """One contiguous record per token-head:
    [key codes | QJL sign bits | value codes | r_k f32 | rho f32 | r_v f32 | zero pad to 16 B],
    the code fields zero-padded to whole 32-bit words.
    """
    parts = [
        _pad_to(_pack_stream(f["kc"], codec.key_bits), codec.kbytes),
        _pack_stream(f["bits"], 1),
        _pad_to(_pack_stream(f["vc"], codec.value_bits), codec.vbytes),
        np.stack([f["r_k"], f["rho"], f["r_v"]], axis=-1).astype("<f4").view(np.uint8),
    ]
    rec = np.concatenate(parts, axis=-1)
    pad = codec.record_bytes - rec.shape[-1]
    return np.concatenate([rec, np.zeros(rec.shape[:-1] + (pad,), np.uint8)], axis=-1)


def unpack_records(codec: Codec, rec: np.ndarray) -> dict:
    d, m = codec.head_dim, codec.qjl_dim
    o1, o2, o3 = codec.kbytes, codec.kbytes + codec.sbytes, codec.kbytes + codec.sbytes + codec.vbytes
    norms = np.ascontiguousarray(rec[..., o3:o3 + 12]).view("<f4")
    return dict(kc=_unpack_stream(rec[..., :o1], d, codec.key_bits),
                bits=_unpack_stream(rec[..., o1:o2], m, 1),
                vc=_unpack_stream(rec[..., o2:o3], d, codec.value_bits),
                r_k=norms[..., 0], rho=norms[..., 1], r_v=norms[..., 2])


def compress_cache(codec: Codec, K: np.ndarray, V: np.ndarray, capacity: int | None = None):
    """K, V [B, T, Hkv, d] -> records [B, Hkv, capacity, record_bytes] (slots >= T zero)."""
    B, T, H, d = K.shape
    cap = T if capacity is None else capacity
    out = np.zeros((B, H, cap, codec.record_bytes), np.uint8)
    kk = np.transpose(K, (0, 2, 1, 3))
    vv = np.transpose(V, (0, 2, 1, 3))
    out[:, :, :T] = codec.pack(codec.compress_fields(kk, vv))
    return out


def quantize_from_rotated(codec: Codec, z_k, p, r_k, rho, z_v, r_v) -> np.ndarray:
    """Records from given float32 rotated coordinates: z_k, z_v [n, d] (already scaled by
    sqrt(d)/r), QJL projections p [n, m], norms [n]."""
    f = dict(kc=quantize(np.asarray(z_k, np.float32), codec.key_bounds),
             bits=(np.asarray(p, np.float32) >= 0).astype(np.int64),
             vc=quantize(np.asarray(z_v, np.float32), codec.val_bounds),
             r_k=np.asarray(r_k, np.float32), rho=np.asarray(rho, np.float32),
             r_v=np.asarray(r_v, np.float32))
    return pack_records(codec, f)


# ----------------------------------------------------------------------------------------
# Scores from the compressed keys (TurboQuant page, "QJL", the asymmetric estimator)
# ----------------------------------------------------------------------------------------
def prepare_query(codec: Codec, q: np.ndarray):
    """q_x = Pi q (the query in the rotated basis) and q_s = S q_x."""
    qx = np.asarray(q, np.float64) @ codec.Pi64.T
    qs = qx @ codec.S64.T
    return qx, qs


def score_estimates(codec: Codec, qx: np.ndarray, qs: np.ndarray, f: dict) -> np.ndarray:
    """Inner-product estimates for one query against records [n]:

    s_t = (r_t / sqrt(d)) * <q_x, gamma[c_t]> + sqrt(pi/2) / m * rho_t * <q_s, 2 bit_t - 1>.

    The second term is the QJL estimator of <q_x, e_t>; its constant comes from
    E[sign(<s, e>) <s, q>] = sqrt(2/pi) <q, e> / |e| for s ~ N(0, I) (reading: the page
    names only "a special estimator" that is unbiased).
    """
    m = codec.qjl_dim
    s = codec.key_part(qx, f)
    if m:
        sgn = 2.0 * f["bits"].astype(np.float64) - 1.0
        s = s + math.sqrt(math.pi / 2.0) / m * f["rho"].astype(np.float64) * (sgn @ qs)
    return s


def value_sum_rotated(codec: Codec, f: dict, w: np.ndarray) -> np.ndarray:
    """sum_t w_t * (r_v,t / sqrt(d)) * gamma_v[c_t] in the rotated basis."""
    d = codec.head_dim
    gv = codec.val_levels.astype(np.float64)
    vhat = (f["r_v"].astype(np.float64) / math.sqrt(d))[:, None] * gv[f["vc"]]
    return w @ vhat


# ----------------------------------------------------------------------------------------
# Decode attention over the compressed cache (+ optional exact segment, optional gather)
# ----------------------------------------------------------------------------------------
def decode_attention(codec: Codec, q, records, seq_lens, hot_k=None, hot_v=None,
                     hot_lens=None, sel_idx=None, scale=None, heads=None):
    """Attention of decode queries q [B, Hq, d] over records [B, Hkv, cap, R].

    Cold token t of sequence b: logit = scale * s_t (score_estimates).  Exact (hot)
    tokens hot_k/hot_v [B, Hkv, cap_hot, d]: logit = scale * <q, k>; they share one
    softmax with the cold tokens (Monarch v3 page, "Wie es funktioniert": recent tokens
    exact, older compressed).  sel_idx [B, Hkv, k] (-1 padded) restricts the cold tokens
    to a selected set (Self-Indexing page, sparse attention on selected tokens).
    Output o = Pi^T (sum_cold p_t vhat_t) + sum_hot p_t v_t, normalised by sum p.
    scale defaults to 1/sqrt(d) (reading: the pages do not state a logit scale).
    Returns out [B, Hq, d] f64, lse [B, Hq] f64 and per-head cold logits (dict).
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = records.shape[1]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d) if not scale else float(scale)
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    logits = {}
    for b in range(B):
        for h in range(Hq) if heads is None else heads:
            g = h // G
            if sel_idx is not None:
                idx = np.asarray(sel_idx[b, g])
                idx = idx[idx >= 0]
            else:
                idx = np.arange(int(seq_lens[b]))
            f = codec.unpack(records[b, g, idx])
            qx, qs = prepare_query(codec, q[b, h])
            lc = sc * score_estimates(codec, qx, qs, f)
            nh = 0 if hot_lens is None else int(hot_lens[b])
            lh = np.zeros(0)
            if nh:
                hk = np.asarray(hot_k[b, g, :nh], np.float64)
                lh = sc * (hk @ np.asarray(q[b, h], np.float64))
            logits[(b, h)] = (lc, lh)
            allv = np.concatenate([lc, lh])
            if allv.size == 0:
                continue
            mx = np.max(allv)
            pc, ph = np.exp(lc - mx), np.exp(lh - mx)
            l = pc.sum() + ph.sum()
            o = codec.Pi64.T @ value_sum_rotated(codec, f, pc)
            if nh:
                o = o + ph @ np.asarray(hot_v[b, g, :nh], np.float64)
            out[b, h] = o / l
            lse[b, h] = mx + math.log(l)
    return out, lse, logits


def score_scan(codec: Codec, q, records, n_tokens: int):
    """Bulk scan: q [B, Hkv, nq, d] against every record [B, Hkv, :n_tokens] ->
    estimates [B, Hkv, nq, n_tokens] (no softmax).  TurboQuant page, "Leistung bei der
    Vektorsuche": inner-product search over the compressed vectors."""
    B, H, nq, d = q.shape
    out = np.zeros((B, H, nq, n_tokens))
    for b in range(B):
        for h in range(H):
            f = codec.unpack(records[b, h, :n_tokens])
            for i in range(nq):
                qx, qs = prepare_query(codec, q[b, h, i])
                out[b, h, i] = score_estimates(codec, qx, qs, f)
    return out


def recall_1_at_k(approx: np.ndarray, exact: np.ndarray, ks) -> dict:
    """1@k recall (TurboQuant page, "Leistung bei der Vektorsuche"): the fraction of queries
    whose best database vector by exact inner product is among the k best by the approximate
    scores.  approx, exact [n_queries, n].  Readings: the exact best is the lowest index
    among the exact maxima; in the approximate ranking a tie goes to the lower index, so the
    best's rank is #{j : a_j > a_best} + #{j < best : a_j = a_best}."""
    approx = np.asarray(approx, np.float64)
    exact = np.asarray(exact, np.float64)
    nq, n = exact.shape
    best = np.argmax(exact, axis=1)
    a = approx[np.arange(nq), best][:, None]
    idx = np.arange(n)[None, :]
    rank = np.sum(approx > a, axis=1) + np.sum((approx == a) & (idx < best[:, None]), axis=1)
    return {int(k): float(np.mean(rank < k)) for k in ks}


# ----------------------------------------------------------------------------------------
# Self-Indexing sign index and compressed-domain top-k
# ----------------------------------------------------------------------------------------
def sign_patterns(k: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """4-bit sign pattern of every 4-channel group of keys k [n, d] (float32) against the
    channel mean mu [d] (float32): bit j of group g is [k_(4g+j) >= mu_(4g+j)], a float32
    comparison.  Self-Indexing page, "Methodologie" 1-2.  Returns [n, d/4] int64."""
    n, d = k.shape
    bits = (np.asarray(k, np.float32) >= np.asarray(mu, np.float32)).astype(np.int64).reshape(n, d // 4, 4)
    return np.sum(bits << np.arange(4), axis=-1)


def pattern_centroids(k: np.ndarray, mu: np.ndarray, pat: np.ndarray) -> np.ndarray:
    """The 16 centroids of every group (Self-Indexing page, "Methodologie" 2, built in one
    pass): centroid (g, p) is the float64 mean of (k - mu) over the group-g sub-vectors of the
    tokens whose pattern is p, rounded to float32; 0 when no token has that pattern.
    k [n, d] float32, mu [d] float32, pat [n, d/4].  Returns [d/4, 16, 4] float32."""
    n, d = k.shape
    ng = d // 4
    book = np.zeros((ng, 16, 4), np.float32)
    cen = np.asarray(k, np.float64).reshape(n, ng, 4) - np.asarray(mu, np.float64).reshape(ng, 4)
    for g in range(ng):
        for p in range(16):
            sel = pat[:, g] == p
            if sel.any():
                book[g, p] = np.mean(cen[sel, g], axis=0).astype(np.float32)
    return book


def build_sign_index(codec: Codec, K: np.ndarray, n_tokens: int):
    """Sign index of keys K [B, T, Hkv, d] over tokens [0, n_tokens).

    Self-Indexing page, "Methodologie" 1-2: subtract the channel mean mu (so signs are
    balanced), take the sign of each channel, pack the 4 signs of each 4-dim group into a
    pattern 0..15, and build 16 centroids per group in one pass.  Readings: unrotated
    basis; mu is the float32-rounded mean over the tokens indexed; bit = [k >= mu] in
    float32 (sign_patterns); centroid = mean of the members' (k - mu) sub-vectors (float32),
    0 if the pattern has no member (pattern_centroids); pattern bit j = channel 4g + j.
    Returns index [B, Hkv, cap=T, d/8] u8, codebook [B, Hkv, d/4, 16, 4] f32, mu [B, Hkv, d] f32.
    """
    B, T, H, d = K.shape
    ng = d // 4
    index = np.zeros((B, H, T, d // 8), np.uint8)
    book = np.zeros((B, H, ng, 16, 4), np.float32)
    mus = np.zeros((B, H, d), np.float32)
    for b in range(B):
        for h in range(H):
            k = np.asarray(K[b, :n_tokens, h], np.float32)
            mu = np.mean(k.astype(np.float64), axis=0).astype(np.float32)
            pat = sign_patterns(k, mu)                                        # [n, ng]
            book[b, h] = pattern_centroids(k, mu, pat)
            index[b, h, :n_tokens] = _pack_stream(pat, 4)
            mus[b, h] = mu
    return index, book, mus


def lut_scale_exponent(maxabs: float, n_terms: int) -> int:
    """Largest integer s with n_terms * maxabs * 2^s <= 2^30 (0 when maxabs == 0), so that
    sums of n_terms rounded table entries fit in int32."""
    a = float(n_terms) * maxabs
    if a == 0.0:
        return 0
    f, e = math.frexp(a)  # a = f * 2^e, 0.5 <= f < 1
    return 30 - e + (1 if f == 0.5 else 0)


def select_topk(codec: Codec, q, index, book, seq_lens, k: int):
    """Top-k tokens per (sequence, KV head) from the sign index (Self-Indexing page,
    "Methodologie" 3: LUT-GEMV, a per-query table of <q_g, centroid> read back by
    lookup-and-add).  Readings: the table is built in float64 as
    ((q0 c0 + q1 c1) + q2 c2) + q3 c3, scaled by 2^s (lut_scale_exponent over all G heads
    of the group) and rounded half-to-even to integers; a token's score is the integer sum
    over groups and over the G query heads sharing the KV head; ties go to the lower token
    index; the k chosen indices are returned in ascending order, padded with -1.
    Returns idx [B, Hkv, k] i32, count [B, Hkv] i32, scores [B, Hkv, k] i32 (of idx).
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    H = index.shape[1]
    G = Hq // H
    ng = d // 4
    idx_out = np.full((B, H, k), -1, np.int32)
    cnt = np.zeros((B, H), np.int32)
    sc_out = np.zeros((B, H, k), np.int32)
    for b in range(B):
        n = int(seq_lens[b])
        for h in range(H):
            c = book[b, h].astype(np.float64)                                # [ng, 16, 4]
            luts = []
            for j in range(G):
                qg = q[b, h * G + j].astype(np.float64).reshape(ng, 1, 4)
                t = qg[..., 0] * c[..., 0]
                t = t + qg[..., 1] * c[..., 1]
                t = t + qg[..., 2] * c[..., 2]
                t = t + qg[..., 3] * c[..., 3]
                luts.append(t)                                               # [ng, 16]
            maxabs = max(float(np.max(np.abs(t))) for t in luts)
            s = lut_scale_exponent(maxabs, G * ng)
            lut = sum(np.rint(t * 2.0 ** s).astype(np.int64) for t in luts)   # [ng, 16]
            pat = _unpack_stream(index[b, h, :n], ng, 4)                     # [n, ng]
            score = np.sum(lut[np.arange(ng)[None, :], pat], axis=1)          # [n]
            assert np.all(np.abs(score) < 2 ** 31)
            order = np.lexsort((np.arange(n), -score))[: min(k, n)]
            chosen = np.sort(order)
            cnt[b, h] = len(chosen)
            idx_out[b, h, : len(chosen)] = chosen
            sc_out[b, h, : len(chosen)] = score[chosen]
    return idx_out, cnt, sc_out
