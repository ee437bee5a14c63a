"""Oracle of the hot/cold decode step: a plain numpy state machine.

TEST INFRASTRUCTURE ONLY, like tq_oracle (which it calls for compression, record packing,
score estimates and attention); nothing in the product path imports it.

Monarch v3 page (openclawradar.com), "Wie es funktioniert" and the decode loop printed
below it: recent tokens stay exact in a hot region, older ones are compressed into a cold
region; a query reads the cold region only when the hot scores are low; cold tokens that
draw high attention move back to the hot region, with a sticky rule against thrashing; a
sliding window evicts the oldest hot tokens into the cold region.  The page fixes no
numbers beyond the two command-line thresholds (0.15, 3) and leaves these readings open:

* M1 gate: per query head, the hot "scores" are the logits scale * <q, k> the softmax
  uses; the head reads the cold tokens iff max over hot tokens < cold_gate.
* M2 order: the step's token joins the hot region first; attention sees the state after
  that; promotion and eviction change the state for the next step only.
* M3 promotion weight: a cold token's weight in a step is the largest softmax probability
  it receives from the query heads that read the cold region (0 when none does).
* M4 sticky rule: a per-token count of consecutive steps with weight >= promote_weight
  (reset to 0 otherwise); at promote_steps the token is promoted.
* M5 page swap: a promoted token is decompressed (k = Pi^T (r_k/sqrt(d)) gamma_k[c],
  v = Pi^T (r_v/sqrt(d)) gamma_v[c_v] in float64, rounded to the hot dtype; the QJL bits
  cannot be undone; with polar key codes k = Pi^T (r_k u), u the unit vector of the grid
  angles) and joins the hot region as its newest token, promoted tokens in ascending cold
  order; its cold slot is filled by the last cold token, slots handled from the highest
  down.
* M6 eviction: while the hot region holds more than `window` tokens its oldest are
  compressed (by the codec's own compress: tq_oracle.compress, or the polar codec's) and
  appended to the cold region with count 0; when the cold region is full they are dropped
  and an overflow flag is set.

The codec is either tq_oracle.Codec or polar.PolarCodec (the Monarch page's cold tier codes
keys with polar angles); the step calls only the codec's compress, pack, unpack and key
reconstruction.
"""
from __future__ import annotations

import math

import numpy as np

from . import tq_oracle as O


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits), ties to even."""
    x = np.asarray(x, np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    ax = np.abs(x[nz])
    e = np.floor(np.log2(ax))
    e = e - (np.exp2(e) > ax) + (np.exp2(e + 1) <= ax)       # 2^e <= |x| < 2^(e+1)
    ulp = np.exp2(e - 7)
    out[nz] = np.rint(x[nz] / ulp) * ulp
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> the hot dtype (values kept as float64)."""
    if dtype == "float32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    if dtype == "float16":
        return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)
    return round_to_bf16(x)


class HotColdOracle:
    def __init__(self, codec: O.Codec, batch: int, kv_heads: int, hot_dtype: str, cold_capacity: int):
        d = codec.head_dim
        self.codec, self.dtype, self.cold_cap = codec, hot_dtype, cold_capacity
        self.hot_k = [np.zeros((kv_heads, 0, d)) for _ in range(batch)]
        self.hot_v = [np.zeros((kv_heads, 0, d)) for _ in range(batch)]
        self.cold = [np.zeros((kv_heads, 0, codec.record_bytes), np.uint8) for _ in range(batch)]
        self.hits = [np.zeros(0, np.int64) for _ in range(batch)]
        self.overflow = [False] * batch

    def dequantize(self, rec: np.ndarray):
        """Promoted token of one KV head: its record -> (k, v) in the hot dtype (M5)."""
        c = self.codec
        f = c.unpack(rec[None])
        sd = math.sqrt(c.head_dim)
        xk = c.key_vector(f)[0]
        xv = (float(f["r_v"][0]) / sd) * c.val_levels.astype(np.float64)[f["vc"][0]]
        return round_to(c.Pi64.T @ xk, self.dtype), round_to(c.Pi64.T @ xv, self.dtype)

    def step(self, q, k_new, v_new, window, cold_gate=math.inf, promote_weight=0.15, promote_steps=3,
             scale=None):
        """q [B, Hq, d]; k_new, v_new [B, Hkv, d] (values of the hot dtype).  Returns
        out [B, Hq, d], lse [B, Hq], gate [B, Hq] (bool) and, per sequence, the cold weights
        used by the sticky rule (for margin checks)."""
        c = self.codec
        q = np.asarray(q, np.float64)
        B, Hq, d = q.shape
        H = self.hot_k[0].shape[0]
        G = Hq // H
        sc = 1.0 / math.sqrt(d) if not scale else float(scale)
        out = np.zeros((B, Hq, d))
        lse = np.zeros((B, Hq))
        gate = np.zeros((B, Hq), bool)
        weights = []
        for b in range(B):
            # M2: the step's token joins the hot region
            self.hot_k[b] = np.concatenate([self.hot_k[b], np.asarray(k_new[b], np.float64)[:, None]], axis=1)
            self.hot_v[b] = np.concatenate([self.hot_v[b], np.asarray(v_new[b], np.float64)[:, None]], axis=1)
            nh, nc = self.hot_k[b].shape[1], self.cold[b].shape[1]
            for h in range(Hq):                                              # M1
                gate[b, h] = np.max(sc * (self.hot_k[b][h // G] @ q[b, h])) < cold_gate
            rec = self.cold[b][None]
            hk, hv = self.hot_k[b][None], self.hot_v[b][None]
            open_h = [h for h in range(Hq) if gate[b, h]]
            shut_h = [h for h in range(Hq) if not gate[b, h]]
            lg = {}
            for heads, ncold in ((open_h, nc), (shut_h, 0)):
                if heads:
                    o, l, lgh = O.decode_attention(c, q[b:b + 1], rec, [ncold], hk, hv, [nh], scale=sc,
                                                   heads=heads)
                    for h in heads:
                        out[b, h], lse[b, h] = o[0, h], l[0, h]
                        lg[h] = lgh[(0, h)][0]
            # M3, M4: weights of the cold tokens and the sticky counts
            w = np.zeros(nc)
            for h in open_h:
                w = np.maximum(w, np.exp(lg[h] - lse[b, h]))
            weights.append(w)
            promoted = []
            if promote_steps > 0:
                hits = np.where(w >= promote_weight, self.hits[b] + 1, 0)
                promoted = [int(t) for t in np.nonzero(hits >= promote_steps)[0]]
                hits[promoted] = 0
                self.hits[b] = hits
            # M5: page swap into the hot region, then swap-remove from the cold region
            for t in promoted:
                kv = [self.dequantize(self.cold[b][h, t]) for h in range(H)]
                self.hot_k[b] = np.concatenate([self.hot_k[b], np.stack([x[0] for x in kv])[:, None]], axis=1)
                self.hot_v[b] = np.concatenate([self.hot_v[b], np.stack([x[1] for x in kv])[:, None]], axis=1)
            cold, hits = self.cold[b].copy(), self.hits[b].copy()
            n = nc
            for t in sorted(promoted, reverse=True):
                last = n - 1
                if t != last:
                    cold[:, t] = cold[:, last]
                    hits[t] = hits[last]
                n -= 1
            self.cold[b], self.hits[b] = cold[:, :n], hits[:n]
            # M6: sliding window
            e = max(0, self.hot_k[b].shape[1] - window)
            keep = min(e, self.cold_cap - n)
            if keep:
                kk = self.hot_k[b][:, :keep].astype(np.float32)
                vv = self.hot_v[b][:, :keep].astype(np.float32)
                recs = c.pack(c.compress_fields(kk, vv))                    # [H, keep, R]
                self.cold[b] = np.concatenate([self.cold[b], recs], axis=1)
                self.hits[b] = np.concatenate([self.hits[b], np.zeros(keep, np.int64)])
            if keep < e:
                self.overflow[b] = True
            self.hot_k[b], self.hot_v[b] = self.hot_k[b][:, e:], self.hot_v[b][:, e:]
        return out, lse, gate, weights
