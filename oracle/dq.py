"""Double quantization (DQ) of the NSN byproducts and of the codebook --
numpy reference.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[NSNQuant summary (gist.science), Methodology §3, Double Quantization: the
NSN parameters (the mean o and the scale s1) and the codebook entries are
themselves quantized to 4 bits, for an overhead of about 0.23 bits per
value on average.]

The pages give neither the grids nor the second-level scales.  Readings:

  * s1 (one per token): per group of G tokens, the fp16 minimum and maximum
    of s1 span a 16-level linear grid; code = round((s1 - lo) / (hi - lo) *
    15) clamped to [0, 15] (round half to even; all codes 0 when hi == lo);
    decoded s1 = lo + code * (hi - lo) / 15.
  * o (stored rotated, o' = H o / sqrt(d), one value per channel per group):
    symmetric 4-bit, scale = fp16(max |o'| / 7); code = round(o' / scale)
    clamped to [-7, 7], stored as code + 8 (1..15; 0 when the scale is 0);
    decoded o' = (code - 8) * scale.
  * s2' keeps fp16 (the pages name only o and s1).
  * The decisions (codes) are the reading's definitions evaluated exactly
    (float64) on the unrounded s1 and o' and the stored fp16 lo, hi and
    scale; an implementation that divides in lower precision can land on
    the other side of an exact half step only within its rounding error.
  * Record per group (little-endian): fp16 lo, fp16 hi, fp16 scale, 2 zero
    bytes; 64 bytes of o' codes (channel c in byte c // 2, low nibble for
    even c); G / 2 bytes of s1 codes (token t of the group likewise).
    136 bytes for G = 128.  With s2' (2 bytes per token) the metadata costs
    (2 + 136 / 128) * 8 / 128 = 0.19 bits per value at G = 128, against
    0.375 bits for fp16 (s1, s2', o').
  * Codebook entries: the 16 levels (k - 7.5) * 3/8, k = 0..15 (symmetric,
    exact in fp16, covering the +-2.8 range of N(0,1) k-means codebooks);
    each entry goes to the nearest level (ties to the level of smaller
    magnitude, an entry of 0 to +3/16).

Pins (tests/test_oracle_dq.py): exact round trips for values on the grids;
error bounds of half a grid step otherwise; codes of the end points; sign
symmetry of o'; nibble packing; the record size; grid membership and
nearest-level property of the 4-bit codebook.
"""

import numpy as np

__all__ = ["record_bytes", "dq_encode_group", "dq_decode_group", "dq_pack", "dq_unpack",
           "codebook_4bit", "CB_LEVELS"]

CB_STEP = 0.375
CB_LEVELS = (np.arange(16) - 7.5) * CB_STEP


def record_bytes(G):
    """Bytes of one group record: 8 (lo, hi, scale, pad) + 64 (o') + G / 2 (s1)."""
    return 8 + 64 + G // 2


def _pack_nibbles(v):
    v = np.asarray(v, np.uint8)
    return (v[0::2] | (v[1::2] << 4)).astype(np.uint8)


def _unpack_nibbles(b, n):
    b = np.asarray(b, np.uint8)
    out = np.empty(2 * b.size, np.uint8)
    out[0::2] = b & 15
    out[1::2] = b >> 4
    return out[:n]


def dq_encode_group(s1, o_rot):
    """One group: s1 (G,) float, o_rot (d,) float -> record bytes (uint8)."""
    s1 = np.asarray(s1, np.float64)
    o_rot = np.asarray(o_rot, np.float64)
    lo16, hi16 = np.float16(s1.min()), np.float16(s1.max())
    lo, hi = np.float64(lo16), np.float64(hi16)
    if hi > lo:
        t = (s1 - lo) * 15.0 / (hi - lo)
        c1 = np.clip(np.rint(t).astype(np.int64), 0, 15)
    else:
        c1 = np.zeros(s1.size, np.int64)
    sc16 = np.float16(np.abs(o_rot).max() / 7.0)
    sc = np.float64(sc16)
    if sc > 0:
        t = o_rot / sc
        co = np.clip(np.rint(t).astype(np.int64), -7, 7) + 8
    else:
        co = np.zeros(o_rot.size, np.int64)
    head = np.array([lo16, hi16, sc16, np.float16(0)], np.float16).view(np.uint8)
    return np.concatenate([head, _pack_nibbles(co), _pack_nibbles(c1)])


def dq_decode_group(rec, G, d=128):
    """Record -> (s1 (G,) float64, o_rot (d,) float64), the decoded values."""
    rec = np.asarray(rec, np.uint8)
    head = rec[:8].view(np.float16).astype(np.float64)
    lo, hi, sc = head[0], head[1], head[2]
    co = _unpack_nibbles(rec[8:8 + d // 2], d).astype(np.int64)
    c1 = _unpack_nibbles(rec[8 + d // 2:8 + d // 2 + G // 2], G).astype(np.float64)
    o_rot = np.where(co == 0, 0.0, (co - 8) * sc)
    s1 = lo + c1 * (hi - lo) / 15.0
    return s1, o_rot


def dq_pack(meta, shift, s1_exact, o_rot_exact, G):
    """DQ storage of one sequence from ``quantize``'s outputs and internals:
    s2' fp16 (T,) and records uint8 (T/G, record_bytes(G)).  The codes are
    taken from the unrounded s1 and o' (forward arithmetic is unrounded)."""
    T = meta.shape[0]
    recs = np.stack([dq_encode_group(s1_exact[g * G:(g + 1) * G], o_rot_exact[g])
                     for g in range(T // G)]) if T else np.zeros((0, record_bytes(G)), np.uint8)
    return np.asarray(meta)[:, 1].astype(np.float16), recs


def dq_unpack(s2, recs, G, d=128):
    """-> (meta float64 (T, 2) = (s1, s2'), shift float64 (T/G, d)), the
    decoded values that dequantization and attention take as exact."""
    s2 = np.asarray(s2).astype(np.float64)
    T = s2.shape[0]
    s1 = np.zeros(T)
    shift = np.zeros((T // G, d))
    for g in range(T // G):
        s1[g * G:(g + 1) * G], shift[g] = dq_decode_group(recs[g], G, d)
    return np.stack([s1, s2], axis=-1), shift


def codebook_4bit(C):
    """Each entry to the nearest of the 16 levels; a tie goes to the level of
    smaller magnitude, and between -3/16 and +3/16 (an entry of 0) to +3/16."""
    C = np.asarray(C, np.float64)
    out = np.empty(C.shape, np.float32)
    for idx, v in np.ndenumerate(C):
        dist = np.abs(v - CB_LEVELS)
        cand = CB_LEVELS[dist == dist.min()]
        cand = cand[np.abs(cand) == np.abs(cand).min()]
        out[idx] = cand.max()
    return out
