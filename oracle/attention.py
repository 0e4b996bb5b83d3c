"""Decode attention over an NSN-quantized KV cache plus an fp16 residual
window -- numpy float64 reference.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[NSNQuant summary (gist.science), Methodology §4: the cache is a quantized
part plus a full-precision residual of recent tokens, flushed, quantized and
appended when full (following KIVI); the attention score consumes the NSN
byproducts s1, s2, o directly.]

Definition used here (``decode_attention``): for every batch b and query
head h, with kv head kvh = h // (Hq / Hkv) (contiguous grouping),
    keys   = [dequantize(K cache of (b, kvh), first Nq tokens) ; K_resid(b, kvh, :R)]
    values = [dequantize(V cache ...)                          ; V_resid(b, kvh, :R)]
    s = scale * keys @ q[b, h];  p = softmax(s) (max-subtracted);  out = p @ values.
No RoPE and no mask (reading: the workload carries no positions; keys are
attended as stored).

``decode_attention_rotated`` computes the same result the way the byproducts
enter the score directly: with q' = H q / sqrt(d),
    score_t = scale * s1_t * (s2'_t <q', h_hat_t> + <q', o'_g>)
and the value sum formed in the rotated domain, rotated back once, plus the
residual in the channel domain.  The pin tests check the two agree.

Pins (tests/test_oracle_attention.py): agreement with a plain per-head loop
using scipy.special.softmax; the rotated-domain identity; q = 0 gives the
mean of the values; Nq = 0 gives plain attention over the residual; a single
key returns its value.  With the randomized rotation (``signs``; pins in
tests/test_oracle_rht.py): the rotated-domain identity again, and equality
with the plain attention of sign-flipped queries, keys and values, flipped
back.

``decode_attention_rope`` is the same attention with the keys stored before
rotary position embedding, the order the pages give for keys (Methodology
§4: NSN is applied to keys before RoPE).  The pages fix neither the RoPE
variant nor its base nor the positions; readings: the rotate-half form
(channel pairs (i, i + d/2), frequency theta_i = base^(-2i/d)), a caller-given
base, cache token t at position t, residual token r at position n_quant + r,
and the query at a caller-given position; RoPE is applied to the query and
to every key (dequantized or residual), values are unchanged.  Pins: the
closed forms of the pair rotation (sin and cos of the position difference
times the pair's frequency), norm preservation, composition of rotations,
invariance of the output under a common position shift, and reduction to
``decode_attention`` when every position is zero.
"""

import numpy as np

from .nsn import dequantize, rht, rht_inverse

__all__ = ["attend", "decode_attention", "decode_attention_rotated", "apply_rope",
           "decode_attention_rope"]


def attend(q, keys, values, scale):
    """Single-query softmax attention in float64.  q (d,), keys/values (N, d)."""
    s = scale * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))
    s = s - s.max()
    p = np.exp(s)
    p /= p.sum()
    return p @ np.asarray(values, np.float64)


def _kv_rows(cache, b, kvh, n_quant, C, G, signs=None):
    codes, meta, shift = cache
    if n_quant == 0:
        return np.zeros((0, codes.shape[-1] * C.shape[1]))
    return dequantize(codes[b, kvh, :n_quant], meta[b, kvh, :n_quant],
                      shift[b, kvh, :n_quant // G], C, G, signs=signs)


def decode_attention(q, k_cache, v_cache, k_resid, v_resid, C, G, n_quant,
                     n_resid, scale, heads=None, signs=None):
    """q: (B, Hq, d); k_cache/v_cache: (codes (B, Hkv, cap, d/m) uint8,
    meta (B, Hkv, cap, 2) fp16, shift (B, Hkv, cap/G, d) fp16);
    k_resid/v_resid: (B, Hkv, Rcap, d) fp16.  Returns float64 (B, Hq, d).
    ``heads``: optional list of (b, h) pairs to compute (others left NaN).
    ``signs``: the caches were quantized with the randomized rotation of
    these channel signs (dequantized with its inverse)."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache[0].shape[1]
    grp = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    cached = {}
    for b, h in todo:
        kvh = h // grp
        if (b, kvh) not in cached:
            keys = np.concatenate([_kv_rows(k_cache, b, kvh, n_quant, C, G, signs),
                                   np.asarray(k_resid[b, kvh, :n_resid], np.float64)])
            vals = np.concatenate([_kv_rows(v_cache, b, kvh, n_quant, C, G, signs),
                                   np.asarray(v_resid[b, kvh, :n_resid], np.float64)])
            cached = {(b, kvh): (keys, vals)}
        keys, vals = cached[(b, kvh)]
        out[b, h] = attend(q[b, h], keys, vals, scale)
    return out


def decode_attention_rotated(q, k_cache, v_cache, k_resid, v_resid, C, G,
                             n_quant, n_resid, scale, signs=None):
    """Same result, with the NSN byproducts folded into the score and the
    quantized values summed in the rotated domain (one rotation back).  With
    ``signs`` the query enters as q' = (H / sqrt(d)) D q and the value sum
    leaves through D (H / sqrt(d))."""
    q = np.asarray(q, np.float64)
    C = np.asarray(C, np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache[0].shape[1]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kvh = h // grp
            qr = rht(q[b, h], signs)
            parts_s = []
            if n_quant:
                kc, km, ks = (a[b, kvh] for a in k_cache)
                kh = C[kc[:n_quant].astype(np.int64)].reshape(n_quant, d)
                s1 = km[:n_quant, 0].astype(np.float64)
                s2 = km[:n_quant, 1].astype(np.float64)
                qo = ks[:n_quant // G].astype(np.float64) @ qr
                sq = scale * s1 * (s2 * (kh @ qr) + np.repeat(qo, G)[:n_quant])
                parts_s.append(sq)
            kr = np.asarray(k_resid[b, kvh, :n_resid], np.float64)
            parts_s.append(scale * (kr @ q[b, h]))
            s = np.concatenate(parts_s)
            p = np.exp(s - s.max())
            p /= p.sum()
            acc_rot = np.zeros(d)
            if n_quant:
                vc, vm, vs = (a[b, kvh] for a in v_cache)
                vh = C[vc[:n_quant].astype(np.int64)].reshape(n_quant, d)
                w = p[:n_quant] * vm[:n_quant, 0].astype(np.float64)
                acc_rot += (w * vm[:n_quant, 1].astype(np.float64)) @ vh
                wg = w.reshape(n_quant // G, G).sum(axis=1)
                acc_rot += wg @ vs[:n_quant // G].astype(np.float64)
            vr = np.asarray(v_resid[b, kvh, :n_resid], np.float64)
            out[b, h] = rht_inverse(acc_rot, signs) + p[n_quant:] @ vr
    return out


def apply_rope(x, pos, base):
    """Rotate-half rotary embedding in float64: for i < d/2 the channel pair
    (x_i, x_{i+d/2}) is rotated by the angle pos * base^(-2i/d).
    x (..., d); pos broadcasts against x's leading dimensions."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = float(base) ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(pos, np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attend_rope(q, keys, values, scale, q_pos, key_pos, base):
    """``attend`` with RoPE applied to the query (at q_pos) and to every key
    (at key_pos[t])."""
    return attend(apply_rope(q, q_pos, base), apply_rope(keys, key_pos, base), values, scale)


def decode_attention_rope(q, k_cache, v_cache, k_resid, v_resid, C, G, n_quant,
                          n_resid, scale, q_pos, base, heads=None, signs=None):
    """``decode_attention`` over keys stored before RoPE: key t of a (b, kv
    head) row (quantized tokens first, then the residual) sits at position t,
    the query at q_pos.  Same arguments plus q_pos and the RoPE base."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache[0].shape[1]
    grp = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    cached = {}
    for b, h in todo:
        kvh = h // grp
        if (b, kvh) not in cached:
            keys = np.concatenate([_kv_rows(k_cache, b, kvh, n_quant, C, G, signs),
                                   np.asarray(k_resid[b, kvh, :n_resid], np.float64)])
            vals = np.concatenate([_kv_rows(v_cache, b, kvh, n_quant, C, G, signs),
                                   np.asarray(v_resid[b, kvh, :n_resid], np.float64)])
            cached = {(b, kvh): (keys, vals)}
        keys, vals = cached[(b, kvh)]
        out[b, h] = attend_rope(q[b, h], keys, vals, scale, q_pos,
                                np.arange(keys.shape[0]), base)
    return out
