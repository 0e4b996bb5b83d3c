"""Comparison rules between the HIP library and the oracle (test helpers).

Codes: a GPU code g that differs from the oracle's o is accepted only as a
near-tie: D(g) - D(o) <= 1e-5 * max(D(o), 1e-12), with D the exact squared
distance computed in float64 on the oracle's own rotated vector h.

Metadata: s1 and the group shift within one fp16 ulp of the oracle; s2'
within one ulp of the oracle's value recomputed with the GPU's codes (a
near-tie flip legitimately changes the scale-adjust factor).

Reconstruction: the GPU's dequantization of its own bytes matches the
oracle's dequantization of the same bytes to 1e-5 relative L2 (fp32
output); against the oracle's own reconstruction, 1e-3 relative L2.

Attention: on the same cache bytes, max-abs 2e-3 against the oracle and,
per (batch, q head), relative L2 1e-4 (the codes are shared, so only the
fp32 accumulation differs; 2e-3 alone would let a dropped token group pass).
"""

import numpy as np

import oracle

TIE_REL = 1e-5
RECON_REL = 1e-3
SAME_BYTES_REL = 1e-5
ATTN_ABS = 2e-3
ATTN_REL = 1e-4


def ulp16(v):
    """Spacing of fp16 at |v| (float64)."""
    v = np.abs(np.asarray(v, dtype=np.float16))
    return np.spacing(v).astype(np.float64)


def _check_codes(h_flat, C64, codes_g, codes_o):
    """Codes equal to the oracle's except validated near-ties; returns their
    number."""
    T, m = h_flat.shape[0], C64.shape[1]
    assert codes_g.shape == codes_o.shape, (codes_g.shape, codes_o.shape)
    h = h_flat.reshape(T, -1, m)
    mism = np.argwhere(codes_g != codes_o)
    n_ties = 0
    for t, j in mism:
        g, o = int(codes_g[t, j]), int(codes_o[t, j])
        dg = float(np.sum((h[t, j] - C64[g]) ** 2))
        do = float(np.sum((h[t, j] - C64[o]) ** 2))
        assert dg - do <= TIE_REL * max(do, 1e-12), (
            f"code mismatch at token {t}, sub-vector {j}: gpu {g} (D={dg:.9g}) vs oracle {o} "
            f"(D={do:.9g})")
        n_ties += 1
    return n_ties


def _check_s2(it, C64, codes_g, s2_g, scale_adjust):
    """s2' within one fp16 ulp of the oracle's value for the GPU's codes."""
    T = codes_g.shape[0]
    hh = C64[codes_g.astype(np.int64)].reshape(T, -1)
    alpha = oracle.scale_adjust(it["h"], hh) if scale_adjust else np.ones(T)
    s2p = it["s2"] * alpha
    s2_g = np.asarray(s2_g).astype(np.float64)
    bad = np.abs(s2_g - s2p.astype(np.float16).astype(np.float64)) > ulp16(s2p) * 1.0001
    assert not bad.any(), f"s2' off by more than 1 ulp at tokens {np.argwhere(bad)[:5].ravel()}"


def _nibbles(b, n):
    b = np.asarray(b, np.uint8)
    out = np.empty(2 * b.size, np.int64)
    out[0::2] = b & 15
    out[1::2] = b >> 4
    return out[:n]


# Double-quantized codes: the oracle decides them exactly (float64); the GPU
# divides in float32 from its own float32 s1 and o'.  A code may differ by one
# only where the exact grid coordinate t lies within the GPU's rounding error
# of a half step: DQ_TIE grid steps for o' (t = o'/sc, the float32 mean is
# good to ~1e-6 absolute and sc >= 1e-3 on these inputs), plus, for s1
# (t = (s1 - lo) * 15 / (hi - lo)), the float32 s1's relative error S1_REL
# scaled by 15 * s1 / (hi - lo).
DQ_TIE = 1e-3
S1_REL = 4e-6


def check_dq_sequence(x, C4, codes_g, s2_g, recs_g, scale_adjust=True, G=128, signs=None):
    """Double-quantized output of one sequence against the oracle run on the
    4-bit codebook C4: codes and s2' as in check_quantized_sequence; in each
    group record lo, hi and the o' scale within one fp16 ulp; where they are
    equal to the oracle's, the 4-bit codes equal its codes except near a half
    step of the grid (differing by one); elsewhere the decoded values within
    half a step of the exact ones.  Returns statistics."""
    C64 = np.asarray(C4, np.float64)
    codes_o, meta_o, shift_o, it = oracle.quantize(x, C4, G, scale_adjust_on=scale_adjust,
                                                   return_internals=True, signs=signs)
    n_ties = _check_codes(it["h"], C64, codes_g, codes_o)
    _check_s2(it, C64, codes_g, s2_g, scale_adjust)
    _, recs_o = oracle.dq_pack(meta_o, shift_o, it["s1"], it["o_rot"], G)
    recs_g = np.asarray(recs_g, np.uint8).reshape(recs_o.shape)
    d = 128
    n_hdr = n_near = 0
    for g in range(recs_o.shape[0]):
        hg = recs_g[g, :6].view(np.float16).astype(np.float64)
        ho = recs_o[g, :6].view(np.float16).astype(np.float64)
        assert np.all(np.abs(hg - ho) <= ulp16(ho) * 1.0001), (g, hg, ho)
        assert recs_g[g, 6] == 0 and recs_g[g, 7] == 0
        s1x = it["s1"][g * G:(g + 1) * G]
        ox = it["o_rot"][g]
        if np.array_equal(recs_g[g, :8], recs_o[g, :8]):
            lo, hi, sc = (float(v) for v in ho)
            for part, n, exact, ref in (("o", d, ox, None), ("s1", G, s1x, None)):
                off = 8 if part == "o" else 8 + d // 2
                cg = _nibbles(recs_g[g, off:off + n // 2], n)
                co = _nibbles(recs_o[g, off:off + n // 2], n)
                diff = np.argwhere(cg != co).ravel()
                if diff.size == 0:
                    continue
                if part == "o":
                    t = exact / sc
                    win = DQ_TIE
                else:
                    t = (exact - lo) * 15.0 / (hi - lo)
                    win = DQ_TIE + 15.0 * S1_REL * max(abs(lo), abs(hi)) / (hi - lo)
                near = np.abs(t - np.floor(t) - 0.5) < win
                assert np.all(near[diff]) and np.all(np.abs(cg[diff] - co[diff]) == 1), (
                    f"group {g} {part} codes differ away from a half step at {diff[:5]}")
                n_near += diff.size
        else:
            n_hdr += 1
            s1d, od = oracle.dq_decode_group(recs_g[g], G, d)
            lo, hi, sc = hg
            assert np.abs(s1d - s1x).max() <= (hi - lo) / 30 * 1.001 + 2 * ulp16(hi)
            assert np.abs(od - ox).max() <= sc / 2 * 1.001 + max(0.0, np.abs(ox).max() - 7 * sc) + 1e-7
    return dict(ties=n_ties, codes=codes_o.size, near=n_near, hdr=n_hdr, groups=recs_o.shape[0])


def check_quantized_sequence(x, C, G, codes_g, meta_g, shift_g, scale_adjust=True, signs=None):
    """Compare one sequence's GPU output to the oracle (with the randomized
    rotation of ``signs`` when given).  Returns a dict of statistics (number
    of accepted ties, ...).  Raises AssertionError."""
    C64 = np.asarray(C, np.float64)
    m = C64.shape[1]
    codes_o, meta_o, shift_o, it = oracle.quantize(x, C, G, scale_adjust_on=scale_adjust,
                                                   return_internals=True, signs=signs)
    n_ties = _check_codes(it["h"], C64, codes_g, codes_o)
    # s1
    s1_o = it["s1"]
    s1_g = meta_g[:, 0].astype(np.float64)
    bad = np.abs(s1_g - s1_o.astype(np.float16).astype(np.float64)) > ulp16(s1_o) * 1.0001
    assert not bad.any(), f"s1 off by more than 1 ulp at tokens {np.argwhere(bad)[:5].ravel()}"
    _check_s2(it, C64, codes_g, meta_g[:, 1], scale_adjust)
    # rotated group mean
    sh_o = it["o_rot"]
    bad = np.abs(shift_g.astype(np.float64) - sh_o.astype(np.float16).astype(np.float64)) > \
        ulp16(sh_o) * 1.0001 + 1e-7
    assert not bad.any(), f"shift off by more than 1 ulp at {np.argwhere(bad)[:5].tolist()}"
    return dict(ties=n_ties, codes=codes_o.size, codes_o=codes_o, meta_o=meta_o, shift_o=shift_o)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_attention(got, want, what=""):
    """Attention output `got` against the oracle's `want` (same shape, last
    axis the 128 channels): max-abs <= ATTN_ABS over all entries and relative
    L2 <= ATTN_REL for every (batch, q head) row.  Rows where the oracle is
    not finite (heads it was not asked for) are skipped.  Prints and returns
    (max-abs, worst per-row relative L2)."""
    g = np.asarray(got, np.float64).reshape(-1, np.shape(got)[-1])
    w = np.asarray(want, np.float64).reshape(-1, np.shape(want)[-1])
    keep = np.isfinite(w).all(axis=1)
    assert keep.any(), "no oracle rows to compare"
    g, w = g[keep], w[keep]
    assert np.isfinite(g).all(), "non-finite attention output"
    err = float(np.abs(g - w).max())
    rel = np.linalg.norm(g - w, axis=1) / np.maximum(np.linalg.norm(w, axis=1), 1e-30)
    worst = float(rel.max())
    print(f"  {what} attention: max-abs {err:.2e}, worst per-head rel-L2 {worst:.2e} "
          f"over {w.shape[0]} heads", flush=True)
    assert err <= ATTN_ABS, f"max-abs {err:.3e} > {ATTN_ABS}"
    assert worst <= ATTN_REL, f"per-head rel-L2 {worst:.3e} > {ATTN_REL} (row {int(rel.argmax())})"
    return err, worst
