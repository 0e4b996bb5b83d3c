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

Attention: max-abs 2e-3 against the oracle on the same cache bytes.
"""

import numpy as np

import oracle

TIE_REL = 1e-5
RECON_REL = 1e-3
SAME_BYTES_REL = 1e-5
ATTN_ABS = 2e-3


def ulp16(v):
    """Spacing of fp16 at |v| (float64)."""
    v = np.abs(np.asarray(v, dtype=np.float16))
    return np.spacing(v).astype(np.float64)


def check_quantized_sequence(x, C, G, codes_g, meta_g, shift_g, scale_adjust=True):
    """Compare one sequence's GPU output to the oracle.  Returns a dict of
    statistics (number of accepted ties, ...).  Raises AssertionError."""
    C64 = np.asarray(C, np.float64)
    m = C64.shape[1]
    codes_o, meta_o, shift_o, it = oracle.quantize(x, C, G, scale_adjust_on=scale_adjust,
                                                   return_internals=True)
    T = x.shape[0]
    assert codes_g.shape == codes_o.shape, (codes_g.shape, codes_o.shape)
    h = it["h"].reshape(T, -1, m)
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
    # s1
    s1_o = it["s1"]
    s1_g = meta_g[:, 0].astype(np.float64)
    bad = np.abs(s1_g - s1_o.astype(np.float16).astype(np.float64)) > ulp16(s1_o) * 1.0001
    assert not bad.any(), f"s1 off by more than 1 ulp at tokens {np.argwhere(bad)[:5].ravel()}"
    # s2' with the GPU's codes
    hh = C64[codes_g.astype(np.int64)].reshape(T, -1)
    alpha = oracle.scale_adjust(it["h"], hh) if scale_adjust else np.ones(T)
    s2p = it["s2"] * alpha
    s2_g = meta_g[:, 1].astype(np.float64)
    bad = np.abs(s2_g - s2p.astype(np.float16).astype(np.float64)) > ulp16(s2p) * 1.0001
    assert not bad.any(), f"s2' off by more than 1 ulp at tokens {np.argwhere(bad)[:5].ravel()}"
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
