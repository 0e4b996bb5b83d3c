"""Pins for the oracle's decode attention (NSNQuant summary, Methodology §4:
quantized part plus a full-precision residual; the score uses the NSN
byproducts directly)."""

import numpy as np
import pytest
import scipy.special

import oracle
import synth

D = 128


def _cache(B, Hkv, Nq, R, cb, G, seed):
    """Small cache built by the oracle's own quantizer (K with outliers)."""
    K, V = synth.kv_numpy(B * Hkv, Nq + R, 5.0, seed=seed)
    m = cb.shape[1]
    kc = np.zeros((B, Hkv, Nq, D // m), np.uint8)
    km = np.zeros((B, Hkv, Nq, 2), np.float16)
    ks = np.zeros((B, Hkv, max(Nq // G, 1), D), np.float16)
    vc, vm, vs = kc.copy(), km.copy(), ks.copy()
    for b in range(B):
        for h in range(Hkv):
            s = b * Hkv + h
            if Nq:
                kc[b, h], km[b, h], ks[b, h, :Nq // G] = oracle.quantize(K[s, :Nq], cb, G)
                vc[b, h], vm[b, h], vs[b, h, :Nq // G] = oracle.quantize(V[s, :Nq], cb, G)
    kr = K[:, Nq:].reshape(B, Hkv, R, D)
    vr = V[:, Nq:].reshape(B, Hkv, R, D)
    return (kc, km, ks), (vc, vm, vs), kr, vr


def test_matches_scipy_softmax_attention(cb2):
    B, Hq, Hkv, Nq, R, G = 2, 8, 2, 256, 16, 128
    kcache, vcache, kr, vr = _cache(B, Hkv, Nq, R, cb2, G, seed=21)
    q = synth.query_numpy((B, Hq, D), seed=22)
    scale = 1 / np.sqrt(D)
    out = oracle.decode_attention(q, kcache, vcache, kr, vr, cb2, G, Nq, R, scale)
    for b in range(B):
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            keys = np.concatenate([
                oracle.dequantize(kcache[0][b, kv], kcache[1][b, kv], kcache[2][b, kv], cb2, G),
                kr[b, kv].astype(np.float64)])
            vals = np.concatenate([
                oracle.dequantize(vcache[0][b, kv], vcache[1][b, kv], vcache[2][b, kv], cb2, G),
                vr[b, kv].astype(np.float64)])
            p = scipy.special.softmax(scale * keys @ q[b, h].astype(np.float64))
            np.testing.assert_allclose(out[b, h], p @ vals, rtol=1e-12, atol=1e-14)


def test_rotated_domain_identity(cb2):
    """Score with s1, s2', o' folded in and values summed in the rotated
    domain equals plain attention over the dequantized cache."""
    B, Hq, Hkv, Nq, R, G = 1, 8, 2, 384, 8, 128
    kcache, vcache, kr, vr = _cache(B, Hkv, Nq, R, cb2, G, seed=23)
    q = synth.query_numpy((B, Hq, D), seed=24)
    s = 1 / np.sqrt(D)
    a = oracle.decode_attention(q, kcache, vcache, kr, vr, cb2, G, Nq, R, s)
    b = oracle.decode_attention_rotated(q, kcache, vcache, kr, vr, cb2, G, Nq, R, s)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_zero_query_gives_mean_of_values(cb2):
    B, Hq, Hkv, Nq, R, G = 1, 4, 1, 256, 4, 128
    kcache, vcache, kr, vr = _cache(B, Hkv, Nq, R, cb2, G, seed=25)
    q = np.zeros((B, Hq, D), np.float16)
    out = oracle.decode_attention(q, kcache, vcache, kr, vr, cb2, G, Nq, R, 0.1)
    vals = np.concatenate([oracle.dequantize(*(a[0, 0] for a in vcache), cb2, G),
                           vr[0, 0].astype(np.float64)])
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], vals.mean(0), rtol=1e-12, atol=1e-14)


def test_no_quantized_tokens_is_plain_attention(cb2):
    R = 32
    rng = np.random.default_rng(0)
    kr = rng.standard_normal((1, 1, R, D)).astype(np.float16)
    vr = rng.standard_normal((1, 1, R, D)).astype(np.float16)
    q = rng.standard_normal((1, 2, D)).astype(np.float16)
    empty = (np.zeros((1, 1, 0, 32), np.uint8), np.zeros((1, 1, 0, 2), np.float16),
             np.zeros((1, 1, 0, D), np.float16))
    out = oracle.decode_attention(q, empty, empty, kr, vr, cb2, 128, 0, R, 0.09)
    for h in range(2):
        p = scipy.special.softmax(0.09 * kr[0, 0].astype(np.float64) @ q[0, h].astype(np.float64))
        np.testing.assert_allclose(out[0, h], p @ vr[0, 0].astype(np.float64), rtol=1e-12)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, D))
    v = rng.standard_normal((1, D))
    np.testing.assert_allclose(oracle.attend(rng.standard_normal(D), k, v, 1.0), v[0])


@pytest.mark.parametrize("shift", [0.0, 1000.0])
def test_softmax_is_shift_invariant(shift):
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((50, D))
    vals = rng.standard_normal((50, D))
    q = rng.standard_normal(D)
    # adding a constant along q to every key shifts every score equally
    k2 = keys + shift * q / (q @ q)
    np.testing.assert_allclose(oracle.attend(q, k2, vals, 1.0), oracle.attend(q, keys, vals, 1.0),
                               rtol=1e-9, atol=1e-12)
