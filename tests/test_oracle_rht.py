"""Pins for the oracle's randomized Hadamard rotation (the ``signs`` option).

[NSNQuant summary (gist.science), Methodology §2: the analysis pairs NSN with
the randomized Hadamard transform -- random channel sign flips followed by
the Hadamard matrix -- which guarantees channel variances close to 1.]

Each test checks the oracle against something other than itself: scipy's
Hadamard matrix, exact moments by enumeration of every sign vector, the
plain (already pinned) quantizer and attention under a change of variables.
"""

import itertools

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

D = 128


@pytest.fixture(scope="module")
def cb2():
    from tests.golden import load_codebook
    return load_codebook(4)


def test_rht_is_scipy_hadamard_times_sign_diagonal():
    """rht(u, s) = (H / sqrt(d)) diag(s) u with H from scipy (Sylvester)."""
    s = synth.rht_signs(3)
    assert set(np.unique(s)) == {-1.0, 1.0}
    rng = np.random.default_rng(2)
    u = rng.standard_normal((5, D))
    R = scipy.linalg.hadamard(D).astype(np.float64) @ np.diag(s) / np.sqrt(D)
    np.testing.assert_allclose(oracle.rht(u, s), u @ R.T, rtol=0, atol=1e-13)
    # orthonormal: R R^T = I, so norms are kept and rht_inverse undoes it
    Rm = oracle.rht(np.eye(D), s).T          # columns = images of the basis
    np.testing.assert_allclose(Rm @ Rm.T, np.eye(D), atol=1e-14)
    np.testing.assert_allclose(oracle.rht_inverse(oracle.rht(u, s), s), u, atol=1e-13)
    np.testing.assert_allclose(oracle.rht(oracle.rht_inverse(u, s), s), u, atol=1e-13)


def test_all_plus_signs_reduce_to_plain_rotation_and_bad_signs_are_rejected():
    rng = np.random.default_rng(4)
    u = rng.standard_normal((3, D))
    assert np.array_equal(oracle.rht(u, np.ones(D)), oracle.rotate(u))
    assert np.array_equal(oracle.rht(u, None), oracle.rotate(u))
    np.testing.assert_allclose(oracle.rht(u, -np.ones(D)), -oracle.rotate(u), atol=0)
    with pytest.raises(ValueError):
        oracle.rht(u, np.ones(D - 1))
    with pytest.raises(ValueError):
        oracle.rht(u, np.full(D, 0.5))


@pytest.mark.parametrize("d", [8, 16])
def test_exact_channel_moments_over_every_sign_vector(d):
    """For any fixed u, over all 2^d sign vectors every output channel has
    mean exactly 0 and second moment exactly ||u||^2 / d (the randomized
    transform's guarantee: unit variances once ||u|| = sqrt(d), as NSN
    makes it), while the plain transform of a spiky u is far from that."""
    rng = np.random.default_rng(d)
    u = rng.standard_normal(d)
    u[1] += 40.0                                   # two equal outlier channels:
    u[2] += 40.0                                   # H adds or cancels them
    u *= np.sqrt(d) / np.linalg.norm(u)            # NSN's token norm
    S = np.array(list(itertools.product((1.0, -1.0), repeat=d)))
    h = np.stack([oracle.rht(u, s) for s in S])    # (2^d, d)
    np.testing.assert_allclose(h.mean(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose((h * h).mean(axis=0), 1.0, atol=1e-12)
    hp = oracle.rotate(u)
    assert np.abs(hp * hp - 1.0).max() > 0.5


def test_channel_variances_near_one_on_outlier_keys():
    """NSN output of outlier-model keys (x5 noise on 4 channels of offset
    ~20): with a fresh sign draw per token, every channel's second moment is
    within sampling error of 1 (8192 samples: standard error ~0.016); the
    plain rotation of the same tokens is off by ~0.2 on some channel."""
    K, _ = synth.kv_numpy(1, 128, 5.0, seed=11)
    u = oracle.nsn(K[0].astype(np.float64), 128)[0]
    acc = np.zeros(D)
    n = 0
    for t in range(u.shape[0]):
        for r in range(64):
            h = oracle.rht(u[t], synth.rht_signs(100000 + 64 * t + r))
            acc += h * h
            n += 1
    assert np.abs(acc / n - 1.0).max() < 0.07, np.abs(acc / n - 1.0).max()
    hp = oracle.rotate(u)
    assert np.abs((hp * hp).mean(axis=0) - 1.0).max() > 0.15


def test_quantizer_is_sign_equivariant(cb2):
    """NSN commutes with flipping channel signs (norms, and group means up to
    the same flips), so quantizing x with signs s stores exactly the bytes
    the plain quantizer stores for s * x, and dequantizing with s returns s
    times the plain reconstruction.  A flip applied after H instead of
    before, or left out of the inverse, breaks this."""
    s = synth.rht_signs(7)
    K, V = synth.kv_numpy(2, 256, 5.0, seed=21, dtype=np.float64)
    for x in (K[0], V[1]):
        c, m, sh, it = oracle.quantize(x, cb2, 128, return_internals=True, signs=s)
        cp, mp, shp = oracle.quantize(x * s, cb2, 128)
        assert np.array_equal(c, cp) and np.array_equal(m, mp) and np.array_equal(sh, shp)
        xr = oracle.dequantize(c, m, sh, cb2, 128, signs=s)
        xp = oracle.dequantize(cp, mp, shp, cb2, 128)
        np.testing.assert_allclose(xr, s * xp, rtol=0, atol=1e-12)
        # and the quantizer differs from the plain one on x itself
        assert not np.array_equal(c, oracle.quantize(x, cb2, 128)[0])


def test_round_trip_exact_when_vq_is_lossless():
    """A codebook holding every sub-vector of h = R(s) u exactly gives
    alpha = 1 and an exact reconstruction through the inverse rotation."""
    G = 2
    s = synth.rht_signs(9)
    x = np.random.default_rng(9).standard_normal((2, D)) * 3.0
    u, s1, o, s2 = oracle.nsn(x, G)
    h = oracle.rht(u, s)
    C = np.concatenate([h.reshape(-1, 4), np.full((192, 4), 50.0)])
    codes, _, _, it = oracle.quantize(x, C, G, return_internals=True, signs=s)
    np.testing.assert_allclose(it["alpha"], 1.0, rtol=1e-13)
    xr = oracle.dequantize(codes, np.stack([s1, s2], axis=1), oracle.rht(o, s), C, G, signs=s)
    np.testing.assert_allclose(xr, x, rtol=1e-12, atol=1e-12)
    # the plain inverse does not undo the randomized rotation
    xw = oracle.dequantize(codes, np.stack([s1, s2], axis=1), oracle.rht(o, s), C, G)
    assert np.abs(xw - x).max() > 1e-3


def _cache(x, C, G, cap, signs):
    """(codes, meta, shift) of a (B, H, T, d) array, quantized per (b, h)."""
    B, H, T, d = x.shape
    m = C.shape[1]
    codes = np.zeros((B, H, cap, d // m), np.uint8)
    meta = np.zeros((B, H, cap, 2), np.float16)
    shift = np.zeros((B, H, cap // G, d), np.float16)
    for b in range(B):
        for h in range(H):
            c, mt, sh = oracle.quantize(x[b, h], C, G, signs=signs)
            codes[b, h, :T], meta[b, h, :T], shift[b, h, :T // G] = c, mt, sh
    return codes, meta, shift


def test_attention_with_signs_equals_flipped_plain_attention(cb2):
    """Attention over caches quantized with signs s equals s times the plain
    attention of s * q over caches of s * K, s * V (residuals flipped too),
    and the rotated-domain form agrees with the dequantizing one."""
    s = synth.rht_signs(13)
    G, T, R = 128, 256, 5
    B, Hq, Hkv = 1, 4, 2
    rng = np.random.default_rng(13)
    K = rng.standard_normal((B, Hkv, T, D)) * 2.0
    V = rng.standard_normal((B, Hkv, T, D))
    kr = rng.standard_normal((B, Hkv, 8, D)).astype(np.float16)
    vr = rng.standard_normal((B, Hkv, 8, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    kc, vc = _cache(K, cb2, G, T, s), _cache(V, cb2, G, T, s)
    scale = 1 / np.sqrt(D)
    out = oracle.decode_attention(q, kc, vc, kr, vr, cb2, G, T, R, scale, signs=s)
    rot = oracle.decode_attention_rotated(q, kc, vc, kr, vr, cb2, G, T, R, scale, signs=s)
    np.testing.assert_allclose(rot, out, rtol=0, atol=1e-12)
    kp, vp = _cache(K * s, cb2, G, T, None), _cache(V * s, cb2, G, T, None)
    q64 = q.astype(np.float64)
    plain = oracle.decode_attention(q64 * s, kp, vp, kr.astype(np.float64) * s,
                                    vr.astype(np.float64) * s, cb2, G, T, R, scale)
    np.testing.assert_allclose(out, plain * s, rtol=0, atol=1e-12)
