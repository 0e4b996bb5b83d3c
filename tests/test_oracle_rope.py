"""Pins for the oracle's decode attention over keys stored before rotary
position embedding (NSNQuant summary, Methodology §4: for keys, NSN comes
before RoPE).  The RoPE form is the rotate-half reading: channel pair
(i, i + 64) turns by the angle pos * base^(-i/64)."""

import math

import numpy as np
import pytest
import scipy.special

import oracle
from tests.test_oracle_attention import _cache

D = 128


def _unit(i):
    e = np.zeros(D)
    e[i] = 1.0
    return e


def _freq(i, base):
    # written out independently of the oracle: base to the power -2i/d, d = 128
    return math.pow(base, -i / 64.0)


@pytest.mark.parametrize("base", [10000.0, 500000.0])
@pytest.mark.parametrize("i", [0, 5, 37, 63])
def test_pair_rotation_closed_forms(i, base):
    th = _freq(i, base)
    for p in (0, 1, 7, 1000, 32895):
        ang = p * th
        a = oracle.apply_rope(_unit(i), p, base)
        b = oracle.apply_rope(_unit(i + 64), p, base)
        want_a = np.zeros(D)
        want_a[i], want_a[i + 64] = math.cos(ang), math.sin(ang)
        want_b = np.zeros(D)
        want_b[i], want_b[i + 64] = -math.sin(ang), math.cos(ang)
        np.testing.assert_allclose(a, want_a, atol=1e-12)
        np.testing.assert_allclose(b, want_b, atol=1e-12)
    # scores depend on the position difference only, with the sign of the
    # rotation fixed by the sin term
    for p, pp in ((5, 2), (2, 5), (40000, 123)):
        s = oracle.apply_rope(_unit(i), p, base) @ oracle.apply_rope(_unit(i + 64), pp, base)
        c = oracle.apply_rope(_unit(i), p, base) @ oracle.apply_rope(_unit(i), pp, base)
        assert s == pytest.approx(math.sin((p - pp) * th), abs=1e-10)
        assert c == pytest.approx(math.cos((p - pp) * th), abs=1e-10)


def test_rotation_keeps_norm_and_composes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, D))
    for p in (0, 3, 777, 123456):
        y = oracle.apply_rope(x, p, 10000.0)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    np.testing.assert_allclose(
        oracle.apply_rope(oracle.apply_rope(x, 300, 10000.0), 45, 10000.0),
        oracle.apply_rope(x, 345, 10000.0), atol=1e-10)
    np.testing.assert_array_equal(oracle.apply_rope(x, 0, 10000.0), x)


def _rotation_matrix(p, base):
    """The same rotation as an explicit block matrix (pairs (i, i + 64))."""
    R = np.zeros((D, D))
    for i in range(64):
        a = p * _freq(i, base)
        R[i, i], R[i, i + 64] = math.cos(a), -math.sin(a)
        R[i + 64, i], R[i + 64, i + 64] = math.sin(a), math.cos(a)
    return R


def test_matches_explicit_rotation_matrices(cb2):
    B, Hq, Hkv, Nq, R, G = 1, 4, 1, 256, 9, 128
    kcache, vcache, kr, vr = _cache(B, Hkv, Nq, R, cb2, G, seed=41)
    q = np.random.default_rng(42).standard_normal((B, Hq, D))
    scale, base, q_pos = 1 / math.sqrt(D), 10000.0, Nq + R + 3
    got = oracle.decode_attention_rope(q, kcache, vcache, kr, vr, cb2, G, Nq, R, scale, q_pos, base)
    keys = np.concatenate([oracle.dequantize(*(a[0, 0][:n] for a, n in zip(kcache, (Nq, Nq, Nq // G))),
                                             cb2, G), kr[0, 0].astype(np.float64)])
    vals = np.concatenate([oracle.dequantize(*(a[0, 0][:n] for a, n in zip(vcache, (Nq, Nq, Nq // G))),
                                             cb2, G), vr[0, 0].astype(np.float64)])
    krot = np.stack([_rotation_matrix(t, base) @ keys[t] for t in range(keys.shape[0])])
    for h in range(Hq):
        qrot = _rotation_matrix(q_pos, base) @ q[0, h]
        p = scipy.special.softmax(scale * (krot @ qrot))
        np.testing.assert_allclose(got[0, h], p @ vals, rtol=1e-10, atol=1e-12)


def test_common_position_shift_leaves_output_unchanged():
    rng = np.random.default_rng(5)
    q, K, V = rng.standard_normal(D), rng.standard_normal((40, D)), rng.standard_normal((40, D))
    pos = np.arange(40) * 3
    a = oracle.attention.attend_rope(q, K, V, 0.1, 200, pos, 10000.0)
    b = oracle.attention.attend_rope(q, K, V, 0.1, 200 + 9999, pos + 9999, 10000.0)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)


def test_zero_positions_reduce_to_plain_attention():
    rng = np.random.default_rng(6)
    q, K, V = rng.standard_normal(D), rng.standard_normal((30, D)), rng.standard_normal((30, D))
    np.testing.assert_allclose(oracle.attention.attend_rope(q, K, V, 0.2, 0, np.zeros(30), 10000.0),
                               oracle.attend(q, K, V, 0.2), rtol=1e-12)


def test_single_residual_key_returns_its_value():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, D))
    kr = rng.standard_normal((1, 1, 1, D)).astype(np.float16)
    vr = rng.standard_normal((1, 1, 1, D)).astype(np.float16)
    empty = (np.zeros((1, 1, 0, 32), np.uint8), np.zeros((1, 1, 0, 2), np.float16),
             np.zeros((1, 1, 0, D), np.float16))
    out = oracle.decode_attention_rope(q, empty, empty, kr, vr, np.zeros((256, 4)), 128, 0, 1,
                                       0.1, 77, 10000.0)
    np.testing.assert_allclose(out[0], np.repeat(vr[0, 0].astype(np.float64), 2, axis=0), rtol=1e-12)
