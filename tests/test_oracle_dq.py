"""Pins for the oracle's double quantization of the NSN byproducts and of
the codebook (NSNQuant summary, Methodology §3, Double Quantization: s1, o
and the codebook entries at 4 bits)."""

import numpy as np
import pytest

import oracle
from oracle import dq


def test_record_size_and_nibble_packing():
    assert oracle.record_bytes(128) == 136 and oracle.record_bytes(256) == 200
    v = np.random.default_rng(1).integers(0, 16, 128).astype(np.uint8)
    np.testing.assert_array_equal(dq._unpack_nibbles(dq._pack_nibbles(v), 128), v)
    assert dq._pack_nibbles(np.array([3, 12], np.uint8))[0] == 3 + 16 * 12


def test_values_on_the_grids_round_trip_exactly():
    rng = np.random.default_rng(2)
    k = rng.integers(0, 16, 128)
    k[0], k[1] = 0, 15                                   # both end points present
    s1 = 1.0 + 0.125 * k                                 # lo 1, hi 2.875: step 1/8, fp16-exact
    q = rng.integers(-7, 8, 128)
    q[5] = 7
    o = 0.25 * q                                         # max |o| / 7 = 0.25 exactly
    s1d, od = oracle.dq_decode_group(oracle.dq_encode_group(s1, o), 128)
    np.testing.assert_array_equal(s1d, s1)
    np.testing.assert_array_equal(od, o)


def test_error_bounds_off_the_grid():
    rng = np.random.default_rng(3)
    for _ in range(20):
        s1 = rng.uniform(0.3, 4.0, 128)
        o = rng.standard_normal(128) * 0.3
        rec = oracle.dq_encode_group(s1, o)
        s1d, od = oracle.dq_decode_group(rec, 128)
        lo, hi, sc = rec[:6].view(np.float16).astype(np.float64)
        slack = max(abs(lo - s1.min()), abs(hi - s1.max()))
        assert np.abs(s1d - s1).max() <= (hi - lo) / 30 + slack + 1e-12
        assert s1d.min() >= lo - 1e-15 and s1d.max() <= hi + 1e-15
        # o: half a step, except beyond +-7 steps when the fp16 scale rounded down
        over = max(0.0, np.abs(o).max() - 7 * sc)
        assert np.abs(od - o).max() <= sc / 2 + over + 1e-12


def test_sign_symmetry_and_degenerate_groups():
    rng = np.random.default_rng(4)
    o = rng.standard_normal(128)
    s1 = rng.uniform(1, 2, 128)
    _, a = oracle.dq_decode_group(oracle.dq_encode_group(s1, o), 128)
    _, b = oracle.dq_decode_group(oracle.dq_encode_group(s1, -o), 128)
    np.testing.assert_array_equal(a, -b)
    s1d, od = oracle.dq_decode_group(oracle.dq_encode_group(np.full(128, 1.5), np.zeros(128)), 128)
    assert np.all(s1d == 1.5) and np.all(od == 0)


def test_pack_unpack_of_a_quantized_sequence(cb2):
    x = np.random.default_rng(5).standard_normal((256, 128))
    codes, meta, shift, it = oracle.quantize(x, cb2, 128, return_internals=True)
    s2, recs = oracle.dq_pack(meta, shift, it["s1"], it["o_rot"], 128)
    assert recs.shape == (2, 136) and s2.dtype == np.float16
    m2, sh2 = oracle.dq_unpack(s2, recs, 128)
    np.testing.assert_array_equal(m2[:, 1], meta[:, 1].astype(np.float64))
    # the decoded metadata stays close to the fp16 one: s1 within half a
    # step of its group's range, o' within half a scale step
    for g in range(2):
        lo, hi, sc = recs[g, :6].view(np.float16).astype(np.float64)
        sl = slice(128 * g, 128 * g + 128)
        assert np.abs(m2[sl, 0] - it["s1"][sl]).max() <= (hi - lo) / 30 + 2e-3 * hi
        assert np.abs(sh2[g] - it["o_rot"][g]).max() <= sc / 2 + 1e-3


def test_codebook_levels_nearest_and_ties():
    rng = np.random.default_rng(6)
    C = rng.standard_normal((256, 4)) * 1.2
    C4 = oracle.codebook_4bit(C)
    assert set(np.unique(C4)).issubset(set(dq.CB_LEVELS.astype(np.float32)))
    d_got = np.abs(C - C4)
    d_best = np.abs(C[..., None] - dq.CB_LEVELS).min(-1)
    np.testing.assert_allclose(d_got, d_best, atol=1e-12)
    ties = np.array([0.0, 0.375, -0.375, 0.75, 2.625, -2.625, 5.0, -5.0])
    np.testing.assert_array_equal(oracle.codebook_4bit(ties),
                                  np.array([0.1875, 0.1875, -0.1875, 0.5625, 2.4375, -2.4375,
                                            2.8125, -2.8125], np.float32))
    assert np.all(np.float16(dq.CB_LEVELS) == dq.CB_LEVELS)   # exact in fp16
