"""Pins for the oracle's k-means codebook (NSNQuant summary, Methodology §3,
codebook construction; README, Overview)."""

import numpy as np
import pytest

import oracle
import synth
from oracle.codebook import distortion, lloyd_step
from tests.golden import load_codebook


def test_lloyd_matches_python_loop_brute_force():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((40, 2))
    K, iters = 4, 6
    C = X[:K].copy()
    for _ in range(iters):
        lab = []
        for n in range(len(X)):
            best, bi = None, -1
            for k in range(K):
                dd = (X[n, 0] - C[k, 0]) ** 2 + (X[n, 1] - C[k, 1]) ** 2
                if best is None or dd < best:
                    best, bi = dd, k
            lab.append(bi)
        newC = C.copy()
        for k in range(K):
            mem = [n for n in range(len(X)) if lab[n] == k]
            if mem:
                for i in range(2):
                    s = 0.0
                    for n in mem:
                        s += X[n, i]
                    newC[k, i] = s / len(mem)
        C = newC
    got = oracle.kmeans_codebook(X, K, iters, round_fp16=False)
    np.testing.assert_array_equal(got, C)


def test_distortion_is_non_increasing():
    X = synth.codebook_samples(4, 8192, seed=3)
    _, hist = oracle.kmeans_codebook(X, 64, 12, return_history=True, round_fp16=False)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:])), hist
    assert hist[-1] < hist[0]


def test_two_level_scalar_case_converges_to_lloyd_max():
    """1-D, K=2 on N(0,1): the fixed point is +-sqrt(2/pi) (Lloyd-Max 1-bit)."""
    X = synth.codebook_samples(1, 200000, seed=5)
    X[0, 0], X[1, 0] = -1.0, 1.0  # start on both sides of zero
    C = np.sort(oracle.kmeans_codebook(X, 2, 30, round_fp16=False)[:, 0])
    np.testing.assert_allclose(C, [-np.sqrt(2 / np.pi), np.sqrt(2 / np.pi)], atol=6e-3)


def test_empty_cluster_keeps_its_centroid():
    X = np.array([[0.0, 0], [0.1, 0], [5.0, 5.0], [0.2, 0]])
    C0 = np.array([[0.0, 0], [100.0, 100.0]])
    C1, labels, counts = lloyd_step(np.concatenate([X]), C0)
    assert counts[1] == 0 and np.array_equal(C1[1], C0[1])


def test_centroid_condition_at_convergence():
    X = synth.codebook_samples(2, 4000, seed=8)
    C = oracle.kmeans_codebook(X, 16, 200, round_fp16=False)
    C2, labels, counts = lloyd_step(X, C)
    np.testing.assert_allclose(C2, C, rtol=0, atol=1e-12)
    for k in range(16):
        np.testing.assert_allclose(C[k], X[labels == k].mean(0), atol=1e-12)


def test_round_to_fp16_is_nearest_even():
    v = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 0.4528, -1.5104])
    r = oracle.round_to_fp16(v)
    assert r[0] == 1.0 and r[1] == 1.0 + 2 ** -9
    assert np.all(r.astype(np.float16).astype(np.float32) == r)


@pytest.mark.parametrize("m,lo,hi", [(4, 2.0 ** -4, 0.1175), (8, 2.0 ** -2, 1 - 2 / np.pi)])
def test_golden_codebook_mse_inside_rate_distortion_bracket(m, lo, hi):
    """Per-dimension MSE on fresh N(0,1) data lies strictly between the
    Gaussian rate-distortion bound 2^(-2R) (R = 8/m bits per dimension) and
    the scalar Lloyd-Max MSE at that rate (0.1175 at 2 bits, 1-2/pi at 1)."""
    C = load_codebook(m).astype(np.float64)
    assert C.shape == (256, m)
    X = synth.codebook_samples(m, 100000, seed=77)
    mse = distortion(X, C)
    assert lo < mse < hi, mse
    # entries are fp16-representable
    assert np.array_equal(C.astype(np.float16).astype(np.float64), C)


def test_golden_2bit_codebook_is_the_oracle_output():
    X = synth.codebook_samples(4, 65536, seed=0)
    C = oracle.kmeans_codebook(X, 256, 20)
    np.testing.assert_array_equal(C, load_codebook(4))
