"""Pins for the oracle's codebook fine-tuning on cosine distance (NSNQuant
summary, Methodology §3, codebook construction: after k-means the codebook
is fine-tuned to minimize the cosine distance between original and
quantized vectors)."""

import numpy as np
import pytest

import oracle
from oracle import tune
from tests.golden import load_codebook


def _direct_loss(H, C, labels):
    """1 - cos(h, h_hat) averaged over rows, written with library norms."""
    n, d = H.shape
    Hq = C[labels].reshape(n, d)
    cos = np.einsum("ij,ij->i", H, Hq) / (np.linalg.norm(H, axis=1) * np.linalg.norm(Hq, axis=1))
    return float(np.mean(1.0 - cos))


def _small(seed, n=6, d=16, m=4, K=8):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((n, d))
    C = rng.standard_normal((K, m))
    labels = oracle.nearest_codeword(H.reshape(-1, m), C)
    return H, C, labels


@pytest.mark.parametrize("seed,m", [(1, 4), (2, 4), (3, 8)])
def test_gradient_matches_central_differences(seed, m):
    """With the assignment held fixed, the loss is smooth in the codebook:
    the analytic gradient equals central differences of the loss written
    out directly."""
    H, C, labels = _small(seed, m=m, d=32)
    G = tune.cosine_grad(H, C, labels)
    eps = 1e-6
    num = np.zeros_like(C)
    for k in range(C.shape[0]):
        for e in range(C.shape[1]):
            Cp, Cm = C.copy(), C.copy()
            Cp[k, e] += eps
            Cm[k, e] -= eps
            num[k, e] = (_direct_loss(H, Cp, labels) - _direct_loss(H, Cm, labels)) / (2 * eps)
    np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-10)
    used = np.unique(labels)
    assert np.abs(G[used]).max() > 1e-4                   # not trivially zero
    unused = np.setdiff1d(np.arange(C.shape[0]), used)
    assert np.all(G[unused] == 0)


def test_loss_matches_direct_definition_and_is_scale_invariant():
    H, C, labels = _small(4, n=20, d=32)
    L = tune.cosine_loss(H, C, labels)
    assert L == pytest.approx(_direct_loss(H, C, labels), rel=1e-13)
    rng = np.random.default_rng(5)
    s = rng.uniform(0.1, 10.0, (H.shape[0], 1))
    assert tune.cosine_loss(s * H, C, labels) == pytest.approx(L, rel=1e-13)
    # a global rescale of the codebook leaves the loss unchanged too (for the
    # same assignment)
    assert tune.cosine_loss(H, 2.5 * C, labels) == pytest.approx(L, rel=1e-13)


def test_adam_closed_form_under_a_constant_gradient():
    """Bias correction makes the moments exact for a constant gradient: every
    step moves each coordinate by lr g / (|g| + eps) against the gradient."""
    rng = np.random.default_rng(6)
    C = rng.standard_normal((8, 4))
    G = rng.standard_normal((8, 4)) * 1e-3
    G[0, 0] = 0.0
    mom = np.zeros_like(C)
    vel = np.zeros_like(C)
    b1t = b2t = 1.0
    X = C.copy()
    lr = 0.01
    for t in range(5):
        b1t *= 0.9
        b2t *= 0.999
        X, mom, vel = tune.adam_step(X, G, mom, vel, b1t, b2t, lr)
    step = lr * G / (np.abs(G) + 1e-8)
    np.testing.assert_allclose(X - C, -5 * step, rtol=1e-10, atol=1e-15)
    assert X[0, 0] == C[0, 0]


def test_first_tuning_step_closed_form():
    H, C, _ = _small(7, n=12, d=32)
    labels = oracle.nearest_codeword(H.reshape(-1, 4), C)
    G = tune.cosine_grad(H, C, labels)
    lr = 0.02
    C1 = tune.cosine_tune(H, C, 1, lr=lr, round_fp16=False)
    np.testing.assert_allclose(C1 - C, -lr * G / (np.abs(G) + 1e-8), rtol=1e-9, atol=1e-15)


def test_exact_codebook_is_a_fixed_point():
    """Vectors made of codewords: the loss is 0, the gradient exactly 0, and
    Adam leaves every codeword where it is."""
    rng = np.random.default_rng(8)
    C = rng.standard_normal((8, 4))
    idx = rng.integers(0, 8, (10, 8))
    H = C[idx].reshape(10, 32)
    labels = oracle.nearest_codeword(H.reshape(-1, 4), C)
    assert np.array_equal(labels, idx.ravel())
    assert tune.cosine_loss(H, C) == pytest.approx(0.0, abs=1e-15)
    assert np.all(tune.cosine_grad(H, C, labels) == 0)
    np.testing.assert_array_equal(tune.cosine_tune(H, C, 3, lr=0.1, round_fp16=False), C)


def test_zero_vector_contributes_nothing():
    H, C, _ = _small(9, n=5, d=32)
    H[2] = 0.0
    labels = oracle.nearest_codeword(H.reshape(-1, 4), C)
    G = tune.cosine_grad(H, C, labels)
    G_without = tune.cosine_grad(np.delete(H, 2, axis=0), C,
                                 np.delete(labels.reshape(5, 8), 2, axis=0).ravel())
    np.testing.assert_allclose(G * 5 / 4, G_without, rtol=1e-12, atol=1e-18)


def test_tuning_lowers_the_training_loss_and_rounds_to_fp16():
    C = load_codebook(4).astype(np.float64)
    H = np.random.default_rng(11).standard_normal((512, 128))
    Cf, hist = tune.cosine_tune(H, C, 25, lr=3e-3, return_history=True)
    assert hist[-1] < hist[0] - 1e-3, hist
    assert Cf.dtype == np.float32
    np.testing.assert_array_equal(Cf, Cf.astype(np.float16).astype(np.float32))
    assert np.abs(Cf - C).max() > 1e-3
