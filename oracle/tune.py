"""Codebook fine-tuning for cosine distance -- numpy float64 reference.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[NSNQuant summary (gist.science), Methodology §3, codebook construction:
after k-means on synthetic standard-normal data the codebook is fine-tuned
to minimize the cosine distance between the original and the quantized
vectors, in minutes and without back-propagating through any model; the
authors' README, Codebook tuning.]

The pages give the objective only.  Readings:

  * Training vectors are an input: n full d-dimensional vectors (the
    NSN + Hadamard output is standard normal, so callers pass N(0,1)
    vectors of d = 128), each split into d/m contiguous sub-vectors as the
    quantizer splits a token.
  * The quantized vector h_hat is the concatenation of the nearest codewords
    (exact squared distance, lowest index on ties: the quantizer's own
    rule).  The objective is the mean over the n vectors of
    1 - cos(h, h_hat).  The assignment is piecewise constant in the
    codebook, so the gradient is taken with the assignment held fixed:
        dL/dc_k = -(1/n) sum over sub-vectors (i, j) assigned to k of
                  w_i (h_ij - r_i c_k),
    with w_i = 1 / sqrt(|h_i|^2 |h_hat_i|^2) and r_i = <h_i, h_hat_i> /
    |h_hat_i|^2 (w_i = r_i = 0 when a norm is zero).
  * Optimizer: Adam (Kingma and Ba, 2015: bias-corrected first and second
    moments, default beta1 = 0.9, beta2 = 0.999, eps = 1e-8) on the full
    batch, one step per iteration, learning rate a parameter; the moments
    start at zero and codewords with no members still move by their
    momentum, as in the published algorithm.
  * The start is the given codebook (a k-means result); the result is
    rounded to fp16-representable values like the k-means codebook.
  * The README's 2-bit ``--abs`` option is not described and is not
    implemented.

Every sum runs left to right in a fixed order (coordinates in index order;
gradient terms in sample order, sub-vectors of a vector consecutively), so
the result is reproducible bit for bit.

Pins (tests/test_oracle_tune.py): the gradient against central finite
differences of the loss written out directly; the first Adam step's closed
form (each coordinate moves by lr g / (|g| + eps) against its gradient's
sign); a codebook that reproduces the vectors exactly is a fixed point
(zero loss, zero gradient); the loss is invariant under rescaling the
vectors; fine-tuning lowers the mean cosine distance on fresh N(0,1)
vectors below the k-means start's.
"""

import numpy as np

from .codebook import round_to_fp16
from .nsn import nearest_codeword

__all__ = ["cosine_loss", "cosine_grad", "adam_step", "cosine_tune"]


def _seq_dot(a, b):
    """Row-wise dot products of (n, d) arrays, summed over d left to right."""
    acc = np.zeros(a.shape[0])
    for c in range(a.shape[1]):
        acc = acc + a[:, c] * b[:, c]
    return acc


def _stats(H, C, labels):
    """Per vector: the quantized vector, p = <h, h_hat>, a = |h|^2, b = |h_hat|^2."""
    n, d = H.shape
    Hq = C[labels].reshape(n, d)
    return Hq, _seq_dot(H, Hq), _seq_dot(H, H), _seq_dot(Hq, Hq)


def cosine_loss(H, C, labels=None):
    """Mean over vectors of 1 - cos(h, h_hat); h_hat from ``labels`` (the
    nearest codewords if None).  A vector with a zero norm counts 1."""
    H = np.asarray(H, np.float64)
    C = np.asarray(C, np.float64)
    m = C.shape[1]
    if labels is None:
        labels = nearest_codeword(H.reshape(-1, m), C)
    _, p, a, b = _stats(H, C, labels)
    ab = a * b
    cos = np.where(ab > 0, p / np.sqrt(np.where(ab > 0, ab, 1.0)), 0.0)
    return float(np.mean(1.0 - cos))


def cosine_grad(H, C, labels):
    """Gradient of cosine_loss with respect to C, the assignment held fixed."""
    H = np.asarray(H, np.float64)
    C = np.asarray(C, np.float64)
    n, d = H.shape
    K, m = C.shape
    _, p, a, b = _stats(H, C, labels)
    ab = a * b
    ok = ab > 0
    w = np.where(ok, 1.0 / np.sqrt(np.where(ok, ab, 1.0)), 0.0)
    r = np.where(ok, p / np.where(ok, b, 1.0), 0.0)
    X = H.reshape(-1, m)                      # sub-vectors in sample order
    wi = np.repeat(w, d // m)
    ri = np.repeat(r, d // m)
    G = np.zeros((K, m))
    for e in range(m):
        terms = (X[:, e] - ri * C[labels, e]) * wi
        # bincount adds the weights into their bins in index order: a plain
        # sequential sum per codeword
        G[:, e] = -np.bincount(labels, weights=terms, minlength=K) / n
    return G


def adam_step(C, G, mom, vel, t_b1, t_b2, lr, b1=0.9, b2=0.999, eps=1e-8):
    """One Adam update.  t_b1, t_b2 = b1^t, b2^t of this step.  Returns
    (C, mom, vel)."""
    mom = b1 * mom + (1.0 - b1) * G
    vel = b2 * vel + (1.0 - b2) * (G * G)
    mhat = mom / (1.0 - t_b1)
    vhat = vel / (1.0 - t_b2)
    C = C - lr * mhat / (np.sqrt(vhat) + eps)
    return C, mom, vel


def cosine_tune(H, C0, iters, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, return_history=False,
                round_fp16=True):
    """Fine-tune codebook C0 (K, m) on vectors H (n, d) for ``iters`` full-batch
    Adam steps on the mean cosine distance.  Returns float32 (K, m) rounded to
    fp16-representable values (float64 unrounded if ``round_fp16`` is False);
    with ``return_history`` also the loss before each step and at the end."""
    H = np.asarray(H, np.float64)
    C = np.asarray(C0, np.float64).copy()
    m = C.shape[1]
    mom = np.zeros_like(C)
    vel = np.zeros_like(C)
    t_b1 = t_b2 = 1.0
    hist = []
    for _ in range(iters):
        labels = nearest_codeword(H.reshape(-1, m), C)
        if return_history:
            hist.append(cosine_loss(H, C, labels))
        G = cosine_grad(H, C, labels)
        t_b1 = t_b1 * b1
        t_b2 = t_b2 * b2
        C, mom, vel = adam_step(C, G, mom, vel, t_b1, t_b2, lr, b1, b2, eps)
    if return_history:
        hist.append(cosine_loss(H, C))
    out = round_to_fp16(C) if round_fp16 else C
    return (out, hist) if return_history else out
