"""Codebook construction: Lloyd k-means on standard-normal samples.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[NSNQuant summary (gist.science), Methodology §3, codebook construction:
k-means over synthetic standard-normal data gives one global codebook, no
calibration set; README (DHdroid/NSNQuant), Overview and Codebook tuning.]

The samples are an *input* (the random draw is not part of this function):
callers pass N(0,1) vectors, shape (n, m).

Readings where the pages are silent:
  * initialisation = the first K samples;
  * one Lloyd iteration = assign every sample to its nearest centroid
    (exact-form squared distance, lowest index on ties), then replace each
    centroid by the mean of its members, accumulated in sample order; a
    centroid with no members keeps its value;
  * the final centroids are rounded to fp16-representable values (stored as
    float32), so that exact fp16 copies of the codebook exist;
  * the cosine-distance fine-tuning and the 2-bit ``--abs`` variant the
    pages mention are not part of this function.

Pins (tests/test_oracle_codebook.py): distortion non-increasing per
iteration; per-dimension MSE on fresh N(0,1) samples strictly inside
(Gaussian rate-distortion bound 2^(-2R), scalar Lloyd-Max MSE); centroid
condition after the last update; a 1-D two-cluster case against its closed
form; brute-force Python-loop Lloyd on a tiny set.
"""

import numpy as np

from .nsn import nearest_codeword, sq_dist_exact

__all__ = ["kmeans_codebook", "round_to_fp16", "lloyd_step", "distortion"]


def lloyd_step(samples, C):
    """One Lloyd iteration.  Returns (new centroids, labels, counts)."""
    K, m = C.shape
    labels = nearest_codeword(samples, C)
    counts = np.bincount(labels, minlength=K)
    newC = C.copy()
    for i in range(m):
        # bincount with weights adds samples[n, i] into bin labels[n] in
        # sample order: a plain sequential sum per centroid.
        sums = np.bincount(labels, weights=samples[:, i], minlength=K)
        nz = counts > 0
        newC[nz, i] = sums[nz] / counts[nz]
    return newC, labels, counts


def distortion(samples, C):
    """Mean squared distance of samples to their nearest centroid, per
    dimension."""
    labels = nearest_codeword(samples, C)
    d = sq_dist_exact(samples, C)[np.arange(samples.shape[0]), labels]
    return float(d.mean() / C.shape[1])


def kmeans_codebook(samples, n_codes=256, iters=20, return_history=False,
                    round_fp16=True):
    """Lloyd k-means codebook from N(0,1) samples (float64 throughout).

    samples: (n, m) float64, n >= n_codes.  Returns float32 (n_codes, m),
    rounded to fp16-representable values unless ``round_fp16`` is False
    (then float64).  With ``return_history`` also the per-iteration
    distortion measured before each update.
    """
    samples = np.asarray(samples, dtype=np.float64)
    n, m = samples.shape
    if n < n_codes:
        raise ValueError("need at least n_codes samples")
    C = samples[:n_codes].copy()
    hist = []
    for _ in range(iters):
        if return_history:
            hist.append(distortion(samples, C))
        C, _, _ = lloyd_step(samples, C)
    if return_history:
        hist.append(distortion(samples, C))
    out = round_to_fp16(C) if round_fp16 else C
    return (out, hist) if return_history else out


def round_to_fp16(C):
    """Round to the nearest fp16 value (ties to even), stored as float32."""
    return np.asarray(C, dtype=np.float64).astype(np.float16).astype(np.float32)
