"""NSN transform, Hadamard rotation, nearest-codeword VQ, scale adjustment,
quantize and dequantize -- numpy float64 reference.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation follows the NSNQuant technical summary (gist.science), Methodology:
a KV tensor ``v`` of shape (l, d) per head; byproducts ``s1, o, s2``.

Readings taken where the pages leave a step open (each is listed in the
design notes too):
  * ``s1``/``s2`` are the multipliers that restore the token
    (``x = s1 * y``), i.e. ``s = ||x|| / sqrt(d)``.  A zero-norm token maps
    to ``y = 0`` (so it reconstructs to exactly 0).
  * The channel mean of the Shift step runs over groups of ``G`` contiguous
    tokens of one sequence (one (batch, layer, head) of K or of V).
  * The "naive" Hadamard transform is the Sylvester matrix in natural order
    with orthonormal scaling ``H / sqrt(d)``; no random signs by default.
  * Randomized variant (``signs``): the rotation becomes ``H D / sqrt(d)``
    with ``D = diag(signs)``, one +-1 per channel, the flips applied before
    the transform.  The pages name the randomized transform without fixing
    how its signs are drawn or shared; reading: one sign vector for the
    whole cache, drawn by the caller and passed in (so both sides of a test
    take the same draw).  Dequantization applies the inverse ``D H / sqrt(d)``.
  * Sub-vector ``j`` of a token is the contiguous slice ``h[m*j : m*j+m]``.
  * Nearest codeword = argmin of the exact squared distance; ties go to the
    lowest index.
  * Scale adjustment is per token: ``alpha = ||h||^2 / <h, h_hat>`` so that
    the component of ``alpha * h_hat`` along ``h`` equals ``h``; it is folded
    into the stored second scale ``s2' = s2 * alpha``.  If
    ``<h, h_hat> <= 0`` then ``alpha = 1``.
  * Storage: codes uint8, metadata fp16 ``(s1, s2')`` per token, and the
    group mean stored already rotated (``o' = H o / sqrt(d)``) in fp16.
    All forward arithmetic uses unrounded values; only storage rounds.

Pins (tests/test_oracle_*.py): H H^T = d I and equality with
scipy.linalg.hadamard; norms after each Normalize; zero channel means after
Shift; scale invariance and permutation equivariance of NSN; commutation of
NSN with the rotation; moments of NSN+H output approaching N(0,1);
brute-force nearest codeword by explicit Python loops; product codebooks
reducing to the scalar Lloyd-Max quantizer; exact ties built from binary
fractions; the scale-adjust identity; exact round trip with VQ bypassed.
Randomized variant (tests/test_oracle_rht.py): equality with
scipy.linalg.hadamard times the sign diagonal, orthonormality, all-plus signs
reducing to the plain rotation, the exact first two moments of every output
channel over all 2^d sign vectors at small d, channel-sign equivariance of
the whole quantizer, and near-unit channel variances on outlier inputs.
"""

import numpy as np

__all__ = [
    "hadamard_matrix",
    "rotate",
    "rht",
    "rht_inverse",
    "normalize_tokens",
    "shift_channels",
    "nsn",
    "sq_dist_exact",
    "nearest_codeword",
    "scale_adjust",
    "quantize",
    "dequantize",
]


def hadamard_matrix(d):
    """Sylvester Hadamard matrix of order d (power of two), natural order.

    H_1 = [1];  H_2n = [[H_n, H_n], [H_n, -H_n]].
    [NSNQuant summary, Methodology §2: the implementation uses the plain
    (non-randomized) Hadamard transform.]
    """
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def rotate(u):
    """Orthonormal Hadamard rotation of the last axis: u @ (H / sqrt(d))^T.

    H is symmetric, so this is also its own inverse.
    [NSNQuant summary, Methodology §2; README Overview: the Hadamard
    transform makes the KV distribution Gaussian-like.]
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    H = hadamard_matrix(d)
    return u @ H.T / np.sqrt(d)


def _sign_vector(signs, d):
    s = np.asarray(signs, dtype=np.float64)
    if s.shape != (d,) or not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be d values of +1 or -1")
    return s


def rht(u, signs=None):
    """Randomized Hadamard rotation of the last axis: (H / sqrt(d)) D u with
    D = diag(signs); ``signs=None`` is the plain rotation.

    [NSNQuant summary, Methodology §2: the analysis pairs NSN with the
    randomized Hadamard transform -- random sign flips of the channels, then
    the Hadamard matrix -- whose guarantee is that channel variances come out
    close to 1; the implementation keeps the plain transform.]
    """
    u = np.asarray(u, dtype=np.float64)
    if signs is None:
        return rotate(u)
    return rotate(u * _sign_vector(signs, u.shape[-1]))


def rht_inverse(h, signs=None):
    """Inverse of ``rht``: D (H / sqrt(d)) h  (H symmetric with H H = d I,
    D D = I)."""
    r = rotate(h)
    if signs is None:
        return r
    return r * _sign_vector(signs, r.shape[-1])


def normalize_tokens(x):
    """Token-wise normalize to L2 norm sqrt(d).

    Returns (y, s) with s = ||x|| / sqrt(d) and x = s * y.  Zero tokens give
    y = 0, s = 0.
    [NSNQuant summary, Methodology §1, first and third steps.]
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    s = np.sqrt(np.sum(x * x, axis=-1)) / np.sqrt(d)
    safe = np.where(s > 0, s, 1.0)
    y = np.where((s > 0)[..., None], x / safe[..., None], 0.0)
    return y, s


def shift_channels(y, G):
    """Channel-wise centering over groups of G contiguous tokens.

    y: (T, d) with T % G == 0.  Returns (z, o) with o of shape (T/G, d), the
    per-group per-channel mean, and z = y - o[group].
    [NSNQuant summary, Methodology §1, Shift step.]
    """
    y = np.asarray(y, dtype=np.float64)
    T, d = y.shape
    if T % G:
        raise ValueError("token count must be a multiple of the group size")
    yg = y.reshape(T // G, G, d)
    o = yg.mean(axis=1)
    z = (yg - o[:, None, :]).reshape(T, d)
    return z, o


def nsn(x, G):
    """Normalize-Shift-Normalize of one sequence x (T, d).

    Returns (u, s1, o, s2): u has every token at norm sqrt(d); the
    byproducts reconstruct x as x = s1 * (s2 * u + o[group]).
    [NSNQuant summary, Methodology §1.]
    """
    y, s1 = normalize_tokens(x)
    z, o = shift_channels(y, G)
    u, s2 = normalize_tokens(z)
    return u, s1, o, s2


def sq_dist_exact(v, C):
    """Exact-form squared distances ||v - C_k||^2, summed over the sub-vector
    dimension left to right (each square rounded, then added).

    v: (..., m), C: (K, m) -> (..., K), float64.
    """
    v = np.asarray(v, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    m = C.shape[1]
    acc = None
    for i in range(m):
        t = v[..., i, None] - C[:, i]
        sq = t * t
        acc = sq if acc is None else acc + sq
    return acc


def nearest_codeword(v, C, chunk=512):
    """Index of the nearest codeword of every sub-vector (ties: lowest index).

    v: (N, m) float64, C: (K, m).  Returns int64 (N,).
    [NSNQuant summary, Methodology §3: each rotated sub-vector is replaced by
    its codeword in one global codebook.]
    """
    v = np.asarray(v, dtype=np.float64).reshape(-1, np.shape(C)[1])
    out = np.empty(v.shape[0], dtype=np.int64)
    for a in range(0, v.shape[0], chunk):
        # numpy's argmin returns the first (lowest) index among equal minima
        out[a:a + chunk] = np.argmin(sq_dist_exact(v[a:a + chunk], C), axis=1)
    return out


def scale_adjust(h, h_hat):
    """Per-token scale that keeps the component of the quantized vector
    parallel to the original: alpha = ||h||^2 / <h, h_hat>  (1 if <= 0).

    h, h_hat: (T, d).  Returns alpha (T,).
    [NSNQuant summary, Methodology §3, scale adjustment.  Reading: per token,
    folded into the stored s2.]
    """
    h = np.asarray(h, dtype=np.float64)
    h_hat = np.asarray(h_hat, dtype=np.float64)
    num = np.sum(h * h, axis=-1)
    den = np.sum(h * h_hat, axis=-1)
    safe = np.where(den > 0, den, 1.0)
    return np.where(den > 0, num / safe, 1.0)


def quantize(x, C, G, scale_adjust_on=True, return_internals=False, signs=None):
    """Quantize one sequence x (T, d) against codebook C (K, m).

    Steps in the pages' order: Normalize, Shift, Normalize (NSN), Hadamard
    rotation (randomized by ``signs`` when given), nearest codeword per
    sub-vector, scale adjustment.

    Returns (codes uint8 (T, d/m), meta fp16 (T, 2) = (s1, s2'),
    shift fp16 (T/G, d) = rotated group mean o').  With
    ``return_internals`` also a dict of the float64 intermediates.
    """
    x = np.asarray(x, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    T, d = x.shape
    K, m = C.shape
    if K > 256:
        raise ValueError("codes are stored in one byte")
    u, s1, o, s2 = nsn(x, G)
    h = rht(u, signs)
    codes = nearest_codeword(h.reshape(-1, m), C).reshape(T, d // m)
    h_hat = C[codes].reshape(T, d)
    alpha = scale_adjust(h, h_hat) if scale_adjust_on else np.ones(T)
    s2p = s2 * alpha
    meta = np.stack([s1, s2p], axis=-1).astype(np.float16)
    o_rot = rht(o, signs)
    shift = o_rot.astype(np.float16)
    out = (codes.astype(np.uint8), meta, shift)
    if return_internals:
        return out + (dict(u=u, s1=s1, o=o, s2=s2, h=h, h_hat=h_hat,
                           alpha=alpha, s2p=s2p, o_rot=o_rot),)
    return out


def dequantize(codes, meta, shift, C, G, signs=None):
    """Reconstruct one sequence from codes and stored fp16 byproducts.

    x_hat_t = (H / sqrt(d)) [ s1_t (s2'_t h_hat_t + o'_g) ], the stored fp16
    numbers taken as exact values; with ``signs`` the inverse rotation is
    D (H / sqrt(d)).
    [NSNQuant summary, Methodology §1 (byproducts reconstruct the tensor) and
    §4 (dequantization kernels).]
    """
    codes = np.asarray(codes)
    C = np.asarray(C, dtype=np.float64)
    T, nsub = codes.shape
    m = C.shape[1]
    d = nsub * m
    meta = np.asarray(meta).astype(np.float64)
    shift = np.asarray(shift).astype(np.float64)
    h_hat = C[codes.astype(np.int64)].reshape(T, d)
    s1 = meta[:, 0:1]
    s2p = meta[:, 1:2]
    o_rot = np.repeat(shift, G, axis=0)[:T]
    return rht_inverse(s1 * (s2p * h_hat + o_rot), signs)
