"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and nothing else: it holds none of the
quantizer's arithmetic, and neither the oracle nor the HIP library imports
it.  Both sides are fed the *same bytes* produced here (on the host with
numpy, or on the device with torch and then copied back for the oracle).

The data model stands in for real LLaMA/Mistral KV caches, which are not
available: i.i.d. N(0,1) entries, plus, for keys only, a few high-variance
"outlier" channels per head -- the structure that the NSNQuant summary
(gist.science, plain-language part, "the fine print": early layers keep
high-variance outlier channels) says NSN has to cope with.

Outlier model (per sequence = one (batch, layer, head) of K):
  * 4 distinct channels chosen uniformly at random;
  * each gets a constant offset 10 * N(0, 4) (variance 4, i.e. std 2),
    drawn once per (sequence, channel) and held over all tokens;
  * with ``outlier_scale`` s, those channels' N(0,1) noise is multiplied by
    s before the offset is added (s = 5 for the full-size workloads, 1 for
    the tiny one).
Values V are plain N(0,1).  Queries are N(0,1).

Codebook training samples are N(0,1) float64 vectors from numpy's PCG64
with the given seed (the pages' k-means runs on torch.randn data; any
N(0,1) stream is the same method).
"""

import numpy as np

__all__ = [
    "WORKLOADS",
    "codebook_samples",
    "kv_numpy",
    "kv_torch",
    "query_numpy",
    "query_torch",
    "rht_signs",
]

HEAD_DIM = 128

# The five workloads, sizes only: tiny (fp32, G = 256: the oracle finishes it
# at once), one layer's K and V at 2 and at 1 bit, the decode-attention shape
# (batch 16, 32 query heads on 8 kv heads, 32768 quantized + 128 fp16
# residual tokens) and the full prefill (32 layers x batch 4 x 8 kv heads x
# 131072 tokens, K and V).
WORKLOADS = {
    "tiny": dict(n_seq=1, T=256, G=256, m=4, dtype="f32", outlier_scale=1.0,
                 cb_samples=65536, seed=1000),
    "layer2b": dict(n_seq=8, T=4096, G=128, m=4, dtype="f16", outlier_scale=5.0,
                    cb_samples=65536, seed=1001),
    "layer1b": dict(n_seq=8, T=4096, G=128, m=8, dtype="f16", outlier_scale=5.0,
                    cb_samples=262144, seed=1001),
    "decode": dict(B=16, Hq=32, Hkv=8, Nq=32768, R=128, G=128, m=4,
                   outlier_scale=5.0, cb_samples=65536, seed=1003),
    "prefill": dict(B=4, L=32, Hkv=8, T=131072, G=128, m=4, outlier_scale=5.0,
                    steps=512, cb_samples=65536, seed=1004),
}


def codebook_samples(m, n, seed=0):
    """n standard-normal m-vectors, float64, PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((n, m))


def kv_numpy(n_seq, T, outlier_scale, seed, d=HEAD_DIM, dtype=np.float16,
             n_outlier=4):
    """(K, V) of shape (n_seq, T, d) in ``dtype``; K carries the outlier
    channels, V is plain N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    K = rng.standard_normal((n_seq, T, d), dtype=np.float32)
    V = rng.standard_normal((n_seq, T, d), dtype=np.float32)
    for s in range(n_seq):
        ch = rng.choice(d, size=n_outlier, replace=False)
        off = 10.0 * rng.normal(0.0, 2.0, size=n_outlier)
        K[s][:, ch] = K[s][:, ch] * outlier_scale + off.astype(np.float32)
    return K.astype(dtype), V.astype(dtype)


def query_numpy(shape, seed, dtype=np.float16):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float32).astype(dtype)


def kv_torch(n_seq, T, outlier_scale, seed, device, d=HEAD_DIM, dtype=None,
             n_outlier=4, out_k=None, out_v=None):
    """Device-side generator with the same model (different stream from the
    numpy one; the oracle always reads back the device bytes).  Optionally
    fills caller-provided (n_seq, T, d) views ``out_k``/``out_v``."""
    import torch

    dtype = dtype or torch.float16
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    K = out_k if out_k is not None else torch.empty((n_seq, T, d), dtype=dtype, device=device)
    V = out_v if out_v is not None else torch.empty((n_seq, T, d), dtype=dtype, device=device)
    K.normal_(0.0, 1.0, generator=g)
    V.normal_(0.0, 1.0, generator=g)
    gc = torch.Generator(device="cpu")
    gc.manual_seed(seed)
    ch = torch.stack([torch.randperm(d, generator=gc)[:n_outlier] for _ in range(n_seq)])
    off = 10.0 * torch.normal(0.0, 2.0, size=(n_seq, n_outlier), generator=gc)
    ch = ch.to(device)
    off = off.to(device=device, dtype=torch.float32)
    idx = ch[:, None, :].expand(n_seq, T, n_outlier)
    cols = torch.gather(K, 2, idx).float() * outlier_scale + off[:, None, :]
    K.scatter_(2, idx, cols.to(dtype))
    return K, V


def query_torch(shape, seed, device, dtype=None):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=dtype or torch.float16)


def rht_signs(seed, d=HEAD_DIM):
    """d channel signs (+1.0 / -1.0, float64), each +-1 with probability 1/2,
    from PCG64(seed): the random diagonal of a randomized Hadamard rotation
    (drawn here and handed to both sides as an input)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.where(rng.integers(0, 2, size=d) == 1, -1.0, 1.0)
