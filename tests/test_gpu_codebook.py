"""nsn_build_codebook (HIP k-means in float64) reproduces the oracle's
codebooks bit for bit from the same N(0,1) samples."""

import numpy as np
import pytest

import oracle
import synth
from tests.golden import load_codebook
from tests.gpu_common import DEV, requires_gpu, torch

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def _build(X, iters):
    n, m = X.shape
    xs = torch.from_numpy(X).to(DEV)
    cb = torch.empty((256, m), dtype=torch.float32, device=DEV)
    ws = torch.empty(nsnq.nsn_build_codebook_workspace_size(m, n), dtype=torch.uint8, device=DEV)
    nsnq.nsn_build_codebook(xs, cb, ws, iters=iters)
    torch.cuda.synchronize()
    return cb.cpu().numpy()


@pytest.mark.parametrize("m,n", [(4, 65536), (8, 262144)])
def test_codebook_matches_golden(m, n):
    print(f"codebook m={m} n={n}", flush=True)
    X = synth.codebook_samples(m, n, seed=0)
    got = _build(X, 20)
    np.testing.assert_array_equal(got, load_codebook(m))


def test_codebook_small_matches_oracle_and_empty_clusters():
    """Few samples per code: some clusters go empty and keep their centroid."""
    X = synth.codebook_samples(4, 300, seed=3)
    X[256:] = X[0]  # duplicates of sample 0 pile into one cluster
    got = _build(X, 7)
    want = oracle.kmeans_codebook(X, 256, 7)
    np.testing.assert_array_equal(got, want)
