"""Parity of nsn_tune_codebook (HIP, through the C ABI) with the oracle's
cosine fine-tuning (NSNQuant summary, Methodology §3, codebook
construction): float64 with every sum in the same fixed order on both
sides, so the tuned codebooks are compared bit for bit."""

import sys

import numpy as np
import pytest

import oracle
from tests.gpu_common import DEV, requires_gpu, torch
from tests.golden import load_codebook

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tune_gpu(H, C0, iters, lr):
    m = C0.shape[1]
    h = torch.from_numpy(np.ascontiguousarray(H, np.float64)).to(DEV)
    cb = torch.from_numpy(np.ascontiguousarray(C0, np.float32)).to(DEV)
    ws = torch.empty(nsnq.nsn_tune_codebook_workspace_size(m, H.shape[0]), dtype=torch.uint8,
                     device=DEV)
    nsnq.nsn_tune_codebook(h, cb, ws, iters, lr)
    torch.cuda.synchronize()
    return cb.cpu().numpy()


@pytest.mark.parametrize("m,n_vec,iters,lr", [
    (4, 256, 6, 3e-3),
    (8, 256, 6, 3e-3),
    (4, 300, 0, 1e-3),       # no step: the start rounded to fp16
    (4, 1, 4, 1e-2),         # one vector
    (4, 2048, 20, 3e-3),     # the 2-bit codebook's sample budget
])
def test_tune_bit_exact(m, n_vec, iters, lr):
    _say(f"tune m={m} n_vec={n_vec} iters={iters}")
    H = np.random.default_rng(100 + m + n_vec).standard_normal((n_vec, 128))
    C0 = load_codebook(m)
    got = tune_gpu(H, C0, iters, lr)
    want = oracle.cosine_tune(H, C0, iters, lr=lr)
    np.testing.assert_array_equal(got, want)
    if iters:
        assert np.abs(got - C0).max() > 0


def test_tune_zero_vectors_and_start_off_fp16():
    """All-zero vectors contribute nothing; a start codebook that is not
    fp16-representable is taken as given (float32) and rounded at the end."""
    rng = np.random.default_rng(5)
    H = rng.standard_normal((64, 128))
    H[3] = 0.0
    H[40] = 0.0
    C0 = (load_codebook(4).astype(np.float64) + rng.uniform(-1e-4, 1e-4, (256, 4))).astype(np.float32)
    got = tune_gpu(H, C0, 5, 5e-3)
    np.testing.assert_array_equal(got, oracle.cosine_tune(H, C0, 5, lr=5e-3))


@pytest.mark.parametrize("m,n_vec,iters,lr", [(4, 8192, 60, 2e-3), (8, 16384, 30, 1e-3)])
def test_tune_lowers_held_out_cosine_distance(m, n_vec, iters, lr):
    """What the fine-tuning is for: on fresh N(0,1) vectors the mean cosine
    distance after tuning is below that of the k-means start (measured by
    the oracle on the CPU)."""
    _say(f"tune held-out m={m} n_vec={n_vec} iters={iters}")
    H = np.random.default_rng(7 + m).standard_normal((n_vec, 128))
    C0 = load_codebook(m)
    got = tune_gpu(H, C0, iters, lr)
    Ht = np.random.default_rng(1234).standard_normal((2048, 128))
    before, after = oracle.cosine_loss(Ht, C0), oracle.cosine_loss(Ht, got)
    _say(f"  held-out mean cosine distance {before:.6f} -> {after:.6f}")
    assert after < before
