"""The exact nearest-codeword search (certified candidate tables for 4-d
sub-vectors, full scan for 8-d) against the oracle's brute force, through
nsn_nearest_codeword, including points on the grid's bin edges, far tails,
off-grid points and exact ties."""

import numpy as np
import pytest

import oracle
from tests.gpu_common import DEV, requires_gpu, table_for, torch
from tests.parity import TIE_REL

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]

EDGES_OFFSET = 17408   # byte offset of the float32 bin edges inside the table


def _nearest(p, table, V):
    v = torch.from_numpy(np.ascontiguousarray(V, dtype=np.float32)).to(DEV)
    out = torch.empty(len(V), dtype=torch.uint8, device=DEV)
    nsnq.nsn_nearest_codeword(p, table, v, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64)


def _check(V, got, C):
    V64 = np.asarray(V, np.float64)
    want = oracle.nearest_codeword(V64, C)
    bad = np.argwhere(got != want).ravel()
    C64 = np.asarray(C, np.float64)
    for i in bad:
        dg = float(np.sum((V64[i] - C64[got[i]]) ** 2))
        do = float(np.sum((V64[i] - C64[want[i]]) ** 2))
        assert dg - do <= TIE_REL * max(do, 1e-12), (i, V[i], got[i], want[i], dg, do)
    return len(bad)


def test_nearest_4d_random_and_adversarial():
    print("nearest 4-d", flush=True)
    p, table, C = table_for(4)
    rng = np.random.default_rng(0)
    parts = [rng.standard_normal((400000, 4)) * s for s in (1.0, 1.6)]
    edges = table.cpu().numpy()[EDGES_OFFSET:EDGES_OFFSET + 100].view(np.float32).astype(np.float64)
    # coordinates exactly on, and one float32 step around, every bin edge
    on = rng.choice(edges, size=(50000, 4))
    nudge = rng.choice([-1, 0, 1], size=on.shape)
    on32 = on.astype(np.float32)
    up = np.nextafter(on32, np.float32(np.inf))
    dn = np.nextafter(on32, np.float32(-np.inf))
    on = np.where(nudge > 0, up, np.where(nudge < 0, dn, on32)).astype(np.float64)
    mix = rng.standard_normal((50000, 4))
    mask = rng.random((50000, 4)) < 0.5
    mix[mask] = on[mask]
    parts += [on, mix]
    # tails and off-grid points (full scan path)
    tails = rng.standard_normal((20000, 4))
    tails[:, 0] = rng.uniform(3.5, 8.0, 20000) * rng.choice([-1, 1], 20000)
    parts.append(tails)
    # exact midpoints of codeword pairs (ties up to rounding)
    i, j = rng.integers(0, 256, 20000), rng.integers(0, 256, 20000)
    parts.append((C[i].astype(np.float64) + C[j]) / 2)
    parts.append(C.astype(np.float64))          # the codewords themselves
    V = np.concatenate(parts).astype(np.float32)
    got = _nearest(p, table, V)
    n_ties = _check(V, got, C)
    assert n_ties <= len(V) * 1e-3, n_ties
    # every codeword maps to itself (distance 0 is unique for distinct codewords)
    assert np.array_equal(got[-256:], np.arange(256))


def test_nearest_8d_full_scan():
    print("nearest 8-d", flush=True)
    p, table, C = table_for(8)
    rng = np.random.default_rng(1)
    V = np.concatenate([rng.standard_normal((100000, 8)), C.astype(np.float64)]).astype(np.float32)
    got = _nearest(p, table, V)
    _check(V, got, C)
    assert np.array_equal(got[-256:], np.arange(256))


def test_nearest_non_finite_does_not_fault():
    p, table, C = table_for(4)
    V = np.array([[np.nan, 0, 0, 0], [np.inf, 1, 1, 1], [-np.inf, 0, 0, 0], [1e30, 0, 0, 0]],
                 np.float32)
    got = _nearest(p, table, V)
    assert got.shape == (4,)
