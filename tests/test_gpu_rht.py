"""Parity of the randomized Hadamard rotation (NSN_RHT; NSNQuant summary,
Methodology §2) with the oracle run on the same channel signs, through the C
ABI: quantize (matrix-core kernels for fp16 at G = 128, the generic kernel
for fp32 or G = 256; 2- and 1-bit; plain and double-quantized metadata),
dequantize, and decode attention, to the same bars as the plain rotation."""

import math
import sys

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import DEV, requires_gpu, torch
from tests.golden import load_codebook
from tests.parity import (SAME_BYTES_REL, check_attention, check_dq_sequence,
                          check_quantized_sequence, rel_l2)

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]

SIGNS = synth.rht_signs(2024)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _setup(m, G, dq=False, signs=SIGNS):
    """(Params with NSN_RHT, device table, the codebook the oracle uses)."""
    C = load_codebook(m)
    p = nsnq.Params(sub_dim=m, group_size=G, dq=dq, rht_signs=signs)
    table = torch.empty(nsnq.nsn_table_size(p), dtype=torch.uint8, device=DEV)
    nsnq.nsn_prepare_codebook(p, torch.from_numpy(C).to(DEV), table)
    return p, table, (oracle.codebook_4bit(C) if dq else C)


def _quantize(p, table, x_np):
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    n_seq, T, _ = x.shape
    codes, meta, shift = (torch.zeros(sh, dtype=dt, device=DEV)
                          for sh, dt in nsnq.cache_layout(p, n_seq, T))
    nsnq.nsn_quantize(p, x, table, codes, meta, shift)
    torch.cuda.synchronize()
    return codes, meta, shift


@pytest.mark.parametrize("m,G,dt", [(4, 128, np.float16), (8, 128, np.float16),
                                    (4, 256, np.float16), (4, 256, np.float32),
                                    (8, 128, np.float32)])
def test_quantize_rht_parity(m, G, dt):
    _say(f"quantize RHT m={m} G={G} {np.dtype(dt).name}")
    K, V = synth.kv_numpy(2, 1024, 5.0, seed=61, dtype=dt)
    x = np.concatenate([K, V])
    p, table, C = _setup(m, G)
    codes, meta, shift = (t.cpu().numpy() for t in _quantize(p, table, x))
    ties = total = 0
    for s in range(x.shape[0]):
        st = check_quantized_sequence(x[s].astype(np.float64), C, G, codes[s], meta[s], shift[s],
                                      signs=SIGNS)
        ties += st["ties"]
        total += st["codes"]
    assert ties <= max(2, total * 1e-4), (ties, total)
    _say(f"  {ties} near-ties of {total} codes")


@pytest.mark.parametrize("m", [4, 8])
def test_quantize_rht_dq_parity(m):
    _say(f"quantize RHT + DQ m={m}")
    K, V = synth.kv_numpy(2, 1024, 5.0, seed=62, dtype=np.float16)
    x = np.concatenate([K, V])
    p, table, C4 = _setup(m, 128, dq=True)
    codes, meta, recs = (t.cpu().numpy() for t in _quantize(p, table, x))
    for s in range(x.shape[0]):
        check_dq_sequence(x[s].astype(np.float64), C4, codes[s], meta[s], recs[s], signs=SIGNS)


@pytest.mark.parametrize("m", [4, 8])
def test_all_plus_signs_give_the_plain_bytes(m):
    """NSN_RHT with every sign +1 is the plain rotation: identical bytes."""
    K, _ = synth.kv_numpy(2, 512, 5.0, seed=63, dtype=np.float16)
    pr, tr, _ = _setup(m, 128, signs=np.ones(128))
    pp = nsnq.Params(sub_dim=m, group_size=128)
    a = _quantize(pr, tr, K)
    b = _quantize(pp, tr, K)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("m,G,dt,dq", [(4, 128, torch.float32, False), (8, 256, torch.float32, False),
                                       (4, 128, torch.float16, False), (4, 128, torch.float32, True),
                                       (8, 128, torch.float32, True)])
def test_dequantize_rht_parity(m, G, dt, dq):
    """GPU dequantization of the GPU's bytes against the oracle's inverse
    randomized rotation of the same bytes (double-quantized records decoded
    first); the plain inverse would be far."""
    _say(f"dequantize RHT m={m} G={G} {dt} dq={dq}")
    K, V = synth.kv_numpy(2, 1024, 5.0, seed=64, dtype=np.float16)
    x = np.concatenate([K, V])
    p, table, C = _setup(m, G, dq=dq)
    dc, dm, ds = _quantize(p, table, x)
    out = torch.empty((x.shape[0], x.shape[1], 128), dtype=dt, device=DEV)
    nsnq.nsn_dequantize(p, dc, dm, ds, table, out)
    torch.cuda.synchronize()
    xh = out.float().cpu().numpy().astype(np.float64)
    codes, meta, shift = (t.cpu().numpy() for t in (dc, dm, ds))
    if dq:
        dec = [oracle.dq_unpack(meta[s], shift[s], G) for s in range(x.shape[0])]
        meta = np.stack([d[0] for d in dec])
        shift = np.stack([d[1] for d in dec])
    tol = SAME_BYTES_REL if dt == torch.float32 else 1e-3
    for s in range(x.shape[0]):
        same = oracle.dequantize(codes[s], meta[s], shift[s], C, G, signs=SIGNS)
        assert rel_l2(xh[s], same) <= tol
        assert rel_l2(xh[s], x[s]) < (0.4 if m == 4 else 0.75)
        plain = oracle.dequantize(codes[s], meta[s], shift[s], C, G)
        assert rel_l2(plain, same) > 0.5


def _cache(p, table, B, Hkv, Nq, R, seed, cap=None, rcap=None):
    n_seq = B * Hkv
    cap = cap or max(Nq, p.group_size)
    rcap = rcap or max(R, 1)
    Kn, Vn = synth.kv_numpy(n_seq, Nq + R, 5.0, seed=seed)
    K, V = torch.from_numpy(Kn).to(DEV), torch.from_numpy(Vn).to(DEV)
    kc = [torch.zeros(sh, dtype=dt, device=DEV) for sh, dt in nsnq.cache_layout(p, n_seq, cap)]
    vc = [torch.zeros(sh, dtype=dt, device=DEV) for sh, dt in nsnq.cache_layout(p, n_seq, cap)]
    if Nq:
        nsnq.nsn_quantize(p, K[:, :Nq], table, *kc)
        nsnq.nsn_quantize(p, V[:, :Nq], table, *vc)
    kr = torch.zeros((n_seq, rcap, 128), dtype=torch.float16, device=DEV)
    vr = torch.zeros_like(kr)
    kr[:, :R] = K[:, Nq:]
    vr[:, :R] = V[:, Nq:]
    v4 = lambda t: t.view(B, Hkv, *t.shape[1:])  # noqa: E731
    return tuple(map(v4, kc)), tuple(map(v4, vc)), v4(kr), v4(vr)


def _host_cache(part, p, B, Hkv):
    """Host (codes, meta, shift) the oracle reads; double-quantized records
    decoded to (s1, s2') and o'."""
    c, mt, sh = (t.cpu().numpy() for t in part)
    if not p.dq:
        return c, mt, sh
    cap = c.shape[2]
    meta = np.zeros((B, Hkv, cap, 2))
    shift = np.zeros((B, Hkv, cap // 128, 128))
    for b in range(B):
        for h in range(Hkv):
            meta[b, h], shift[b, h] = oracle.dq_unpack(mt[b, h], sh[b, h], 128)
    return c, meta, shift


@pytest.mark.parametrize("B,Hq,Hkv,Nq,R,m,G,dq", [
    (2, 8, 2, 1024, 16, 4, 128, False),     # GQA 4:1
    (1, 8, 2, 2048, 64, 8, 128, False),     # 1-bit codes
    (1, 4, 1, 10240, 7, 4, 256, False),     # several chunks, ragged chunk end, G = 256
    (1, 16, 2, 3072, 5, 4, 128, True),      # double-quantized, two head blocks
    (1, 4, 1, 0, 9, 4, 128, False),         # residual only
])
def test_attention_rht_parity(B, Hq, Hkv, Nq, R, m, G, dq):
    _say(f"attention RHT B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} R={R} m={m} G={G} dq={dq}")
    p, table, C = _setup(m, G, dq=dq)
    k, v, kr, vr = _cache(p, table, B, Hkv, Nq, R, seed=65)
    q = synth.query_torch((B, Hq, 128), seed=66, device=DEV)
    scale = 1.0 / math.sqrt(128)
    ws = nsnq.nsn_decode_attention_workspace_size(p, B, Hq, Hkv, Nq, R, k[0].shape[2],
                                                  kr.shape[2], scale)
    work = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    nsnq.nsn_decode_attention(p, q, k, v, kr, vr, table, work, out, Nq, R, scale)
    out2 = torch.full_like(out, float("nan"))
    nsnq.nsn_decode_attention_noalloc(p, q, k, v, kr, vr, table, out2, Nq, R, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, out2.cpu().numpy())
    kh, vh = _host_cache(k, p, B, Hkv), _host_cache(v, p, B, Hkv)
    want = oracle.decode_attention(q.cpu().numpy(), kh, vh, kr.cpu().numpy(), vr.cpu().numpy(),
                                   C, G, Nq, R, scale, signs=SIGNS)
    check_attention(got, want, "RHT")
