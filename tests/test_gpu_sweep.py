"""A seeded sweep of small configurations through the C ABI against the
oracle, to the bars of the dedicated tests.

Quantize + dequantize: sequence counts, lengths, fp16 / fp32 input, 1- and
2-bit codes, G = 128 / 256, scale adjustment on and off, double
quantization, the randomized rotation.  Decode attention: batch and head
counts, GQA ratios from 1 to 8, fill levels (none to ten groups, spare cache
and residual capacity), residual lengths, the same code and metadata
options, rotary keys.  Every case is drawn from a fixed seed and printed
before it runs."""

import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import DEV, requires_gpu, torch
from tests.golden import load_codebook
from tests.parity import (SAME_BYTES_REL, check_attention, check_dq_sequence,
                          check_quantized_sequence, rel_l2)
from tests.test_gpu_rht import _cache, _host_cache

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def _quant_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        m = int(rng.choice([4, 8]))
        G = int(rng.choice([128, 256]))
        dq = G == 128 and bool(rng.random() < 0.35)
        rht = bool(rng.random() < 0.4)
        dt = "float16" if (dq or rng.random() < 0.6) else "float32"   # DQ quantizes fp16 input
        sa = bool(rng.random() < 0.8)
        n_seq = int(rng.integers(1, 6))
        T = G * int(rng.integers(1, 7))
        out_dt = "float32" if rng.random() < 0.5 else "float16"
        cases.append(dict(i=i, m=m, G=G, dq=dq, rht=rht, dt=dt, sa=sa, n_seq=n_seq, T=T, out=out_dt))
    return cases


def _attn_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        m = int(rng.choice([4, 8]))
        G = int(rng.choice([128, 128, 256]))
        dq = G == 128 and bool(rng.random() < 0.3)
        rope = bool(rng.random() < 0.3)
        rht = not rope and bool(rng.random() < 0.3)
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 4))
        grp = int(rng.choice([1, 2, 3, 4, 5, 8]))
        Nq = G * int(rng.integers(0, 11))
        R = int(rng.integers(0 if Nq else 1, 151))
        cap = Nq + G * int(rng.integers(0, 3))
        rcap = R + int(rng.integers(0, 21))
        dpos = int(rng.integers(0, 5001))
        base = float(rng.choice([10000.0, 500000.0]))
        cases.append(dict(i=i, m=m, G=G, dq=dq, rope=rope, rht=rht, B=B, Hkv=Hkv, Hq=Hkv * grp,
                          Nq=Nq, R=R, cap=max(cap, G), rcap=max(rcap, 1), dpos=dpos, base=base))
    return cases


def _table(m, G, dq, sa, signs):
    C = load_codebook(m)
    p = nsnq.Params(sub_dim=m, group_size=G, dq=dq, scale_adjust=sa, rht_signs=signs)
    table = torch.empty(nsnq.nsn_table_size(p), dtype=torch.uint8, device=DEV)
    nsnq.nsn_prepare_codebook(p, torch.from_numpy(C).to(DEV), table)
    return p, table, (oracle.codebook_4bit(C) if dq else C)


@pytest.mark.parametrize("case", _quant_cases(24, 2026), ids=lambda c: f"q{c['i']}")
def test_sweep_quantize_dequantize(case):
    c = case
    print(f"sweep quantize {c}", flush=True)
    signs = synth.rht_signs(3000 + c["i"]) if c["rht"] else None
    p, table, C = _table(c["m"], c["G"], c["dq"], c["sa"], signs)
    n_seq, T, G = c["n_seq"], c["T"], c["G"]
    K, V = synth.kv_numpy((n_seq + 1) // 2, T, 5.0, seed=3100 + c["i"], dtype=np.dtype(c["dt"]))
    x = np.ascontiguousarray(np.concatenate([K, V])[:n_seq])
    xd = torch.from_numpy(x).to(DEV)
    codes, meta, shift = (torch.zeros(sh, dtype=dt, device=DEV) for sh, dt in nsnq.cache_layout(p, n_seq, T))
    nsnq.nsn_quantize(p, xd, table, codes, meta, shift)
    torch.cuda.synchronize()
    cg, mg, sg = (t.cpu().numpy() for t in (codes, meta, shift))
    ties = total = 0
    for s in range(n_seq):
        xs = x[s].astype(np.float64)
        if c["dq"]:
            st = check_dq_sequence(xs, C, cg[s], mg[s], sg[s], scale_adjust=c["sa"], signs=signs)
        else:
            st = check_quantized_sequence(xs, C, G, cg[s], mg[s], sg[s], scale_adjust=c["sa"], signs=signs)
        ties += st["ties"]
        total += st["codes"]
    assert ties <= max(2, total * 1e-4), (ties, total)
    # dequantize the GPU's bytes: the oracle's inverse of the same bytes, and
    # the reconstruction of x
    out_t = torch.float32 if c["out"] == "float32" else torch.float16
    out = torch.empty((n_seq, T, 128), dtype=out_t, device=DEV)
    nsnq.nsn_dequantize(p, codes, meta, shift, table, out)
    torch.cuda.synchronize()
    xh = out.float().cpu().numpy().astype(np.float64)
    if c["dq"]:
        dec = [oracle.dq_unpack(mg[s], sg[s], G) for s in range(n_seq)]
        mg = np.stack([d[0] for d in dec])
        sg = np.stack([d[1] for d in dec])
    tol = SAME_BYTES_REL if out_t == torch.float32 else 1e-3
    for s in range(n_seq):
        same = oracle.dequantize(cg[s], mg[s], sg[s], C, G, signs=signs)
        assert rel_l2(xh[s], same) <= tol, (s, rel_l2(xh[s], same))
        assert rel_l2(xh[s], x[s].astype(np.float64)) < (0.45 if c["m"] == 4 else 0.8)
    print(f"  {ties} near-ties of {total} codes", flush=True)


@pytest.mark.parametrize("case", _attn_cases(36, 2027), ids=lambda c: f"a{c['i']}")
def test_sweep_decode_attention(case):
    c = case
    print(f"sweep attention {c}", flush=True)
    signs = synth.rht_signs(3200 + c["i"]) if c["rht"] else None
    p, table, C = _table(c["m"], c["G"], c["dq"], True, signs)
    B, Hq, Hkv, Nq, R, G = c["B"], c["Hq"], c["Hkv"], c["Nq"], c["R"], c["G"]
    k, v, kr, vr = _cache(p, table, B, Hkv, Nq, R, seed=3300 + c["i"], cap=c["cap"], rcap=c["rcap"])
    q = synth.query_torch((B, Hq, 128), seed=3400 + c["i"], device=DEV)
    scale = 1.0 / math.sqrt(128)
    ws = nsnq.nsn_decode_attention_workspace_size(p, B, Hq, Hkv, Nq, R, c["cap"], c["rcap"], scale)
    work = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    q_pos = Nq + R - 1 + c["dpos"]
    if c["rope"]:
        nsnq.nsn_decode_attention_rope(p, q, k, v, kr, vr, table, work, out, Nq, R, scale, q_pos, c["base"])
    else:
        nsnq.nsn_decode_attention(p, q, k, v, kr, vr, table, work, out, Nq, R, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    kh, vh = _host_cache(k, p, B, Hkv), _host_cache(v, p, B, Hkv)
    qn, krn, vrn = q.cpu().numpy(), kr.cpu().numpy(), vr.cpu().numpy()
    if c["rope"]:
        want = oracle.decode_attention_rope(qn, kh, vh, krn, vrn, C, G, Nq, R, scale, q_pos, c["base"])
    else:
        want = oracle.decode_attention(qn, kh, vh, krn, vrn, C, G, Nq, R, scale, signs=signs)
    check_attention(got, want, f"sweep a{c['i']}")
