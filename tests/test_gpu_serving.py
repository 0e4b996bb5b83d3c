"""End-to-end decode loop through the C ABI, as a serving engine drives it:
prefill into a cache with spare capacity, then per step append one token per
(batch, kv head) to the fp16 residual window, quantize a full window into the
cache at its group offset, and attend (NSNQuant summary, Methodology §4:
quantized part plus full-precision residual, flushed when full).  The
attention is compared with the oracle at sampled steps, and the flushed
cache with one quantize call over the same tokens; plain and
double-quantized caches, keys before rotary embedding, and the randomized
rotation."""

import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import DEV, requires_gpu, torch
from tests.golden import load_codebook
from tests.parity import check_attention

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def _host(part, B, Hkv, cap, G, dq):
    c, mt, sh = (x.cpu().numpy() for x in part)
    if not dq:
        return c, mt, sh
    meta = np.zeros((B, Hkv, cap, 2))
    shift = np.zeros((B, Hkv, cap // G, 128))
    for b in range(B):
        for h in range(Hkv):
            meta[b, h], shift[b, h] = oracle.dq_unpack(mt[b, h], sh[b, h], G)
    return c, meta, shift


@pytest.mark.parametrize("dq,rope,rht", [(False, False, False), (True, False, False),
                                         (False, True, False), (True, True, False),
                                         (False, False, True), (True, False, True)])
def test_decode_loop(dq, rope, rht):
    m, G, B, Hq, Hkv = 4, 128, 2, 8, 2
    n_seq = B * Hkv
    pre, steps = 3 * G, 2 * G + 37          # an odd number of prefill groups: odd flush offsets
    cap, rcap = ((pre + steps) // G + 2) * G, G
    print(f"decode loop dq={dq} rope={rope} rht={rht}", flush=True)
    C = load_codebook(m)
    signs = synth.rht_signs(77) if rht else None
    p = nsnq.Params(sub_dim=m, group_size=G, dq=dq, rht_signs=signs)
    t = torch.empty(nsnq.nsn_table_size(p), dtype=torch.uint8, device=DEV)
    nsnq.nsn_prepare_codebook(p, torch.from_numpy(C).to(DEV), t)
    Cref = oracle.codebook_4bit(C) if dq else C
    Kn, Vn = synth.kv_numpy(n_seq, pre + steps, 5.0, seed=17)
    K, V = torch.from_numpy(Kn).to(DEV), torch.from_numpy(Vn).to(DEV)
    lay = nsnq.cache_layout(p, n_seq, cap)
    kc = tuple(torch.zeros(s, dtype=d, device=DEV) for s, d in lay)
    vc = tuple(torch.zeros(s, dtype=d, device=DEV) for s, d in lay)
    nsnq.nsn_quantize(p, K[:, :pre], t, *kc)
    nsnq.nsn_quantize(p, V[:, :pre], t, *vc)
    kr = torch.zeros((n_seq, rcap, 128), dtype=torch.float16, device=DEV)
    vr = torch.zeros_like(kr)

    def v4(x):
        return x.view(B, Hkv, *x.shape[1:])
    scale = 1 / math.sqrt(128)
    ws = nsnq.nsn_decode_attention_workspace_size(p, B, Hq, Hkv, cap, rcap, cap, rcap, scale)
    work = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    nq, nr = pre, 0
    for step in range(steps):
        pos = pre + step
        nsnq.nsn_residual_append(K[:, pos].contiguous(), kr, nr)
        nsnq.nsn_residual_append(V[:, pos].contiguous(), vr, nr)
        nr += 1
        if nr == G:
            g = nq // G
            nsnq.nsn_quantize(p, kr, t, kc[0][:, nq:], kc[1][:, nq:], kc[2][:, g:])
            nsnq.nsn_quantize(p, vr, t, vc[0][:, nq:], vc[1][:, nq:], vc[2][:, g:])
            nq, nr = nq + G, 0
        q = synth.query_torch((B, Hq, 128), seed=1000 + step, device=DEV)
        k4, vv4 = tuple(v4(x) for x in kc), tuple(v4(x) for x in vc)
        if rope:
            nsnq.nsn_decode_attention_rope(p, q, k4, vv4, v4(kr), v4(vr), t, work, out, nq, nr, scale,
                                           nq + nr - 1, 10000.0)
        else:
            nsnq.nsn_decode_attention(p, q, k4, vv4, v4(kr), v4(vr), t, work, out, nq, nr, scale)
        if step in (0, 127, 128, 200, steps - 1):
            torch.cuda.synchronize()
            k, v = _host(k4, B, Hkv, cap, G, dq), _host(vv4, B, Hkv, cap, G, dq)
            krn, vrn = v4(kr).cpu().numpy(), v4(vr).cpu().numpy()
            if rope:
                want = oracle.decode_attention_rope(q.cpu().numpy(), k, v, krn, vrn, Cref, G, nq, nr,
                                                    scale, nq + nr - 1, 10000.0)
            else:
                want = oracle.decode_attention(q.cpu().numpy(), k, v, krn, vrn, Cref, G, nq, nr, scale,
                                               signs=signs)
            check_attention(out.cpu().numpy(), want, f"decode loop step {step}")
    # the flushed cache equals one quantize call over the same tokens
    kc2 = tuple(torch.zeros(s, dtype=d, device=DEV) for s, d in nsnq.cache_layout(p, n_seq, nq))
    nsnq.nsn_quantize(p, K[:, :nq], t, *kc2)
    torch.cuda.synchronize()
    for a, b in zip(kc, kc2):
        assert torch.equal(a[:, :b.shape[1]], b)
