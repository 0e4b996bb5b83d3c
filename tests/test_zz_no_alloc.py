"""nsn_decode_attention_noalloc (static device scratch, no workspace argument)
against nsn_decode_attention on the same inputs, through the C ABI: two calls
in a row, the second on a smaller input, each bit-identical to the entry
point with a workspace and within the parity bar of the oracle."""

import ctypes
import math

import numpy as np
import pytest

import oracle
import synth
from kv_cache_calibration_amd import _lib
from tests.gpu_common import DEV, requires_gpu, torch
from tests.parity import check_attention
from tests.test_gpu_attention import build_cache, run_gpu, to_np

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def _noalloc(cache, q, scale):
    B, Hq, _ = q.shape
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    nsnq.nsn_decode_attention_noalloc(cache["p"], q, cache["k"], cache["v"], cache["kr"], cache["vr"],
                                      cache["table"], out, cache["Nq"], cache["R"], scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("m,G", [(4, 128), (8, 256)])
def test_noalloc_matches_workspace_entry_point_twice(m, G):
    scale = 1 / math.sqrt(128)
    # first call: 4 batches, 16 q heads on 4 kv heads, 8192 quantized + 37 residual tokens
    # second call: a smaller cache (fewer partials) right after, on the same scratch
    for B, Hq, Hkv, Nq, R, seed in ((4, 16, 4, 8192, 37, 401), (1, 4, 1, 2 * G, 3, 402)):
        print(f"noalloc m={m} G={G} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} R={R}", flush=True)
        cache = build_cache(B, Hkv, Nq, R, m, G, seed=seed)
        q = synth.query_torch((B, Hq, 128), seed=seed + 1, device=DEV)
        want_ws = run_gpu(cache, q, scale)
        got = _noalloc(cache, q, scale)
        assert np.array_equal(got, want_ws), np.abs(got - want_ws).max()
        k, v, kr, vr = to_np(cache)
        heads = [(0, 0), (B - 1, Hq - 1)]
        qn = q.cpu().numpy()
        for b, h in heads:
            kvh = h // (Hq // Hkv)
            sl = lambda t: t[b:b + 1, kvh:kvh + 1]  # noqa: E731
            want = oracle.decode_attention(qn[b:b + 1, h:h + 1], tuple(sl(t) for t in k),
                                           tuple(sl(t) for t in v), sl(kr), sl(vr), cache["C"], G,
                                           Nq, R, scale)
            check_attention(got[b, h], want[0, 0], f"noalloc (b={b}, h={h})")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """64 batches x 64 q heads on 8 kv heads at 16384 tokens need 6.5 MB of
    partials: refused with NSN_ERR_UNSUPPORTED before anything runs (the
    pointers are never used)."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x10000)
    p = _lib.nsn_params(128, 4, 256, 128, 1)
    s = _lib.nsn_attn_shape(64, 64, 8, 16384, 1, 16384, 1, 0.088)
    assert lib.nsn_decode_attention_workspace_size(ctypes.byref(p), ctypes.byref(s)) > (4 << 20)
    st = lib.nsn_decode_attention_noalloc(ctypes.byref(p), ctypes.byref(s), *([fake] * 10), fake,
                                          ctypes.c_void_p(0))
    assert st == _lib.NSN_ERR_UNSUPPORTED
    assert b"static" in lib.nsn_last_error()
    s = _lib.nsn_attn_shape(16, 32, 8, 32768, 128, 32768, 128, 0.088)
    assert lib.nsn_decode_attention_workspace_size(ctypes.byref(p), ctypes.byref(s)) <= (4 << 20)
