"""Calls issued on two HIP streams at once.  The library keeps no state
between calls besides the thread-local error string (the static scratch of
the no-allocation entry point aside), so quantize, dequantize and decode
attention running concurrently on two streams, each with its own outputs
and workspace, write the same bytes as when they run one after the other;
the binding's `stream` argument is the stream the kernels run on."""

import math

import numpy as np
import pytest

import synth
from tests.gpu_common import DEV, alloc_outputs, requires_gpu, torch
from tests.test_gpu_attention import build_cache

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def test_two_streams_at_once_write_what_they_write_in_sequence():
    B, Hq, Hkv, Nq, R, m, G = 4, 32, 8, 4096, 64, 4, 128
    print("two streams: quantize, dequantize and attention", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=501, device_gen=True)
    p, table = cache["p"], cache["table"]
    scale = 1.0 / math.sqrt(128)
    ws = nsnq.nsn_decode_attention_workspace_size(p, B, Hq, Hkv, Nq, R, Nq, R, scale)
    n_seq, T = 32, 8192
    K, V = synth.kv_torch(n_seq, T, 5.0, 503, DEV)
    xs = (K, V)
    qs = [synth.query_torch((B, Hq, 128), seed=504 + i, device=DEV) for i in range(2)]
    works = [torch.empty(ws, dtype=torch.uint8, device=DEV) for _ in range(2)]
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV) for _ in range(2)]
    qouts = [alloc_outputs(n_seq, T, m, G) for _ in range(2)]
    recs = [torch.empty((n_seq, T, 128), dtype=torch.float32, device=DEV) for _ in range(2)]

    def work_on(i, stream):
        codes, meta, shift = qouts[i]
        nsnq.nsn_quantize(p, xs[i], table, codes, meta, shift, stream=stream)
        nsnq.nsn_dequantize(p, codes, meta, shift, table, recs[i], stream=stream)
        for _ in range(4):
            nsnq.nsn_decode_attention(p, qs[i], cache["k"], cache["v"], cache["kr"], cache["vr"],
                                      table, works[i], outs[i], Nq, R, scale, stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        return [[t.cpu().numpy().copy() for t in (*qouts[i], recs[i], outs[i])] for i in range(2)]

    def clear():
        for i in range(2):
            for t in qouts[i]:
                t.zero_()
            recs[i].fill_(float("nan"))
            outs[i].fill_(float("nan"))
            works[i].fill_(255)
        torch.cuda.synchronize()

    for i in range(2):
        work_on(i, None)
    ref = snapshot()
    for i in range(2):
        assert np.isfinite(ref[i][3]).all() and np.isfinite(ref[i][4]).all()

    streams = [torch.cuda.Stream(device=DEV) for _ in range(2)]
    for rep in range(2):
        clear()
        cur = torch.cuda.current_stream()
        for s in streams:
            s.wait_stream(cur)
        for i in range(2):
            work_on(i, streams[i])
        for s in streams:
            cur.wait_stream(s)
        got = snapshot()
        for i in range(2):
            for a, b in zip(got[i], ref[i]):
                assert np.array_equal(a, b, equal_nan=True), (rep, i)
