"""Parity of nsn_decode_attention_rope (HIP, through the C ABI) with the
oracle's attention over keys stored before rotary embedding, on the same
cache bytes: max-abs error <= 2e-3 and per-head relative L2 <= 1e-4 (the
output is fp32)."""

import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import DEV, requires_gpu, torch
from tests.parity import check_attention
from tests.test_gpu_attention import build_cache, to_np

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def run_rope(cache, q, q_pos, base, scale=None):
    B, Hq, _ = q.shape
    Hkv = cache["k"][0].shape[1]
    scale = scale or 1.0 / math.sqrt(128)
    p = cache["p"]
    ws = nsnq.nsn_decode_attention_workspace_size(
        p, B, Hq, Hkv, cache["Nq"], cache["R"], cache["k"][0].shape[2], cache["kr"].shape[2], scale)
    work = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    nsnq.nsn_decode_attention_rope(p, q, cache["k"], cache["v"], cache["kr"], cache["vr"],
                                   cache["table"], work, out, cache["Nq"], cache["R"], scale,
                                   q_pos, base)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_rope(cache, q, q_pos, base, heads=None, scale=None):
    scale = scale or 1.0 / math.sqrt(128)
    got = run_rope(cache, q, q_pos, base, scale)
    k, v, kr, vr = to_np(cache)
    want = oracle.decode_attention_rope(q.cpu().numpy(), k, v, kr, vr, cache["C"], cache["G"],
                                        cache["Nq"], cache["R"], scale, q_pos, base, heads=heads)
    err, _ = check_attention(got, want, "rotary")
    return err


@pytest.mark.parametrize("B,Hq,Hkv,Nq,R,m,G,dpos,base", [
    (2, 8, 2, 1024, 16, 4, 128, 0, 10000.0),      # GQA 4:1, query = last residual position
    (1, 4, 1, 2048, 128, 8, 128, 0, 10000.0),     # 1-bit codes
    (1, 16, 2, 3072, 5, 4, 128, 0, 500000.0),     # two head blocks, another base
    (2, 4, 2, 1536, 33, 4, 256, 1000, 10000.0),   # G = 256, query well past the keys
    (1, 3, 1, 512, 200, 4, 128, 0, 10000.0),      # residual over several 64-key tiles
    (1, 4, 1, 10240, 7, 4, 128, 123456, 10000.0),  # several chunks, large positions
])
def test_attention_rope_parity(B, Hq, Hkv, Nq, R, m, G, dpos, base):
    print(f"rope attention B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} R={R} m={m} G={G} dpos={dpos}", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=51)
    q = synth.query_torch((B, Hq, 128), seed=52, device=DEV)
    check_rope(cache, q, Nq + R - 1 + dpos, base)


def test_attention_rope_residual_only_and_quantized_only():
    print("rope attention: residual only, quantized only", flush=True)
    q = synth.query_torch((1, 8, 128), seed=54, device=DEV)
    cache = build_cache(1, 2, 0, 100, 4, 128, seed=53)
    check_rope(cache, q, 99, 10000.0)
    cache = build_cache(1, 2, 1024, 0, 4, 128, seed=55)
    check_rope(cache, q, 1023, 10000.0)


def test_attention_rope_position_zero_keys_match_plain_attention_for_one_key():
    """One residual key at position 0 and the query at position 0: no
    rotation at all, so the result is the plain attention's (its value)."""
    cache = build_cache(1, 1, 0, 1, 4, 128, seed=56)
    q = synth.query_torch((1, 4, 128), seed=57, device=DEV)
    got = run_rope(cache, q, 0, 10000.0)
    vr = cache["vr"].cpu().numpy()[0, 0, 0].astype(np.float64)
    check_attention(got[0], np.broadcast_to(vr, got[0].shape), "rotary, one key")


def test_attention_rope_decode_workload_sampled():
    """The decode workload at full size with keys before rotary embedding
    (query at the last residual position); sampled heads vs the oracle."""
    w = synth.WORKLOADS["decode"]
    print("rope attention decode workload (full size, sampled heads)", flush=True)
    cache = build_cache(w["B"], w["Hkv"], w["Nq"], w["R"], w["m"], w["G"], seed=w["seed"],
                        device_gen=True)
    q = synth.query_torch((w["B"], w["Hq"], 128), seed=w["seed"] + 1, device=DEV)
    q_pos = w["Nq"] + w["R"] - 1
    got = run_rope(cache, q, q_pos, 10000.0)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(1)
    heads = [(int(b), int(h)) for b, h in zip(rng.integers(0, w["B"], 3), rng.integers(0, w["Hq"], 3))]
    heads += [(0, 0), (w["B"] - 1, w["Hq"] - 1)]
    qn = q.cpu().numpy()
    for b, h in heads:
        kvh = h // (w["Hq"] // w["Hkv"])
        sl = lambda t: t[b:b + 1, kvh:kvh + 1].cpu().numpy()  # noqa: E731
        k = tuple(sl(t) for t in cache["k"])
        v = tuple(sl(t) for t in cache["v"])
        want = oracle.decode_attention_rope(qn[b:b + 1, h:h + 1], k, v, sl(cache["kr"]),
                                            sl(cache["vr"]), cache["C"], w["G"], w["Nq"], w["R"],
                                            1 / math.sqrt(128), q_pos, 10000.0)
        check_attention(got[b, h], want[0, 0], f"rotary (b={b}, h={h})")


def test_attention_rope_two_rounds_of_workgroups_sampled():
    """Twice the decode workload's batch (B = 32): 1024 split workgroups, two
    rounds at two per CU, so workgroups start on CUs that a finished one left;
    sampled heads vs the oracle, and two calls give identical bytes."""
    w = synth.WORKLOADS["decode"]
    B = 2 * w["B"]
    print(f"rope attention B={B} (two rounds of workgroups, sampled heads)", flush=True)
    cache = build_cache(B, w["Hkv"], w["Nq"], w["R"], w["m"], w["G"], seed=w["seed"] + 7,
                        device_gen=True)
    q = synth.query_torch((B, w["Hq"], 128), seed=w["seed"] + 8, device=DEV)
    q_pos = w["Nq"] + w["R"]
    got = run_rope(cache, q, q_pos, 10000.0)
    assert np.array_equal(got, run_rope(cache, q, q_pos, 10000.0))
    qn = q.cpu().numpy()
    for b, h in ((0, 0), (13, 17), (B - 1, w["Hq"] - 1)):
        kvh = h // (w["Hq"] // w["Hkv"])
        sl = lambda t: t[b:b + 1, kvh:kvh + 1].cpu().numpy()  # noqa: E731
        k = tuple(sl(t) for t in cache["k"])
        v = tuple(sl(t) for t in cache["v"])
        want = oracle.decode_attention_rope(qn[b:b + 1, h:h + 1], k, v, sl(cache["kr"]),
                                            sl(cache["vr"]), cache["C"], w["G"], w["Nq"], w["R"],
                                            1 / math.sqrt(128), q_pos, 10000.0)
        check_attention(got[b, h], want[0, 0], f"rotary (b={b}, h={h})")
