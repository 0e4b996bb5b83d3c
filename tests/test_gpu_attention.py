"""Parity of nsn_decode_attention (HIP, through the C ABI) with the oracle on
the same cache bytes: max-abs error <= 2e-3 and per-head relative L2 <= 1e-4
(the output is fp32)."""

import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import DEV, alloc_outputs, requires_gpu, table_for, torch
from tests.parity import check_attention

import kv_cache_calibration_amd as nsnq

pytestmark = [pytest.mark.gpu, requires_gpu]


def build_cache(B, Hkv, Nq, R, m, G, seed, cap=None, rcap=None, device_gen=False):
    """Quantize synthetic K/V (outlier model) into a cache with the library."""
    cap = cap or max(Nq, G)
    rcap = rcap or max(R, 1)
    p, table, C = table_for(m, G)
    n_seq = B * Hkv
    if device_gen:
        K, V = synth.kv_torch(n_seq, Nq + R, 5.0, seed, DEV)
    else:
        Kn, Vn = synth.kv_numpy(n_seq, Nq + R, 5.0, seed=seed)
        K, V = torch.from_numpy(Kn).to(DEV), torch.from_numpy(Vn).to(DEV)
    kc, km, ks = alloc_outputs(n_seq, cap, m, G)
    vc, vm, vs = alloc_outputs(n_seq, cap, m, G)
    if Nq:
        nsnq.nsn_quantize(p, K[:, :Nq], table, kc, km, ks)
        nsnq.nsn_quantize(p, V[:, :Nq], table, vc, vm, vs)
    kr = torch.zeros((n_seq, rcap, 128), dtype=torch.float16, device=DEV)
    vr = torch.zeros_like(kr)
    kr[:, :R] = K[:, Nq:]
    vr[:, :R] = V[:, Nq:]

    def v4(t):
        return t.view(B, Hkv, *t.shape[1:])
    return dict(p=p, table=table, C=C, k=(v4(kc), v4(km), v4(ks)), v=(v4(vc), v4(vm), v4(vs)),
                kr=v4(kr), vr=v4(vr), G=G, Nq=Nq, R=R)


def run_gpu(cache, q, scale=None):
    B, Hq, _ = q.shape
    Hkv = cache["k"][0].shape[1]
    scale = scale or 1.0 / math.sqrt(128)
    p = cache["p"]
    ws = nsnq.nsn_decode_attention_workspace_size(
        p, B, Hq, Hkv, cache["Nq"], cache["R"], cache["k"][0].shape[2], cache["kr"].shape[2], scale)
    work = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    nsnq.nsn_decode_attention(p, q, cache["k"], cache["v"], cache["kr"], cache["vr"],
                              cache["table"], work, out, cache["Nq"], cache["R"], scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def to_np(cache):
    f = lambda t: t.cpu().numpy()  # noqa: E731
    return (tuple(f(t) for t in cache["k"]), tuple(f(t) for t in cache["v"]),
            f(cache["kr"]), f(cache["vr"]))


def check(cache, q, heads=None, scale=None):
    scale = scale or 1.0 / math.sqrt(128)
    got = run_gpu(cache, q, scale)
    k, v, kr, vr = to_np(cache)
    want = oracle.decode_attention(q.cpu().numpy(), k, v, kr, vr, cache["C"], cache["G"],
                                   cache["Nq"], cache["R"], scale, heads=heads)
    err, _ = check_attention(got, want)
    return err


@pytest.mark.parametrize("B,Hq,Hkv,Nq,R,m,G", [
    (2, 8, 2, 1024, 16, 4, 128),       # GQA 4:1
    (1, 2, 2, 2048, 128, 4, 128),      # MHA
    (1, 16, 2, 3072, 5, 4, 128),       # GQA 8:1 (two head blocks), ragged last tile
    (2, 4, 2, 1536, 33, 4, 256),       # G = 256, GQA 2:1
    (1, 8, 2, 2048, 64, 8, 128),       # 1-bit codes
    (1, 4, 1, 10240, 7, 4, 128),       # several chunks, ragged chunk end
    (1, 4, 1, 128, 200, 4, 128),       # one group: two of four waves idle; residual in two passes
    (2, 8, 2, 256, 1024, 8, 256),      # one group of G = 256; the largest residual window
    (1, 3, 1, 512, 17, 4, 128),        # 3 q heads in a head block of 4
])
def test_attention_parity_small(B, Hq, Hkv, Nq, R, m, G):
    print(f"attention B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} R={R} m={m} G={G}", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=31)
    q = synth.query_torch((B, Hq, 128), seed=32, device=DEV)
    check(cache, q)


def test_attention_residual_only_and_quantized_only():
    cache = build_cache(1, 2, 0, 100, 4, 128, seed=33)
    q = synth.query_torch((1, 8, 128), seed=34, device=DEV)
    check(cache, q)
    cache = build_cache(1, 2, 1024, 0, 4, 128, seed=35)
    check(cache, q)


def test_attention_zero_query_is_mean_of_values():
    cache = build_cache(1, 1, 512, 3, 4, 128, seed=36)
    q = torch.zeros((1, 4, 128), dtype=torch.float16, device=DEV)
    got = run_gpu(cache, q)
    _, v, _, vr = to_np(cache)
    vals = np.concatenate([oracle.dequantize(*(a[0, 0, :512] for a in v[:2]), v[2][0, 0, :4],
                                             cache["C"], 128),
                           vr[0, 0, :3].astype(np.float64)])
    check_attention(got[0], np.broadcast_to(vals.mean(0), got[0].shape), "q = 0")


def test_attention_large_scale_softmax_is_stable():
    """A large softmax scale makes a few tokens dominate; still finite."""
    cache = build_cache(1, 1, 2048, 16, 4, 128, seed=37)
    q = synth.query_torch((1, 4, 128), seed=38, device=DEV)
    check(cache, q, scale=2.0)


def test_attention_decode_workload_sampled():
    """The decode workload at full size: B=16, 32 q heads on 8 kv heads,
    32768 quantized tokens + 128 fp16 residual tokens; sampled heads vs the
    oracle on the same cache bytes."""
    w = synth.WORKLOADS["decode"]
    print("attention decode workload (full size, sampled heads)", flush=True)
    cache = build_cache(w["B"], w["Hkv"], w["Nq"], w["R"], w["m"], w["G"], seed=w["seed"],
                        device_gen=True)
    q = synth.query_torch((w["B"], w["Hq"], 128), seed=w["seed"] + 1, device=DEV)
    got = run_gpu(cache, q)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(0)
    heads = [(int(b), int(h)) for b, h in zip(rng.integers(0, w["B"], 4), rng.integers(0, w["Hq"], 4))]
    heads += [(0, 0), (w["B"] - 1, w["Hq"] - 1)]
    qn = q.cpu().numpy()
    for b, h in heads:
        kvh = h // (w["Hq"] // w["Hkv"])
        sl = lambda t: t[b:b + 1, kvh:kvh + 1].cpu().numpy()  # noqa: E731
        k = tuple(sl(t) for t in cache["k"])
        v = tuple(sl(t) for t in cache["v"])
        want = oracle.decode_attention(qn[b:b + 1, h:h + 1], k, v, sl(cache["kr"]), sl(cache["vr"]),
                                       cache["C"], w["G"], w["Nq"], w["R"], 1 / math.sqrt(128))
        check_attention(got[b, h], want[0, 0], f"(b={b}, h={h})")


@pytest.mark.parametrize("m,G", [(4, 128), (8, 256)])
def test_attention_largest_chunk_sampled(m, G):
    """Enough (batch, kv head) rows that one workgroup takes the largest chunk
    (8192 quantized tokens: 128 tiles, 64 groups of 128 in LDS), two chunks
    per row; sampled heads vs the oracle on the same cache bytes."""
    B, Hq, Hkv, Nq, R = 64, 32, 8, 16384, 3
    print(f"attention largest chunk m={m} G={G}", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=71, device_gen=True)
    scale = 1 / math.sqrt(128)
    ws = nsnq.nsn_decode_attention_workspace_size(cache["p"], B, Hq, Hkv, Nq, R, Nq, R, scale)
    assert ws == B * Hq * (2 + 1) * 132 * 4          # two chunks of 8192 + the residual partial
    q = synth.query_torch((B, Hq, 128), seed=72, device=DEV)
    got = run_gpu(cache, q, scale)
    assert np.isfinite(got).all()
    qn = q.cpu().numpy()
    for b, h in [(0, 0), (17, 9), (B - 1, Hq - 1)]:
        kvh = h // (Hq // Hkv)
        sl = lambda t: t[b:b + 1, kvh:kvh + 1].cpu().numpy()  # noqa: E731
        k = tuple(sl(t) for t in cache["k"])
        v = tuple(sl(t) for t in cache["v"])
        want = oracle.decode_attention(qn[b:b + 1, h:h + 1], k, v, sl(cache["kr"]), sl(cache["vr"]),
                                       cache["C"], G, Nq, R, scale)
        check_attention(got[b, h], want[0, 0], f"(b={b}, h={h})")


@pytest.mark.parametrize("m,G", [(4, 128), (8, 256)])
def test_attention_partly_filled_cache_and_residual(m, G):
    """The serving case: the cache rows have room for more groups than are
    filled (cache_capacity > n_quant_tok) and the residual window is partly
    filled (resid_capacity 128, 37 valid); the unused slots hold garbage that
    must not be read."""
    B, Hq, Hkv, Nq, R = 2, 8, 2, 4 * G, 37
    cap, rcap = Nq + 3 * G, 128
    print(f"attention partly filled m={m} G={G}", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=91, cap=cap, rcap=rcap)
    # garbage in the unused slots: NaN metadata and residual tokens, random codes
    for part in (cache["k"], cache["v"]):
        part[0][:, :, Nq:] = torch.randint(0, 256, part[0][:, :, Nq:].shape, dtype=torch.uint8, device=DEV)
        part[1][:, :, Nq:] = float("nan")
        part[2][:, :, Nq // G:] = float("nan")
    cache["kr"][:, :, R:] = float("nan")
    cache["vr"][:, :, R:] = float("nan")
    q = synth.query_torch((B, Hq, 128), seed=92, device=DEV)
    err = check(cache, q)
    assert np.isfinite(err)


def test_attention_long_context_many_chunks():
    """One (batch, kv head) row of 131072 quantized tokens: 256 chunks of 512
    for one head block, so the merge combines 257 partials."""
    B, Hq, Hkv, Nq, R, m, G = 1, 4, 1, 131072, 5, 4, 128
    print("attention long context: 131072 tokens, one row", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=95, device_gen=True)
    scale = 1 / math.sqrt(128)
    ws = nsnq.nsn_decode_attention_workspace_size(cache["p"], B, Hq, Hkv, Nq, R, Nq, R, scale)
    assert ws == B * Hq * (256 + 1) * 132 * 4
    q = synth.query_torch((B, Hq, 128), seed=96, device=DEV)
    check(cache, q)


def test_attention_any_workspace_contents_and_graph_replay():
    """The output does not depend on what the workspace held (every partial is
    written before it is read): all-ones, zero and random bytes, a workspace
    just used by a call with another split count, and replays of a captured
    HIP graph (eager calls and synchronizations in between) all give the same
    bytes, which match the oracle."""
    B, Hq, Hkv, Nq, R, m, G = 2, 8, 2, 4096, 16, 4, 128
    print("attention: workspace contents and graph replay", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=97)
    q = synth.query_torch((B, Hq, 128), seed=98, device=DEV)
    scale = 1 / math.sqrt(128)
    p = cache["p"]
    ws = nsnq.nsn_decode_attention_workspace_size(p, B, Hq, Hkv, Nq, R, Nq, R, scale)
    work = torch.empty(ws, dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)

    def launch(nq):
        nsnq.nsn_decode_attention(p, q, cache["k"], cache["v"], cache["kr"], cache["vr"],
                                  cache["table"], work, out, nq, R, scale)

    def call(nq=Nq):
        out.fill_(float("nan"))
        launch(nq)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    work.fill_(255)
    ref = call()
    k, v, kr, vr = to_np(cache)
    want = oracle.decode_attention(q.cpu().numpy(), k, v, kr, vr, cache["C"], G, Nq, R, scale)
    check_attention(ref, want)
    work.zero_()
    assert np.array_equal(call(), ref)
    work.copy_(torch.randint(0, 256, (ws,), dtype=torch.uint8, device=DEV))
    assert np.array_equal(call(), ref)
    # fewer chunks (a shorter fill of the same cache) on the same workspace
    short = call(1024)
    assert np.isfinite(short).all() and not np.array_equal(short, ref)
    assert np.array_equal(call(), ref)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(Nq)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        launch(Nq)
    torch.cuda.synchronize()
    for i in range(3):
        assert np.array_equal(call(1024), short)      # eager work between replays
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), f"replay {i}"


def test_attention_repeated_calls_many_workgroups():
    """768 split workgroups (six chunks per head block, spread over every XCD)
    and the merge launch: 24 calls queued on one workspace alternate between
    two query sets, and every output is bit-identical to the first output of
    its query set -- a partial of the other set's call read by a merge would
    show.  The first outputs match the oracle on sampled heads."""
    B, Hq, Hkv, Nq, R, m, G = 16, 32, 8, 8192, 128, 4, 128
    print("attention: repeated calls, 768 workgroups", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=101, device_gen=True)
    scale = 1 / math.sqrt(128)
    p = cache["p"]
    ws = nsnq.nsn_decode_attention_workspace_size(p, B, Hq, Hkv, Nq, R, Nq, R, scale)
    work = torch.empty(ws, dtype=torch.uint8, device=DEV)
    qs = [synth.query_torch((B, Hq, 128), seed=102 + i, device=DEV) for i in range(2)]
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV) for _ in range(2)]

    def launch(i):
        outs[i].fill_(float("nan"))
        nsnq.nsn_decode_attention(p, qs[i], cache["k"], cache["v"], cache["kr"], cache["vr"],
                                  cache["table"], work, outs[i], Nq, R, scale)

    refs = []
    for i in range(2):
        launch(i)
        torch.cuda.synchronize()
        refs.append(outs[i].cpu().numpy())
    assert not np.array_equal(refs[0], refs[1])
    for b, h in [(0, 0), (9, 17), (B - 1, Hq - 1)]:
        kvh = h // (Hq // Hkv)
        sl = lambda t: t[b:b + 1, kvh:kvh + 1].cpu().numpy()  # noqa: E731
        k = tuple(sl(t) for t in cache["k"])
        v = tuple(sl(t) for t in cache["v"])
        for i in range(2):
            want = oracle.decode_attention(qs[i].cpu().numpy()[b:b + 1, h:h + 1], k, v, sl(cache["kr"]),
                                           sl(cache["vr"]), cache["C"], G, Nq, R, scale)
            check_attention(refs[i][b, h], want[0, 0], f"(b={b}, h={h}, q set {i})")
    for r in range(12):
        launch(0)
        launch(1)
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(outs[i].cpu().numpy(), refs[i]), f"round {r}, query set {i}"


@pytest.mark.parametrize("rope", [False, True])
def test_prepared_call_matches_per_call(rope):
    """A decode loop through PreparedDecodeAttention (tensors checked once,
    token counts and query position set per step) gives the bytes of the
    per-call function at every step; a missing q_pos with rotary keys and a
    count above the cache are refused."""
    B, Hq, Hkv, Nq, R, m, G = 2, 8, 2, 2048, 40, 4, 128
    print(f"prepared attention call, rope={rope}", flush=True)
    cache = build_cache(B, Hkv, Nq, R, m, G, seed=111, rcap=64)
    p = cache["p"]
    q = synth.query_torch((B, Hq, 128), seed=112, device=DEV)
    scale = 1 / math.sqrt(128)
    ws = nsnq.nsn_decode_attention_workspace_size(p, B, Hq, Hkv, Nq, 64, Nq, 64, scale)
    work = torch.empty(ws, dtype=torch.uint8, device=DEV)
    out_a = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    out_b = torch.empty_like(out_a)
    base = 10000.0
    call = nsnq.PreparedDecodeAttention(p, q, cache["k"], cache["v"], cache["kr"], cache["vr"],
                                        cache["table"], work, out_a, scale,
                                        rope_base=base if rope else None)
    for nq, r in [(0, 5), (128, 0), (640, 17), (1024, 40), (2048, 1), (2048, 40)]:
        q_pos = nq + r + 3
        out_a.fill_(float("nan"))
        out_b.fill_(float("nan"))
        call(nq, r, q_pos=q_pos if rope else None)
        if rope:
            nsnq.nsn_decode_attention_rope(p, q, cache["k"], cache["v"], cache["kr"], cache["vr"],
                                           cache["table"], work, out_b, nq, r, scale, q_pos, base)
        else:
            nsnq.nsn_decode_attention(p, q, cache["k"], cache["v"], cache["kr"], cache["vr"],
                                      cache["table"], work, out_b, nq, r, scale)
        torch.cuda.synchronize()
        a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.isfinite(a).all() and np.array_equal(a, b), (nq, r)
    if rope:
        with pytest.raises(ValueError):
            call(128, 0)
    with pytest.raises(nsnq.NsnError):
        call(Nq + G, 0, q_pos=Nq + G)
