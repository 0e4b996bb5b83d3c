"""Throughput of the NSNQuant hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the whole per-token path over one batch of synthetic
input, all through the C ABI of libnsn.so:
  * prefill quantize: K and V of batch 4 x 32 layers x 8 kv heads, 131072
    tokens each, head_dim 128, fp16, 2-bit codes (one launch over 2048
    sequences)                                   -- the dominant kernel
  * quantized decode attention: batch 16, 32 q heads on 8 kv heads,
    32768 quantized + 128 fp16 residual tokens (rotating over three cache
    copies so the 256 MB Infinity Cache cannot hold the working set)
  * streaming: 128 residual appends of one token per sequence (2048
    sequences) and the flush of the full residual into the cache
  * dequantize of the flushed group.
The codebook (k-means, 20 iterations on 65536 N(0,1) 4-vectors) is built
once on the GPU before the timed region and reported separately.

Prints ONE JSON line.  ``value`` is the step's algorithmic HBM bytes divided
by the step time (GB/s); per-kernel rates and the roofline of the dominant
kernel are attached.  The oracle (numpy float64) is timed on a bounded
sample of the same workload as ``cpu_baseline``.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
D = 128
COPY_CAL_BYTES = 1 << 30
ROPE_BASE = 10000.0          # rotary base of the rotary-key side measurement
QUANT_SRC = os.path.join(ROOT, "kv_cache_calibration_amd", "csrc", "quantize_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_mfma_prefill_hbm_bytes.txt")


DQ_REC = 136   # bytes of a double-quantized group record (G = 128)
TUNE_ITERS, TUNE_LR = 20, 3e-3


def side_ms(events):
    """Median launch time (ms) of a side measurement: its launches run on an
    otherwise idle stream, so one late launch must not move the figure."""
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in events]))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quant_bytes(n_seq, n_tok, m, G, in_bytes=2):
    return n_seq * n_tok * (D * in_bytes + D // m + 4) + n_seq * (n_tok // G) * D * 2


def quant_bytes_dq(n_seq, n_tok, m, G, in_bytes=2):
    """Double-quantized layout: s2' alone per token, one 136-byte record per group."""
    return n_seq * n_tok * (D * in_bytes + D // m + 2) + n_seq * (n_tok // G) * DQ_REC


def attn_bytes_dq(B, Hq, Hkv, Nq, R, m, G):
    per_tok = 2 * (D // m) + 2 * 2                 # K and V codes + s2'
    recs = 2 * (Nq // G) * DQ_REC                  # K and V group records
    resid = 2 * R * D * 2
    return B * Hkv * (Nq * per_tok + recs + resid) + B * Hq * D * (2 + 4)


def attn_bytes(B, Hq, Hkv, Nq, R, m, G):
    per_tok = 2 * (D // m) + 2 * 4                 # K and V codes + meta
    shift = 2 * (Nq // G) * D * 2                  # K and V group shifts
    resid = 2 * R * D * 2
    return B * Hkv * (Nq * per_tok + shift + resid) + B * Hq * D * (2 + 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=32,
                    help="layers of the prefill workload (32 = the full workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB read + 1 GiB write elementwise kernel before the "
                         "steps (a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the quantizer shards by sequence with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_calibration_amd as nsnq
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    G, m = 128, 4
    p = nsnq.Params(sub_dim=m, group_size=G)

    # -- a0: codebook on the GPU (one-time, outside the step)
    X = torch.from_numpy(synth.codebook_samples(m, 65536, seed=0)).to(dev)
    cb = torch.empty((256, m), dtype=torch.float32, device=dev)
    cws = torch.empty(nsnq.nsn_build_codebook_workspace_size(m, 65536), dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    nsnq.nsn_build_codebook(X, cb, cws, iters=20)
    e1.record()
    table = torch.empty(nsnq.nsn_table_size(p), dtype=torch.uint8, device=dev)
    nsnq.nsn_prepare_codebook(p, cb, table)
    torch.cuda.synchronize()
    codebook_ms = e0.elapsed_time(e1)
    log(f"codebook built in {codebook_ms:.1f} ms")
    # cosine fine-tuning of that codebook (one-time, outside the step; the
    # step keeps the k-means codebook): 2048 N(0,1) vectors of 128, the same
    # 262144 values k-means used, TUNE_ITERS full-batch Adam steps
    Hv = torch.from_numpy(synth.codebook_samples(D, 2048, seed=1)).to(dev)
    cbt = cb.clone()
    tws = torch.empty(nsnq.nsn_tune_codebook_workspace_size(m, 2048), dtype=torch.uint8, device=dev)
    e0.record()
    nsnq.nsn_tune_codebook(Hv, cbt, tws, TUNE_ITERS, TUNE_LR)
    e1.record()
    torch.cuda.synchronize()
    tune_ms = e0.elapsed_time(e1)
    del Hv, cbt, tws
    log(f"codebook fine-tuned in {tune_ms:.1f} ms ({TUNE_ITERS} iterations)")

    # -- prefill workload: K and V, batch 4 x layers x 8 heads, 131072 tokens
    w4 = synth.WORKLOADS["prefill"]
    L = args.layers
    per_layer = w4["B"] * w4["Hkv"]
    n_seq_t = per_layer * L                  # sequences per tensor
    T = w4["T"]
    n_seq = 2 * n_seq_t                      # K and V in one launch
    n_flush = 4                              # streaming phase: 512 appends, 4 flushes
    cap = T + n_flush * G                    # room for the streamed groups
    x = torch.empty((n_seq, T, D), dtype=torch.float16, device=dev)
    for layer in range(L):
        a, b = layer * per_layer, (layer + 1) * per_layer
        synth.kv_torch(per_layer, T, w4["outlier_scale"], w4["seed"] + layer, dev,
                       out_k=x[a:b], out_v=x[n_seq_t + a:n_seq_t + b])
    codes = torch.empty((n_seq, cap, D // m), dtype=torch.uint8, device=dev)
    meta = torch.empty((n_seq, cap, 2), dtype=torch.float16, device=dev)
    shift = torch.empty((n_seq, cap // G, D), dtype=torch.float16, device=dev)
    resid = torch.empty((n_seq, G, D), dtype=torch.float16, device=dev)
    newtok = torch.randn((G, n_seq, D), dtype=torch.float16, device=dev)
    deq = torch.empty((n_seq, G, D), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()
    log(f"prefill inputs ready: {n_seq} sequences x {T} tokens ({x.numel() * 2 / 1e9:.1f} GB)")

    # -- decode workload: three independent caches
    w3 = synth.WORKLOADS["decode"]
    B3, Hq, Hkv, Nq, R = w3["B"], w3["Hq"], w3["Hkv"], w3["Nq"], w3["R"]
    scale = 1.0 / math.sqrt(D)
    caches = []
    for c in range(3):
        K3, V3 = synth.kv_torch(B3 * Hkv, Nq + R, w3["outlier_scale"], w3["seed"] + 10 * c, dev)
        kc = torch.empty((B3, Hkv, Nq, D // m), dtype=torch.uint8, device=dev)
        km = torch.empty((B3, Hkv, Nq, 2), dtype=torch.float16, device=dev)
        ks = torch.empty((B3, Hkv, Nq // G, D), dtype=torch.float16, device=dev)
        vc, vm, vs = torch.empty_like(kc), torch.empty_like(km), torch.empty_like(ks)
        f = lambda t: t.view(B3 * Hkv, *t.shape[2:])  # noqa: E731
        nsnq.nsn_quantize(p, K3[:, :Nq], table, f(kc), f(km), f(ks))
        nsnq.nsn_quantize(p, V3[:, :Nq], table, f(vc), f(vm), f(vs))
        kr = K3[:, Nq:].contiguous().view(B3, Hkv, R, D)
        vr = V3[:, Nq:].contiguous().view(B3, Hkv, R, D)
        q = synth.query_torch((B3, Hq, D), seed=w3["seed"] + 10 * c + 1, device=dev)
        caches.append(((kc, km, ks), (vc, vm, vs), kr, vr, q))
        del K3, V3
    # the same decode shape with 1-bit codes (m = 8): a side measurement,
    # not part of the step
    m1 = 8
    p1 = nsnq.Params(sub_dim=m1, group_size=G)
    X1 = torch.from_numpy(synth.codebook_samples(m1, 262144, seed=0)).to(dev)
    cb1 = torch.empty((256, m1), dtype=torch.float32, device=dev)
    cws1 = torch.empty(nsnq.nsn_build_codebook_workspace_size(m1, 262144), dtype=torch.uint8,
                       device=dev)
    nsnq.nsn_build_codebook(X1, cb1, cws1, iters=20)
    table1 = torch.empty(nsnq.nsn_table_size(p1), dtype=torch.uint8, device=dev)
    nsnq.nsn_prepare_codebook(p1, cb1, table1)
    del X1, cws1
    caches1 = []
    for c in range(3):
        K3, V3 = synth.kv_torch(B3 * Hkv, Nq + R, w3["outlier_scale"], w3["seed"] + 10 * c, dev)
        kc = torch.empty((B3, Hkv, Nq, D // m1), dtype=torch.uint8, device=dev)
        km = torch.empty((B3, Hkv, Nq, 2), dtype=torch.float16, device=dev)
        ks = torch.empty((B3, Hkv, Nq // G, D), dtype=torch.float16, device=dev)
        vc, vm, vs = torch.empty_like(kc), torch.empty_like(km), torch.empty_like(ks)
        f = lambda t: t.view(B3 * Hkv, *t.shape[2:])  # noqa: E731
        nsnq.nsn_quantize(p1, K3[:, :Nq], table1, f(kc), f(km), f(ks))
        nsnq.nsn_quantize(p1, V3[:, :Nq], table1, f(vc), f(vm), f(vs))
        caches1.append(((kc, km, ks), (vc, vm, vs), caches[c][2], caches[c][3], caches[c][4]))
        del K3, V3
    ws_bytes = max(nsnq.nsn_decode_attention_workspace_size(p, B3, Hq, Hkv, Nq, R, Nq, R, scale),
                   nsnq.nsn_decode_attention_workspace_size(p1, B3, Hq, Hkv, Nq, R, Nq, R, scale))
    work = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B3, Hq, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("decode caches ready")

    if args.copy_calibration:
        src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: {COPY_CAL_BYTES} bytes read, {COPY_CAL_BYTES} bytes written")
        del src, dst

    names = ["quantize", "attention", "append", "flush", "dequantize"]
    ev = {k: [] for k in names}

    def step(i, record):
        def timed(name, fn):
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                ev[name].append((a, b))
            else:
                fn()
        timed("quantize", lambda: nsnq.nsn_quantize(p, x, table, codes, meta, shift))
        kc, vc, kr, vr, q = caches[i % 3]
        timed("attention", lambda: nsnq.nsn_decode_attention(p, q, kc, vc, kr, vr, table, work, out,
                                                             Nq, R, scale))

        def appends():
            for t in range(G):
                nsnq.nsn_residual_append(newtok[t], resid, t)
        timed("append", appends)
        timed("flush", lambda: nsnq.nsn_quantize(p, resid, table, codes[:, T:], meta[:, T:],
                                                 shift[:, T // G:]))
        timed("dequantize", lambda: nsnq.nsn_dequantize(p, codes[:, T:], meta[:, T:],
                                                        shift[:, T // G:], table, deq))

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
        log(f"step {i + 1}/{args.steps} issued")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in ev[k]])) for k in names}
    ms_step = wall * 1e3 / args.steps
    launch_stats = {}
    for k in names:
        v = np.array([a.elapsed_time(b) for a, b in ev[k]])
        launch_stats[k] = {"median_ms": float(np.median(v)), "p10_ms": float(np.percentile(v, 10)),
                           "p90_ms": float(np.percentile(v, 90)), "n": int(len(v))}

    # side measurement, outside the step: decode attention over 1-bit caches
    ev1 = []
    for i in range(max(args.steps, 3) + 1):
        kc1, vc1, kr1, vr1, q1 = caches1[i % 3]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_decode_attention(p1, q1, kc1, vc1, kr1, vr1, table1, work, out, Nq, R, scale)
        b.record(stream)
        if i > 0:
            ev1.append((a, b))
    torch.cuda.synchronize()
    ms_attn1 = side_ms(ev1)

    # side measurement, outside the step: the 2-bit decode attention with the
    # keys stored before rotary embedding (query at the last residual position)
    evr = []
    for i in range(max(args.steps, 3) + 1):
        kc, vc, kr, vr, q = caches[i % 3]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_decode_attention_rope(p, q, kc, vc, kr, vr, table, work, out, Nq, R, scale,
                                       Nq + R - 1, ROPE_BASE)
        b.record(stream)
        if i > 0:
            evr.append((a, b))
    torch.cuda.synchronize()
    ms_attn_rope = side_ms(evr)

    # side measurement, outside the step: the same prefill quantize with
    # 1-bit codes (its metadata and shifts overwrite the step's outputs)
    codes1 = torch.empty((n_seq, cap, D // m1), dtype=torch.uint8, device=dev)
    evq1 = []
    for i in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_quantize(p1, x, table1, codes1, meta, shift)
        b.record(stream)
        if i > 0:
            evq1.append((a, b))
    torch.cuda.synchronize()
    ms_q1 = side_ms(evq1)
    del codes1

    # side measurements, outside the step: double-quantized metadata (4-bit
    # s1 and rotated shift in one record per group, 4-bit codebook entries),
    # the prefill quantize (its codes overwrite the step's) and the decode
    # attention, same shapes
    pq = nsnq.Params(sub_dim=m, group_size=G, dq=True)
    tableq = torch.empty(nsnq.nsn_table_size(pq), dtype=torch.uint8, device=dev)
    nsnq.nsn_prepare_codebook(pq, cb, tableq)
    meta_q = torch.empty((n_seq, cap), dtype=torch.float16, device=dev)
    recs_q = torch.empty((n_seq, cap // G, DQ_REC), dtype=torch.uint8, device=dev)
    evqd = []
    for i in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_quantize(pq, x, tableq, codes, meta_q, recs_q)
        b.record(stream)
        if i > 0:
            evqd.append((a, b))
    torch.cuda.synchronize()
    ms_qdq = side_ms(evqd)
    del meta_q, recs_q
    cachesq = []
    for c in range(3):
        K3, V3 = synth.kv_torch(B3 * Hkv, Nq + R, w3["outlier_scale"], w3["seed"] + 10 * c, dev)
        kc = torch.empty((B3, Hkv, Nq, D // m), dtype=torch.uint8, device=dev)
        km = torch.empty((B3, Hkv, Nq), dtype=torch.float16, device=dev)
        ks = torch.empty((B3, Hkv, Nq // G, DQ_REC), dtype=torch.uint8, device=dev)
        vc, vm, vs = torch.empty_like(kc), torch.empty_like(km), torch.empty_like(ks)
        f = lambda t: t.view(B3 * Hkv, *t.shape[2:])  # noqa: E731
        nsnq.nsn_quantize(pq, K3[:, :Nq], tableq, f(kc), f(km), f(ks))
        nsnq.nsn_quantize(pq, V3[:, :Nq], tableq, f(vc), f(vm), f(vs))
        cachesq.append(((kc, km, ks), (vc, vm, vs), caches[c][2], caches[c][3], caches[c][4]))
        del K3, V3
    evad = []
    for i in range(max(args.steps, 3) + 1):
        kcq, vcq, krq, vrq, qq = cachesq[i % 3]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_decode_attention(pq, qq, kcq, vcq, krq, vrq, tableq, work, out, Nq, R, scale)
        b.record(stream)
        if i > 0:
            evad.append((a, b))
    torch.cuda.synchronize()
    ms_attn_dq = side_ms(evad)
    # the same double-quantized caches read as keys stored before rotary
    # embedding (query at the last residual position)
    evadr = []
    for i in range(max(args.steps, 3) + 1):
        kcq, vcq, krq, vrq, qq = cachesq[i % 3]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_decode_attention_rope(pq, qq, kcq, vcq, krq, vrq, tableq, work, out, Nq, R, scale,
                                       Nq + R - 1, ROPE_BASE)
        b.record(stream)
        if i > 0:
            evadr.append((a, b))
    torch.cuda.synchronize()
    ms_attn_dq_rope = side_ms(evadr)
    del cachesq

    # side measurements, outside the step: the randomized Hadamard rotation
    # (one seeded draw of channel signs), the prefill quantize (its outputs
    # overwrite the step's) and the decode attention over caches quantized
    # with the same signs, same shapes
    pr = nsnq.Params(sub_dim=m, group_size=G, rht_signs=synth.rht_signs(w4["seed"]))
    evqr = []
    for i in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_quantize(pr, x, table, codes, meta, shift)
        b.record(stream)
        if i > 0:
            evqr.append((a, b))
    torch.cuda.synchronize()
    ms_q_rht = side_ms(evqr)
    cachesr = []
    for c in range(3):
        K3, V3 = synth.kv_torch(B3 * Hkv, Nq + R, w3["outlier_scale"], w3["seed"] + 10 * c, dev)
        kc = torch.empty((B3, Hkv, Nq, D // m), dtype=torch.uint8, device=dev)
        km = torch.empty((B3, Hkv, Nq, 2), dtype=torch.float16, device=dev)
        ks = torch.empty((B3, Hkv, Nq // G, D), dtype=torch.float16, device=dev)
        vc, vm, vs = torch.empty_like(kc), torch.empty_like(km), torch.empty_like(ks)
        f = lambda t: t.view(B3 * Hkv, *t.shape[2:])  # noqa: E731
        nsnq.nsn_quantize(pr, K3[:, :Nq], table, f(kc), f(km), f(ks))
        nsnq.nsn_quantize(pr, V3[:, :Nq], table, f(vc), f(vm), f(vs))
        cachesr.append(((kc, km, ks), (vc, vm, vs), caches[c][2], caches[c][3], caches[c][4]))
        del K3, V3
    evar = []
    for i in range(max(args.steps, 3) + 1):
        kcr, vcr, krr, vrr, qr = cachesr[i % 3]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        nsnq.nsn_decode_attention(pr, qr, kcr, vcr, krr, vrr, table, work, out, Nq, R, scale)
        b.record(stream)
        if i > 0:
            evar.append((a, b))
    torch.cuda.synchronize()
    ms_attn_rht = side_ms(evar)
    del cachesr

    # side measurement, outside the step: the prefill workload's streaming
    # phase at full size -- 512 decode steps, each appending one token per
    # sequence (2048 sequences, K and V) to the residual window, the window
    # flushed into the cache behind the prefill every 128 steps (4 flushes)
    n_app = n_flush * G
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evf = []
    ea.record(stream)
    for t in range(n_app):
        nsnq.nsn_residual_append(newtok[t % G], resid, t % G)
        if (t + 1) % G == 0:
            off = T + (t // G) * G
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            nsnq.nsn_quantize(p, resid, table, codes[:, off:], meta[:, off:], shift[:, off // G:])
            b.record(stream)
            evf.append((a, b))
    eb.record(stream)
    torch.cuda.synchronize()
    stream_ms = ea.elapsed_time(eb)
    flush_ms = [a.elapsed_time(b) for a, b in evf]
    # the same phase with each token buffer's append prepared once (the
    # binding's checks and marshalling outside the loop, as a serving loop
    # with fixed buffers would do)
    prepared = [nsnq.PreparedResidualAppend(newtok[i], resid) for i in range(G)]
    ea2, eb2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea2.record(stream)
    for t in range(n_app):
        prepared[t % G](t % G)
        if (t + 1) % G == 0:
            off = T + (t // G) * G
            nsnq.nsn_quantize(p, resid, table, codes[:, off:], meta[:, off:], shift[:, off // G:])
    eb2.record(stream)
    torch.cuda.synchronize()
    stream_prep_ms = ea2.elapsed_time(eb2)
    del prepared
    streaming = {
        "appends": n_app, "flushes": n_flush, "sequences": n_seq,
        "phase_ms": stream_ms,
        "per_append_us": (stream_ms - sum(flush_ms)) * 1e3 / n_app,
        "flush_ms": flush_ms,
        "decode_positions_per_s": n_app / (stream_ms * 1e-3),
        "bytes": n_app * n_seq * D * 2 * 2 + n_flush * quant_bytes(n_seq, G, m, G),
        "note": "launch-bound (one append launch per position): not a roofline measurement",
        "phase_ms_prepared_appends": stream_prep_ms,
        "per_append_us_prepared": (stream_prep_ms - sum(flush_ms)) * 1e3 / n_app,
    }
    streaming["gbps"] = streaming["bytes"] / (stream_ms * 1e-3) / 1e9
    log(f"streaming phase: {n_app} appends + {n_flush} flushes in {stream_ms:.2f} ms "
        f"({stream_prep_ms:.2f} ms with prepared appends)")

    # side measurements, outside the step: the three small workloads, each
    # exactly as stated (launch-bound, reported for completeness)
    small = small_workloads(nsnq, synth, table, table1, cb, dev, stream)

    qb = quant_bytes(n_seq, T, m, G)
    ab = attn_bytes(B3, Hq, Hkv, Nq, R, m, G)
    app_b = G * n_seq * D * 2 * 2
    fb = quant_bytes(n_seq, G, m, G)
    db = n_seq * G * (D * 2 + D // m + 4) + n_seq * D * 2
    step_bytes = qb + ab + app_b + fb + db
    value = step_bytes / (ms_step * 1e-3) / 1e9
    rates = {
        "quantize_gbps": qb / (ms["quantize"] * 1e-3) / 1e9,
        "quantize_fp16_in_gbps": n_seq * T * D * 2 / (ms["quantize"] * 1e-3) / 1e9,
        "quantize_token_heads_per_s": n_seq * T / (ms["quantize"] * 1e-3),
        "attention_gbps": ab / (ms["attention"] * 1e-3) / 1e9,
        "attention_1bit_gbps": attn_bytes(B3, Hq, Hkv, Nq, R, m1, G) / (ms_attn1 * 1e-3) / 1e9,
        "attention_1bit_ms": ms_attn1,
        "attention_query_tokens_per_s": B3 / (ms["attention"] * 1e-3),
        "attention_rope_gbps": ab / (ms_attn_rope * 1e-3) / 1e9,
        "attention_rope_ms": ms_attn_rope,
        "quantize_1bit_gbps": quant_bytes(n_seq, T, m1, G) / (ms_q1 * 1e-3) / 1e9,
        "quantize_1bit_ms": ms_q1,
        "quantize_dq_gbps": quant_bytes_dq(n_seq, T, m, G) / (ms_qdq * 1e-3) / 1e9,
        "quantize_dq_ms": ms_qdq,
        "attention_dq_gbps": attn_bytes_dq(B3, Hq, Hkv, Nq, R, m, G) / (ms_attn_dq * 1e-3) / 1e9,
        "attention_dq_ms": ms_attn_dq,
        "attention_dq_rope_gbps": attn_bytes_dq(B3, Hq, Hkv, Nq, R, m, G) / (ms_attn_dq_rope * 1e-3) / 1e9,
        "attention_dq_rope_ms": ms_attn_dq_rope,
        "quantize_rht_gbps": qb / (ms_q_rht * 1e-3) / 1e9,
        "quantize_rht_ms": ms_q_rht,
        "attention_rht_gbps": ab / (ms_attn_rht * 1e-3) / 1e9,
        "attention_rht_ms": ms_attn_rht,
        "flush_gbps": fb / (ms["flush"] * 1e-3) / 1e9,
        "dequantize_gbps": db / (ms["dequantize"] * 1e-3) / 1e9,
        # sequence positions of the prefill (batch 4 x 131072) per second:
        # every position is 32 layers x 8 kv heads x (K, V) token-heads
        "prefill_positions_per_s": w4["B"] * T / (ms["quantize"] * 1e-3) * (32 / L),
    }
    rates["quantize_frac_hbm"] = rates["quantize_gbps"] / HBM_PEAK_GBPS
    rates["attention_frac_hbm"] = rates["attention_gbps"] / HBM_PEAK_GBPS
    rates["attention_1bit_frac_hbm"] = rates["attention_1bit_gbps"] / HBM_PEAK_GBPS
    rates["quantize_1bit_frac_hbm"] = rates["quantize_1bit_gbps"] / HBM_PEAK_GBPS
    rates["attention_rope_frac_hbm"] = rates["attention_rope_gbps"] / HBM_PEAK_GBPS
    rates["quantize_dq_frac_hbm"] = rates["quantize_dq_gbps"] / HBM_PEAK_GBPS
    rates["attention_dq_frac_hbm"] = rates["attention_dq_gbps"] / HBM_PEAK_GBPS
    rates["attention_dq_rope_frac_hbm"] = rates["attention_dq_rope_gbps"] / HBM_PEAK_GBPS
    rates["quantize_rht_frac_hbm"] = rates["quantize_rht_gbps"] / HBM_PEAK_GBPS
    rates["attention_rht_frac_hbm"] = rates["attention_rht_gbps"] / HBM_PEAK_GBPS
    log("kernel ms: " + ", ".join(f"{k} {v:.3f}" for k, v in ms.items()))
    log("rates: " + ", ".join(f"{k} {v:.4g}" for k, v in rates.items()))

    roofline = {
        "bound": "hbm",
        "kernel": "quantize_mfma_kernel (prefill launch)",
        "achieved": rates["quantize_gbps"],
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": rates["quantize_gbps"] / HBM_PEAK_GBPS,
        "traffic": None,
        "bytes_per_launch": qb,
        "avg_launch_ms": ms["quantize"],
    }

    tr = measured_traffic(QUANT_SRC, qb)
    if tr is not None:
        roofline["traffic"] = tr["bytes_per_launch"]              # HBM bytes per launch
        roofline["traffic_unit"] = "bytes per launch"
        roofline["traffic_gbps"] = tr["bytes_per_launch"] / (ms["quantize"] * 1e-3) / 1e9
        roofline["traffic_detail"] = tr

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, caches[0], G, m, cb.cpu().numpy(), cb1.cpu().numpy(), qb, ab, R, Nq,
                           scale, step_bytes, n_seq, synth)

    line = {
        "metric": "KV quantize GB/s (fp16 in) + quantized decode-attn GB/s, % of HBM roofline",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"prefill quantize {n_seq_t}x2 seqs x {T} tok fp16 2-bit G={G} "
                         f"({L} layers x 4 batch x 8 kv heads) + decode attention B={B3} "
                         f"Hq={Hq} Hkv={Hkv} {Nq}+{R} tok + 128 appends, flush, dequantize"),
            "head_dim": D, "sub_dim": m, "group_size": G,
            "step_bytes": step_bytes,
        },
        "kernel_ms": ms,
        "launch_stats": launch_stats,
        "gpu_clocks": gpu_clocks(),
        "rates": rates,
        "codebook_build_ms": codebook_ms,
        "codebook_tune_ms": tune_ms,
        "codebook_tune_iters": TUNE_ITERS,
        "roofline": roofline,
        "streaming": streaming,
        "small_workloads": small,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def gpu_clocks():
    """Current clock levels as rocm-smi reports them (best effort)."""
    import shutil
    import subprocess
    if "rocprofiler" in os.environ.get("LD_PRELOAD", "") or any(
            k.startswith("ROCPROF") for k in os.environ):
        return None   # under a profiler: no child processes
    exe = shutil.which("rocm-smi")
    if exe is None:
        return None
    try:
        # run the script with this interpreter (no /usr/bin/env hop)
        r = subprocess.run([sys.executable, os.path.realpath(exe), "--showclocks"],
                           capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    lines = [ln.strip() for ln in r.stdout.splitlines() if "Mhz" in ln or "MHz" in ln]
    return lines[:8] or None


def measured_traffic(src_path, algorithmic_bytes):
    """HBM bytes per launch of the dominant kernel, from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by a plain copy of known size);
    None when that summary was taken on another version of the kernel source
    or for another launch size."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
        with open(src_path, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get("source_sha256", "").strip() != sha:
            return None
        if int(kv["algorithmic_bytes_per_launch"]) != int(algorithmic_bytes):
            return None
        return {"bytes_per_launch": float(kv["hbm_bytes_per_launch"]),
                "read_bytes_per_launch": float(kv["read_bytes_per_launch"]),
                "write_bytes_per_launch": float(kv["write_bytes_per_launch"]),
                "ratio_to_algorithmic": float(kv["hbm_bytes_per_launch"]) / algorithmic_bytes,
                "source": os.path.relpath(TRAFFIC_FILE, ROOT)}
    except (OSError, KeyError, ValueError):
        return None


def small_workloads(nsnq, synth, table2, table1, cb2, dev, stream):
    """Quantize (+ dequantize) of the tiny, 2-bit layer and 1-bit layer
    workloads at their stated sizes: median of 20 launches each, with the
    Infinity Cache and L2 evicted before each (512 MiB written).  These are
    too small to fill the chip (the tiny one is two workgroups) and take
    microseconds, so launch latency dominates: reported for completeness,
    not as roofline measurements."""
    import numpy as np
    import torch
    out = {}
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for name in ("tiny", "layer2b", "layer1b"):
        w = synth.WORKLOADS[name]
        G, m = w["G"], w["m"]
        f32 = w["dtype"] == "f32"
        K, V = synth.kv_numpy(w["n_seq"], w["T"], w["outlier_scale"], seed=w["seed"],
                              dtype=np.float32 if f32 else np.float16)
        x = torch.from_numpy(np.concatenate([K, V])).to(dev)
        n_seq, T = x.shape[0], x.shape[1]
        if name == "tiny":
            p = nsnq.Params(sub_dim=m, group_size=G)
            table = torch.empty(nsnq.nsn_table_size(p), dtype=torch.uint8, device=dev)
            nsnq.nsn_prepare_codebook(p, cb2, table)
        else:
            p = nsnq.Params(sub_dim=m, group_size=G)
            table = table2 if m == 4 else table1
        codes, meta, shift = (torch.empty(sh, dtype=dt, device=dev) for sh, dt in nsnq.cache_layout(p, n_seq, T))
        xh = torch.empty_like(x)
        evq, evd = [], []
        for i in range(21):
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            evict.fill_(i & 255)
            a.record(stream)
            nsnq.nsn_quantize(p, x, table, codes, meta, shift)
            b.record(stream)
            nsnq.nsn_dequantize(p, codes, meta, shift, table, xh)
            c.record(stream)
            if i:
                evq.append((a, b))
                evd.append((b, c))
        torch.cuda.synchronize()
        qms, dms = side_ms(evq), side_ms(evd)
        ib = 4 if f32 else 2
        qbytes = quant_bytes(n_seq, T, m, G, ib)
        dbytes = n_seq * T * (D * ib + D // m + 4) + n_seq * (T // G) * D * 2
        out[name] = {
            "shape": f"{n_seq} seqs x {T} tok, {'fp32' if f32 else 'fp16'}, m={m}, G={G}",
            "quantize_ms": qms, "quantize_gbps": qbytes / (qms * 1e-3) / 1e9,
            "dequantize_ms": dms, "dequantize_gbps": dbytes / (dms * 1e-3) / 1e9,
            "quantize_token_heads_per_s": n_seq * T / (qms * 1e-3),
            "note": "latency-bound at this size, not a roofline measurement (cold Infinity Cache)",
        }
        log(f"{name}: quantize {qms * 1e3:.1f} us, dequantize {dms * 1e3:.1f} us")
    del evict
    return out


def cpu_baseline(x, cache, G, m, C, C1, qb, ab, R, Nq, scale, step_bytes, n_seq_prefill, synth):
    """Time the oracle (numpy float64, as it stands) on the host:
      * the three small workloads whole (quantize + dequantize of every
        sequence);
      * the decode workload whole (every (batch, kv head) row: dequantize the
        cache and attend with its 4 query heads);
      * the prefill: one of the 16 sequences of a (batch, layer) slice,
        extrapolated x16 to the slice and x128 to the whole prefill, plus
        128 of the 2048 sequences of a flush, extrapolated x16.
    The step's CPU time adds the extrapolated prefill, the decode call, the
    flush and the dequantize of the flushed group (appends are copies and
    are not timed).  About 20-30 s of host work."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    affinity = len(os.sched_getaffinity(0))
    cores = blas_threads if blas_threads else 1
    out = {}
    # -- the small workloads, whole
    for name in ("tiny", "layer2b", "layer1b"):
        w = synth.WORKLOADS[name]
        f32 = w["dtype"] == "f32"
        K, V = synth.kv_numpy(w["n_seq"], w["T"], w["outlier_scale"], seed=w["seed"],
                              dtype=np.float32 if f32 else np.float16)
        xs = np.concatenate([K, V]).astype(np.float64)
        Cw = C if w["m"] == 4 else C1
        t0 = time.perf_counter()
        for sq in range(xs.shape[0]):
            co, mo, so = oracle.quantize(xs[sq], Cw, w["G"])
            oracle.dequantize(co, mo, so, Cw, w["G"])
        dt = time.perf_counter() - t0
        nb = quant_bytes(xs.shape[0], w["T"], w["m"], w["G"], 4 if f32 else 2)
        out[name] = {"seconds": dt, "quantize_dequantize_gbps": nb / dt / 1e9}
        log(f"cpu oracle {name}: {dt:.2f} s")
    # -- the decode workload, whole
    kc, vc, kr, vr, q = cache
    B3, Hkv = kc[0].shape[0], kc[0].shape[1]
    Hq = q.shape[1]
    grp = Hq // Hkv
    kcn = tuple(t.cpu().numpy() for t in kc)
    vcn = tuple(t.cpu().numpy() for t in vc)
    krn, vrn, qn = kr.cpu().numpy(), vr.cpu().numpy(), q.cpu().numpy()
    t0 = time.perf_counter()
    for b in range(B3):
        for h in range(Hkv):
            sl = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
            oracle.decode_attention(qn[b:b + 1, h * grp:(h + 1) * grp], tuple(sl(t) for t in kcn),
                                    tuple(sl(t) for t in vcn), sl(krn), sl(vrn), C, G, Nq, R, scale)
    ta = time.perf_counter() - t0
    out["decode"] = {"seconds": ta, "gbps": ab / ta / 1e9}
    log(f"cpu oracle decode workload: {ta:.2f} s")
    # -- prefill: one sequence of a (batch, layer) slice, then x16 x128
    T = x.shape[1]
    xs = x[0].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    oracle.quantize(xs, C, G)
    tq1 = time.perf_counter() - t0
    tq = tq1 * n_seq_prefill
    out["prefill_sample"] = {"seconds_one_sequence": tq1, "sequence_tokens": T,
                             "slice_seconds_extrapolated": tq1 * 16,
                             "prefill_seconds_extrapolated": tq}
    log(f"cpu oracle prefill: one sequence of {T} tokens in {tq1:.2f} s")
    # -- flush: 128 of the 2048 sequences, then x16; dequantize of the same
    nf = 128
    xf = x[:nf, T - G:].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    res = [oracle.quantize(xf[sq], C, G) for sq in range(nf)]
    tf = (time.perf_counter() - t0) * (n_seq_prefill / nf)
    t0 = time.perf_counter()
    for co, mo, so in res:
        oracle.dequantize(co, mo, so, C, G)
    tdq = (time.perf_counter() - t0) * (n_seq_prefill / nf)
    step_s = tq + ta + tf + tdq
    return {
        "value": step_bytes / step_s / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "blas_threads": blas_threads,
        "host_cores_available": affinity,
        "kind": "oracle",
        "sample": ("small workloads and the decode workload whole; prefill from one of its 2048 "
                   f"sequences ({tq1:.1f} s, x{n_seq_prefill}); flush and dequantize from {nf} of its "
                   f"2048 sequences (x{n_seq_prefill // nf}); step time = sum of the parts"),
        "quantize_gbps": qb / tq / 1e9,
        "attention_gbps": ab / ta / 1e9,
        "step_seconds": step_s,
        "parts": out,
    }


if __name__ == "__main__":
    main()
