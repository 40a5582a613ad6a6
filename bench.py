#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache codec on one MI355X.

One step = one pass of the hot path over the Llama-3-8B-shaped cache
(32 layers x {K,V} x batch 4 x 8 KV heads x 8192 tokens = 16,777,216 vectors
of head_dim 128, fp16, 4 GiB; N(0,1) with 1% x15 outlier channels per
(layer, K/V, head)), 4 bits: tq_encode of the whole cache (one launch), then
tq_decode of it (one launch).  Inputs are resident in HBM before timing.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --attn-only [--steps K] [--head-dim D]
                                                (attention side measurement only;
                                                 D = 64, 128 (default) or 256)

Prints one JSON line.  `value` is fp16 key/value bytes passed through the
codec per second (encode and decode both count their 256 B/vector of fp16).
`roofline` rates the slower of the two kernels by its algorithmic bytes
(256 B fp16 + 64 B codes + 4 B norm per vector) against the 8 TB/s HBM peak.
`cpu_baseline` is the plain CPU oracle timed on this host's cores on a
bounded sample of the same cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
D = 128
BITS = 4
CODE_BYTES = D * BITS // 8
ALGO_BYTES = 2 * D + CODE_BYTES + 4          # per vector, per direction
LAYERS, PER_LAYER = 32, 2 * 4 * 8 * 8192
N = LAYERS * PER_LAYER


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def source_digest() -> str:
    """Digest of the codec kernel sources the counters were taken on."""
    h = hashlib.sha256()
    for f in ("tq_codec.hip", "tq_internal.h"):
        with open(os.path.join(ROOT, "kv_cache_vector_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def cpu_baseline(x_host, budget_s: float = 10.0, chunk: int = 2048):
    """The oracle (encode + decode) on consecutive 2048-vector chunks of layers
    0-1 of the cache, on up to 16 host threads, for ~budget_s seconds."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    o = oracle.default()
    threads = max(1, min(16, os.cpu_count() or 1))
    nchunks = x_host.shape[0] // chunk
    lock = threading.Lock()
    state = {"next": 0, "done": 0}
    deadline = [0.0]

    def worker():
        while True:
            with lock:
                if time.perf_counter() > deadline[0] or state["next"] >= nchunks:
                    return
                i = state["next"]
                state["next"] += 1
            xs = x_host[i * chunk:(i + 1) * chunk]
            p, n = o.encode(xs, BITS, 0)
            o.decode(p, n, D, BITS, 0)
            with lock:
                state["done"] += 1

    t0 = time.perf_counter()
    deadline[0] = t0 + budget_s
    ts = [threading.Thread(target=worker) for _ in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    wall = time.perf_counter() - t0
    nvec = state["done"] * chunk
    value = 2 * nvec * 2 * D / wall / 1e9
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "encode+decode of the first %d vectors of layers 0-1 (4 bits), %d threads, "
                      "%.1f s wall; %s" % (nvec, threads, wall, cpu)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the attention and streaming-encode side measurements")
    ap.add_argument("--head-dim", type=int, default=128, choices=(64, 128, 256),
                    help="head_dim of the --attn-only measurement")
    ap.add_argument("--attn-only", action="store_true",
                    help="only the batch-16 x 32K decode-attention measurement (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the codec is data-parallel over independent "
              "vectors, and its figures are one MI355X's (use --gpus 1)", file=sys.stderr)
        return 2
    if args.attn_only:
        import torch
        from kv_cache_vector_amd import _lib
        _lib.load()
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        res = attention_measurement(torch, dev, torch.cuda.current_stream(dev),
                                    reps=max(1, args.steps), head_dim=args.head_dim)
        print(json.dumps(res), flush=True)
        return 0

    import numpy as np
    import torch

    from kv_cache_vector_amd import _lib
    from kv_cache_vector_amd import workloads as W

    _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream

    log("generating the 8B-shaped cache: %d vectors (%.2f GB fp16)" % (N, N * 2 * D / 1e9))
    x = torch.empty((N, D), dtype=torch.float16, device=dev)
    host_sample = []
    for layer in range(LAYERS):
        xl = W.llama8b_layer(layer)
        if layer < 2:
            host_sample.append(xl)
        x[layer * PER_LAYER:(layer + 1) * PER_LAYER].copy_(torch.from_numpy(xl))
        if layer % 8 == 7:
            log("  layer %d/%d uploaded" % (layer + 1, LAYERS))
    packed = torch.empty((N, CODE_BYTES), dtype=torch.uint8, device=dev)
    norms = torch.empty((N,), dtype=torch.float32, device=dev)
    out = torch.empty((N, D), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()

    def enc():
        _lib.check(_lib.tq_encode(x.data_ptr(), N, D, BITS, 0, packed.data_ptr(),
                                  norms.data_ptr(), s), "tq_encode")

    def dec():
        _lib.check(_lib.tq_decode(packed.data_ptr(), norms.data_ptr(), N, D, BITS, 0,
                                  out.data_ptr(), s), "tq_decode")

    for _ in range(args.warmup):
        enc()
        dec()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(K):
        ev[k][0].record(stream)
        enc()
        ev[k][1].record(stream)
        dec()
        ev[k][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    enc_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    ms_step = total_ms / K
    value = 2 * N * 2 * D / (ms_step * 1e-3) / 1e9

    enc_avg, dec_avg = statistics.mean(enc_ms), statistics.mean(dec_ms)
    kern, t_ms = ("encode_kernel<4>", enc_avg) if enc_avg >= dec_avg else ("decode_kernel<4>", dec_avg)
    achieved = N * ALGO_BYTES / (t_ms * 1e-3) / 1e9
    traffic = measured_traffic(kern)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "kernel": kern,
                "algorithmic_bytes_per_launch": N * ALGO_BYTES}

    extra = {
        "encode_ms": round(enc_avg, 4), "decode_ms": round(dec_avg, 4),
        "encode_min_ms": round(min(enc_ms), 4), "decode_min_ms": round(min(dec_ms), 4),
        "encode_fp16_GBps": round(N * 2 * D / (enc_avg * 1e-3) / 1e9, 1),
        "decode_fp16_GBps": round(N * 2 * D / (dec_avg * 1e-3) / 1e9, 1),
        "encode_hbm_frac": round(N * ALGO_BYTES / (enc_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decode_hbm_frac": round(N * ALGO_BYTES / (dec_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "host_wall_s": round(wall, 3),
    }
    # achievable-bandwidth reference: a device-to-device copy of the fp16 cache
    cp = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out.copy_(x)
    cp[0].record(stream)
    for _ in range(5):
        out.copy_(x)
    cp[1].record(stream)
    torch.cuda.synchronize()
    cms = cp[0].elapsed_time(cp[1]) / 5
    extra["copy_GBps"] = round(2 * N * 2 * D / (cms * 1e-3) / 1e9, 1)

    if not args.no_extras:
        del out
        extra.update(side_measurements(torch, dev, stream, x, packed, norms))

    res = {
        "metric": "fp16-KV GB/s encoded/decoded (+% of HBM peak), 4-bit d=128, 1 MI355X",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped KV cache, 32 layers x {K,V} x batch 4 x "
                               "8 KV heads x 8192 tokens x 128 (16,777,216 vectors), N(0,1) "
                               "with 1% x15 outlier channels; bits=4, codec seed 0; "
                               "step = tq_encode + tq_decode of the whole cache",
                   "vectors": N, "head_dim": D, "bits": BITS, "hbm_frac_of_value":
                       round(value / HBM_PEAK_GBPS * ALGO_BYTES / (2 * D), 4)},
        "roofline": roofline,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(np.concatenate(host_sample))
    print(json.dumps(res), flush=True)
    return 0


def side_measurements(torch, dev, stream, x, packed, norms):
    """Decode attention at batch 16, 32/8 heads, 32768 tokens (4 bits, random
    codes), and a 2-bit encode launch the size of one 70B-class 128K-context
    layer (2,097,152 vectors; timed on the first vectors of the resident
    cache, the launch shape of the layer-by-layer streaming encode)."""
    res = attention_measurement(torch, dev, stream)
    res.update(stream_encode_measurement(torch, dev, stream, x, packed, norms))
    res.update(codec_side_measurement(torch, dev, stream, x, packed, norms))
    return res


def _median_min(times):
    return statistics.median(times), min(times)


def codec_side_measurement(torch, dev, stream, x, packed, norms):
    """Other codec launch shapes on the resident cache (timing does not depend
    on the values):
      - 3- and 2-bit encode and decode of the whole 16,777,216-vector cache;
      - 4-bit encode and decode of one layer (524,288 vectors), cache evicted
        before each launch;
      - 4-bit encode and decode latency of 4,096 vectors (cache-resident);
      - latency of the paged write path (tq_encode_paged, 4 bits): the new K
        rows of one decode step at batch 16 x 8 kv heads (128 vectors), and
        the new K and V rows of all 32 layers (8,192 vectors), each scattered
        into distinct random rows of the resident cache."""
    from kv_cache_vector_amd import _lib
    s = stream.cuda_stream
    res = {}
    out = torch.empty_like(x)
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

    def timed(fn, reps, evict):
        fn()
        times = []
        for _ in range(reps):
            if evict:
                flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return _median_min(times)

    def enc(n, bits, pk):
        return lambda: _lib.check(_lib.tq_encode(x.data_ptr(), n, D, bits, 0, pk.data_ptr(),
                                                 norms.data_ptr(), s), "tq_encode")

    def dec(n, bits, pk):
        return lambda: _lib.check(_lib.tq_decode(pk.data_ptr(), norms.data_ptr(), n, D, bits, 0,
                                                 out.data_ptr(), s), "tq_decode")

    for bits in (3, 2):
        P = D * bits // 8
        pk = packed.view(-1)[: N * P].view(N, P)
        for name, fn in (("encode", enc(N, bits, pk)), ("decode", dec(N, bits, pk))):
            med, mn = timed(fn, 5, False)
            res["%s_b%d_ms" % (name, bits)] = round(med, 4)
            res["%s_b%d_min_ms" % (name, bits)] = round(mn, 4)
            res["%s_b%d_hbm_frac" % (name, bits)] = round(
                N * (2 * D + P + 4) / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    n = PER_LAYER
    for name, fn in (("encode", enc(n, BITS, packed)), ("decode", dec(n, BITS, packed))):
        med, mn = timed(fn, 10, True)
        res["%s_layer_us" % name] = round(med * 1e3, 1)
        res["%s_layer_hbm_frac" % name] = round(
            n * ALGO_BYTES / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    n = 4096
    for name, fn in (("encode", enc(n, BITS, packed)), ("decode", dec(n, BITS, packed))):
        med, mn = timed(fn, 20, False)
        res["%s_4096_vectors_us" % name] = round(med * 1e3, 1)
        res["%s_4096_vectors_min_us" % name] = round(mn * 1e3, 1)
    gen = torch.Generator(device=dev).manual_seed(7)
    rows = torch.randperm(N, device=dev, generator=gen)
    for n in (128, 8192):
        slots = rows[:n].contiguous()

        def paged(n=n, slots=slots):
            _lib.check(_lib.tq_encode_paged(x.data_ptr(), slots.data_ptr(), n, D, BITS, 0,
                                            packed.data_ptr(), norms.data_ptr(), N, s),
                       "tq_encode_paged")
        med, mn = timed(paged, 20, False)
        res["encode_paged_%d_us" % n] = round(med * 1e3, 1)
        res["encode_paged_%d_min_us" % n] = round(mn * 1e3, 1)
    del rows
    return res


def attention_measurement(torch, dev, stream, reps: int = 10, head_dim: int = 128):
    """Median time of tq_attn_decode (split + combine kernels) at batch 16,
    32/8 heads, 32768 tokens, 4 bits, random codes and a random block
    permutation, with the last-level cache evicted before each call.  The
    keys are named attn_batch16_32k_* at head_dim 128 and carry a _d<D>
    suffix otherwise."""
    from kv_cache_vector_amd import _lib
    import math
    s = stream.cuda_stream
    res = {}
    B, Hq, Hkv, T, bs = 16, 32, 8, 32768, 16
    maxb = T // bs
    nblk = B * maxb
    g = torch.Generator(device=dev).manual_seed(5)
    d = head_dim
    P = d * 4 // 8                       # packed bytes per row at 4 bits
    kp = torch.randint(0, 256, (nblk, bs, Hkv, P), dtype=torch.uint8, device=dev, generator=g)
    vp = torch.randint(0, 256, (nblk, bs, Hkv, P), dtype=torch.uint8, device=dev, generator=g)
    kn = torch.rand((nblk, bs, Hkv), device=dev, generator=g) * 6 + 8
    vn = torch.rand((nblk, bs, Hkv), device=dev, generator=g) * 6 + 8
    q = torch.randn((B, Hq, d), device=dev, generator=g).half()
    bt = torch.randperm(nblk, device=dev, generator=g).to(torch.int32).reshape(B, maxb)
    cl = torch.full((B,), T, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    wsb = _lib.tq_attn_workspace_bytes(B, Hq, Hkv, d, bs, maxb)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    # Cache eviction between repetitions reads a 512 MB buffer: a write flush
    # would leave dirty lines whose write-back lands inside the timed kernel.
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

    def attn():
        _lib.check(_lib.tq_attn_decode(q.data_ptr(), kp.data_ptr(), kn.data_ptr(),
                                       vp.data_ptr(), vn.data_ptr(), bt.data_ptr(),
                                       cl.data_ptr(), B, Hq, Hkv, d, 4, 0, bs, maxb, nblk,
                                       1 / math.sqrt(d), out.data_ptr(), ws.data_ptr(), wsb,
                                       s), "tq_attn_decode")

    attn()
    times = []
    for _ in range(reps):
        flush.sum()        # evict the 256 MB last-level cache between repetitions
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        attn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    t_us = statistics.median(times) * 1e3
    packed_bytes = B * Hkv * T * 2 * (P + 4)
    sfx = "" if d == 128 else "_d%d" % d
    res["attn_batch16_32k_us" + sfx] = round(t_us, 1)
    res["attn_packed_GBps" + sfx] = round(packed_bytes / (t_us * 1e-6) / 1e9, 1)
    res["attn_fp16_equiv_GBps" + sfx] = round(B * Hkv * T * 2 * 2 * d / (t_us * 1e-6) / 1e9, 1)
    res["attn_hbm_frac" + sfx] = round(packed_bytes / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    return res


def stream_encode_measurement(torch, dev, stream, x, packed, norms):
    """2-bit encode of one 70B-class 128K layer, cache evicted before each."""
    from kv_cache_vector_amd import _lib
    s = stream.cuda_stream
    res = {}
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    n = 2 * 8 * 131072
    xl = x[:n]
    pk2 = packed[: n // 2].view(-1)[: n * 32].view(n, 32)
    times = []
    for layer in range(6):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        _lib.check(_lib.tq_encode(xl.data_ptr(), n, 128, 2, layer, pk2.data_ptr(),
                                  norms.data_ptr(), s), "tq_encode")
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    t_us = statistics.median(times[1:]) * 1e3
    res["stream_b2_layer_us"] = round(t_us, 1)
    res["stream_b2_80_layers_ms"] = round(80 * t_us / 1e3, 3)
    res["stream_b2_hbm_frac"] = round(n * (256 + 32 + 4) / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    return res


if __name__ == "__main__":
    sys.exit(main())
