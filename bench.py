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
    python bench.py --hybrid-only               (hybrid-mode side measurement only)

Prints one JSON line.  `value` is fp16 key/value bytes passed through the
codec per second (encode and decode both count their 256 B/vector of fp16).
`roofline` rates the slower of the two kernels by its algorithmic bytes
(256 B fp16 + 64 B codes + 4 B norm per vector) against the 8 TB/s HBM peak.
`cpu_baseline` is the plain CPU oracle timed on this host: encode + decode of
the same whole cache on up to 16 threads (and, reported in `extra`: layer 0
on one thread, layers 0/40/79 of the 70B-class 128K cache at 2 bits, and the
batch-16 x 32K decode-attention step).  `extra` also rates the two kernels against
no-arithmetic kernels that move the same byte mix (include/tq_ceiling.h).
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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_pieces(pieces, work, threads: int, budget_s: float):
    """work(piece) -> units done, for the pieces in order on `threads` host
    threads (the oracle's C calls release the interpreter lock), until all
    are done or budget_s has passed (the first piece runs regardless).
    Returns (units done, wall seconds)."""
    lock = threading.Lock()
    state = {"next": 0, "done": 0}
    t0 = time.perf_counter()
    deadline = t0 + budget_s

    def worker():
        while True:
            with lock:
                # the first piece always runs, so every leg has a measured basis
                if state["next"] >= len(pieces) or (state["next"] and time.perf_counter() > deadline):
                    return
                piece = pieces[state["next"]]
                state["next"] += 1
            n = work(piece)
            with lock:
                state["done"] += n

    ts = [threading.Thread(target=worker) for _ in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return state["done"], time.perf_counter() - t0


def oracle_codec_rate(chunks, threads: int, budget_s: float, chunk: int = 4096,
                      bits: int = BITS, seeds=None):
    """The unmodified oracle (encode + decode at `bits`, codec seed seeds[c],
    default 0) over the host arrays in `chunks` (each [n, 128] fp16), split
    into `chunk`-vector pieces taken in order by `threads` host threads, until
    done or until budget_s has passed.  Returns (vectors done, wall seconds)."""
    import oracle
    oracle.build(force=False)
    o = oracle.default()
    seeds = [0] * len(chunks) if seeds is None else seeds
    pieces = [(ci, i) for ci, c in enumerate(chunks) for i in range(0, c.shape[0], chunk)]

    def work(piece):
        ci, i = piece
        xs = chunks[ci][i:i + chunk]
        p, n = o.encode(xs, bits, seeds[ci])
        o.decode(p, n, D, bits, seeds[ci])
        return xs.shape[0]

    return run_pieces(pieces, work, threads, budget_s)


def oracle_attention_time(threads: int, budget_s: float, batch: int = 16, tokens: int = 32768):
    """The unmodified oracle's paged decode attention at batch `batch` x
    `tokens` cached tokens, 32 / 8 heads, head_dim 128, 4 bits, random codes,
    norms in [8, 14) and a random block permutation (the GPU side
    measurement's inputs), one sequence per piece on `threads` host threads.
    Returns (sequences done, wall seconds)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    o = oracle.default()
    hq, hkv, bs = 32, 8, 16
    rng = np.random.default_rng(5)
    nblk = batch * tokens // bs
    kp = rng.integers(0, 256, (nblk, bs, hkv, CODE_BYTES), dtype=np.uint8)
    vp = rng.integers(0, 256, (nblk, bs, hkv, CODE_BYTES), dtype=np.uint8)
    kn = (rng.random((nblk, bs, hkv), dtype=np.float32) * 6 + 8).astype(np.float32)
    vn = (rng.random((nblk, bs, hkv), dtype=np.float32) * 6 + 8).astype(np.float32)
    q = rng.standard_normal((batch, hq, D)).astype(np.float16)
    bt = rng.permutation(nblk).astype(np.int32).reshape(batch, tokens // bs)
    cl = np.full(batch, tokens, np.int32)

    def work(b):
        sel = np.zeros((batch, hq), np.uint8)
        sel[b] = 1
        o.attn_decode(q, kp, kn, vp, vn, bt, cl, hkv, BITS, 0, 1.0 / D ** 0.5, sel=sel)
        return 1

    return run_pieces(list(range(batch)), work, threads, budget_s)


def cpu_baseline(layers, budget_s: float = 60.0, single_layer_budget_s: float = 30.0,
                 c4_layers=(0, 40, 79), c4_budget_s: float = 40.0, c5_budget_s: float = 60.0,
                 c4_tokens: int = 131072, c5_tokens: int = 32768, c3_tokens: int = 8192,
                 c3_budget_s: float = 20.0, c4_sample: float = 0.01):
    """The oracle timed on this host:
      - encode + decode of the whole cache (`layers`, a list of [n, 128] fp16
        host arrays) on min(16, hardware threads) threads: the record's value;
      - the same over layer 0 on one thread;
      - the 4,096-vector outlier workload (1 thread);
      - the heavy-tailed (Student-t) layer 0 of the same cache at 3 and at 2
        bits (the layer-0 subset of that workload);
      - the 70B-class 128K cache's layers `c4_layers` in full and a seeded
        `c4_sample` of every other layer's tokens (2 bits, codec seed =
        layer);
      - the batch-16 x 32K decode-attention step, one sequence per thread.
    A leg that hits its budget reports what it finished (scaled up for the
    attention step).  Returns (record, extra figures)."""
    from kv_cache_vector_amd import workloads as W
    hw = os.cpu_count() or 1
    threads = max(1, min(16, hw))
    total = sum(x.shape[0] for x in layers)
    nvec, wall = oracle_codec_rate(layers, threads, budget_s)
    value = 2 * nvec * 2 * D / wall / 1e9
    n1, w1 = oracle_codec_rate(layers[:1], 1, single_layer_budget_s)
    one = 2 * n1 * 2 * D / w1 / 1e9
    c1 = W.outlier_channels_fixed()
    n1c, w1c = oracle_codec_rate([c1], 1, 60.0)
    c3 = W.llama8b_layer(0, dist="student_t", tokens=c3_tokens)
    c3_rates = {}
    for bits in (3, 2):
        n3, w3 = oracle_codec_rate([c3], threads, c3_budget_s, bits=bits)
        c3_rates[bits] = (2 * n3 * 2 * D / w3 / 1e9, n3)
    del c3
    c4 = [W.llama70b_layer(layer, tokens=c4_tokens) for layer in c4_layers]
    c4_seeds = list(c4_layers)
    c4_full = sum(x.shape[0] for x in c4)
    others = [layer for layer in range(80) if layer not in c4_layers] if c4_sample > 0 else []
    c4 += [W.llama70b_layer_sample(layer, c4_sample, tokens=c4_tokens) for layer in others]
    c4_seeds += others
    c4_total = sum(x.shape[0] for x in c4)
    n4, w4 = oracle_codec_rate(c4, threads, c4_budget_s, bits=2, seeds=c4_seeds)
    del c4
    c4_rate = 2 * n4 * 2 * D / w4 / 1e9
    batch = 16
    n5, w5 = oracle_attention_time(threads, c5_budget_s, batch=batch, tokens=c5_tokens)
    c5_ms = w5 / max(n5, 1) * batch * 1e3 if n5 < batch else w5 * 1e3
    what = "the whole cache" if nvec == total else "the first %d of %d vectors" % (nvec, total)
    what4 = ("all %d vectors (%d in the full layers, %d in the %d samples)" % (c4_total, c4_full, c4_total - c4_full, len(others))
             if n4 == c4_total else "the first %d of %d vectors" % (n4, c4_total))
    what5 = "all %d sequences" % batch if n5 == batch else "%d of %d sequences, scaled to %d" % (n5, batch, batch)
    rec = {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": "encode+decode (4 bits) of %s (%d vectors) on %d threads in %.1f s; "
                     "1 thread: %.4f GB/s over %d vectors of layer 0 in %.1f s; "
                     "the 4,096-vector outlier workload on 1 thread in %.1f ms; "
                     "Student-t layer 0 (%d vectors) at 3 / 2 bits: %.4f / %.4f GB/s; "
                     "70B-class 128K cache, layers %s in full plus a %g sample of the others, "
                     "at 2 bits: %.4f GB/s over %s in %.1f s; "
                     "decode attention batch %d x %d tokens, 32/8 heads, 4 bits: %.0f ms per step "
                     "(%s in %.1f s); %d hardware threads visible, at most 16 used (the host "
                     "share of one GPU); %s"
                     % (what, nvec, threads, wall, one, n1, w1, w1c * 1e3,
                        c3_rates[3][1], c3_rates[3][0], c3_rates[2][0],
                        "/".join(str(x) for x in c4_layers), c4_sample, c4_rate, what4, w4,
                        batch, c5_tokens, c5_ms, what5, w5, hw, _cpu_model())}
    extra = {"cpu_oracle_1thread_GBps": round(one, 4),
             "cpu_oracle_outlier_4096_ms": round(w1c * 1e3, 1),
             "cpu_oracle_student_t_b3_GBps": round(c3_rates[3][0], 4),
             "cpu_oracle_student_t_b2_GBps": round(c3_rates[2][0], 4),
             "cpu_oracle_70b_layers_b2_GBps": round(c4_rate, 4),
             "cpu_oracle_attn_batch16_32k_ms": round(c5_ms, 1)}
    return rec, extra


def gpu_clocks():
    """The current sclk / mclk levels as rocm-smi reports them (None when it
    is not available).  Under a profiler (rocprofv3 preloads its library into
    every child, which would start the GPU runtime inside the rocm-smi
    process before that script's interpreter runs) it is not run."""
    import os
    import re
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    found = {}
    for line in r.stdout.splitlines():
        m = re.search(r"\b(sclk|mclk|fclk)\b.*\((\d+)\s*Mhz\)", line, re.I)
        if m and m.group(1).lower() not in found:
            found[m.group(1).lower()] = int(m.group(2))
    return found or None


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
    ap.add_argument("--attn-warmup", type=int, default=100,
                    help="untimed attention calls before the timed ones (--attn-only)")
    ap.add_argument("--hybrid-only", action="store_true",
                    help="only the hybrid-mode (tq35 / tq25) whole-cache measurement (for profiling)")
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
                                    reps=max(1, args.steps), head_dim=args.head_dim,
                                    warmup=max(1, args.attn_warmup))
        print(json.dumps(res), flush=True)
        return 0

    import numpy as np
    import torch

    from kv_cache_vector_amd import _lib

    _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream

    x, host_layers = upload_cache(torch, dev, keep_host=not (args.no_cpu_baseline or args.hybrid_only))
    if args.hybrid_only:
        print(json.dumps(hybrid_measurement(torch, dev, stream, x)), flush=True)
        return 0
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

    clocks = gpu_clocks()
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
    if clocks:
        extra["clocks_MHz_after_timed_steps"] = clocks
    props = torch.cuda.get_device_properties(dev)
    extra["device"] = {k: getattr(props, a) for k, a in (
        ("arch", "gcnArchName"), ("compute_units", "multi_processor_count"),
        ("lds_bytes_per_workgroup", "shared_memory_per_block"),
        ("threads_per_cu", "max_threads_per_multi_processor"), ("l2_bytes", "L2_cache_size"),
        ("hbm_bytes", "total_memory")) if hasattr(props, a)}
    # achievable-bandwidth reference: the no-arithmetic kernels that move the
    # codec's own byte mix with its work mapping (include/tq_ceiling.h)
    extra.update(ceiling_measurement(torch, stream, x, packed, norms, out, enc_avg, dec_avg))
    # one plain device copy of the 4 GiB cache (4,294,967,296 B each way):
    # the known-size reference that scales rocprofv3's HBM byte counters
    out.copy_(x)

    if not args.no_extras:
        del out
        extra.update(side_measurements(torch, dev, stream, x, packed, norms))
        extra.update(ceiling_fractions(extra))

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
        log("timing the CPU oracle: the whole cache (16 threads), layer 0 (1 thread), "
            "70B-class layers 0/40/79, the batch-16 x 32K attention step")
        res["cpu_baseline"], cpu_extra = cpu_baseline(host_layers)
        extra.update(cpu_extra)
    print(json.dumps(res), flush=True)
    return 0


def side_measurements(torch, dev, stream, x, packed, norms):
    """Decode attention at batch 16, 32/8 heads, 32768 tokens (4 bits, random
    codes; head_dim 128, 64 and 256), the 70B-class 128K-context cache
    encoded as a layer-by-layer stream (2 bits), and other codec launch
    shapes."""
    # 100 untimed calls (about 20 ms) before each attention measurement let
    # the clocks settle under the attention's own load (the first follows the
    # codec's sustained load)
    res = attention_measurement(torch, dev, stream)
    for hd in (64, 256):
        res.update(attention_measurement(torch, dev, stream, head_dim=hd))
    for kb, vb in ((4, 2), (3, 3), (2, 2)):        # other widths at head_dim 128
        res.update(attention_measurement(torch, dev, stream, k_bits=kb, v_bits=vb))
    res.update(stream_encode_measurement(torch, dev, stream, x, packed, norms))
    res.update(codec_side_measurement(torch, dev, stream, x, packed, norms))
    res.update(hybrid_measurement(torch, dev, stream, x))
    return res


def upload_cache(torch, dev, keep_host):
    """The 8B-shaped cache, generated layer by layer on the host and uploaded
    to one resident [N, D] fp16 tensor; the host layers too if keep_host."""
    from kv_cache_vector_amd import workloads as W
    log("generating the 8B-shaped cache: %d vectors (%.2f GB fp16)" % (N, N * 2 * D / 1e9))
    x = torch.empty((N, D), dtype=torch.float16, device=dev)
    host_layers = []
    for layer in range(LAYERS):
        xl = W.llama8b_layer(layer)
        if keep_host:
            host_layers.append(xl)
        x[layer * PER_LAYER:(layer + 1) * PER_LAYER].copy_(torch.from_numpy(xl))
        if layer % 8 == 7:
            log("  layer %d/%d uploaded" % (layer + 1, LAYERS))
    return x, host_layers


def hybrid_measurement(torch, dev, stream, x):
    """Hybrid modes tq35 / tq25 (split groups + QJL residual) over the whole
    resident 8B-shaped cache: encode and decode, median of 5 launches each
    (identity channel split; the split does not change the work)."""
    from kv_cache_vector_amd import _lib
    import numpy as np
    s = stream.cuda_stream
    res = {}
    perm = np.arange(D, dtype=np.int32)
    out = torch.empty_like(x)
    for mode, name in ((35, "tq35"), (25, "tq25")):
        row = _lib.tq_hybrid_packed_bytes(D, mode)
        pk = torch.empty((N, row), dtype=torch.uint8, device=dev)
        calls = {"encode": lambda: _lib.tq_hybrid_encode(x.data_ptr(), N, D, mode, 0,
                                                         perm.ctypes.data, pk.data_ptr(), s),
                 "decode": lambda: _lib.tq_hybrid_decode(pk.data_ptr(), N, D, mode, 0,
                                                         perm.ctypes.data, out.data_ptr(), s)}
        for what, fn in calls.items():
            _lib.check(fn(), "tq_hybrid_" + what)
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                _lib.check(fn(), "tq_hybrid_" + what)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = statistics.median(ts)
            res["hybrid_%s_%s_ms" % (name, what)] = round(ms, 4)
            res["hybrid_%s_%s_hbm_frac" % (name, what)] = round(
                N * (2 * D + row) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        del pk
    del out
    return res


def _median_min(times):
    return statistics.median(times), min(times)


def codec_side_measurement(torch, dev, stream, x, packed, norms):
    """Other codec launch shapes on the resident cache (timing does not depend
    on the values):
      - 3- and 2-bit encode and decode of the whole 16,777,216-vector cache
        (5 warm-up steps, then the mean over 20 back-to-back steps, as the
        4-bit headline);
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
        # the headline's protocol: warm-up steps, then back-to-back encode +
        # decode steps with an event around each kernel; mean and minimum
        P = D * bits // 8
        pk = packed.view(-1)[: N * P].view(N, P)
        fe, fd = enc(N, bits, pk), dec(N, bits, pk)
        for _ in range(5):
            fe()
            fd()
        steps = 20
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            ev[k][0].record(stream)
            fe()
            ev[k][1].record(stream)
            fd()
            ev[k][2].record(stream)
        torch.cuda.synchronize()
        for name, i in (("encode", 0), ("decode", 1)):
            t = [e[i].elapsed_time(e[i + 1]) for e in ev]
            avg = statistics.mean(t)
            res["%s_b%d_ms" % (name, bits)] = round(avg, 4)
            res["%s_b%d_min_ms" % (name, bits)] = round(min(t), 4)
            res["%s_b%d_hbm_frac" % (name, bits)] = round(
                N * (2 * D + P + 4) / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
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


def attention_measurement(torch, dev, stream, reps: int = 20, head_dim: int = 128,
                          warmup: int = 100, k_bits: int = 4, v_bits: int = 4):
    """Median (and minimum) time of tq_attn_decode_kv (split + combine kernels) at
    batch 16, 32/8 heads, 32768 tokens, 4-bit keys and values unless stated,
    random codes and a random block permutation, with the last-level cache
    evicted before each call, after `warmup` untimed calls (the first calls
    run while the clocks rise).  The keys are named attn_batch16_32k_* at
    head_dim 128 and 4/4 bits, with a _d<D> suffix at another head_dim and a
    _k<kb>v<vb> suffix at other widths."""
    from kv_cache_vector_amd import _lib
    import math
    s = stream.cuda_stream
    res = {}
    B, Hq, Hkv, T, bs = 16, 32, 8, 32768, 16
    maxb = T // bs
    nblk = B * maxb
    g = torch.Generator(device=dev).manual_seed(5)
    d = head_dim
    PK, PV = d * k_bits // 8, d * v_bits // 8     # packed bytes per key / value row
    kp = torch.randint(0, 256, (nblk, bs, Hkv, PK), dtype=torch.uint8, device=dev, generator=g)
    vp = torch.randint(0, 256, (nblk, bs, Hkv, PV), dtype=torch.uint8, device=dev, generator=g)
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
        _lib.check(_lib.tq_attn_decode_kv(q.data_ptr(), kp.data_ptr(), kn.data_ptr(),
                                          vp.data_ptr(), vn.data_ptr(), bt.data_ptr(),
                                          cl.data_ptr(), B, Hq, Hkv, d, k_bits, v_bits, 0, bs,
                                          maxb, nblk, 1 / math.sqrt(d), out.data_ptr(),
                                          ws.data_ptr(), wsb, s), "tq_attn_decode_kv")

    for _ in range(max(1, warmup)):
        flush.sum()
        attn()
    torch.cuda.synchronize()
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
    sfx = ("" if d == 128 else "_d%d" % d) + ("" if (k_bits, v_bits) == (4, 4) else "_k%dv%d" % (k_bits, v_bits))
    res["attn_batch16_32k_min_us" + sfx] = round(min(times) * 1e3, 1)
    packed_bytes = B * Hkv * T * (PK + 4 + PV + 4)
    res["attn_batch16_32k_us" + sfx] = round(t_us, 1)
    res["attn_packed_GBps" + sfx] = round(packed_bytes / (t_us * 1e-6) / 1e9, 1)
    res["attn_fp16_equiv_GBps" + sfx] = round(B * Hkv * T * 2 * 2 * d / (t_us * 1e-6) / 1e9, 1)
    res["attn_hbm_frac" + sfx] = round(packed_bytes / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    return res


def stream_encode_measurement(torch, dev, stream, x, packed, norms):
    """The 70B-class 128K-context cache (80 layers x {K,V} x 8 KV heads x
    131072 tokens, 2 bits) encoded as a stream, layer by layer: each layer's
    2,097,152 vectors are generated on the device (N(0,1) times the layer's
    per-(K/V, head) scales, drawn from its data seed 300 + layer), the
    last-level cache is evicted, and the layer is encoded with codec seed =
    layer into its own slice of a packed cache that stays resident (80 x 64 MiB
    codes + 80 x 8 MiB norms).  Reported: the sum of the 80 per-layer encode
    times (HIP events around each launch)."""
    from kv_cache_vector_amd import _lib
    from kv_cache_vector_amd import workloads as W
    s = stream.cuda_stream
    layers, heads, tokens = 80, 8, 131072
    n = 2 * heads * tokens
    P = D * 2 // 8
    xl = torch.empty((2, heads, tokens, D), dtype=torch.float16, device=dev)
    pk = torch.empty((layers, n, P), dtype=torch.uint8, device=dev)
    nm = torch.empty((layers, n), dtype=torch.float32, device=dev)
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev)
    times = []
    for layer in range(layers):
        gen.manual_seed(300 + layer)
        sc = torch.from_numpy(W.llama70b_head_scales(layer, heads)).to(dev)
        xl.normal_(generator=gen)
        xl.mul_(sc[:, :, None, None].half())
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        _lib.check(_lib.tq_encode(xl.data_ptr(), n, D, 2, layer, pk[layer].data_ptr(),
                                  nm[layer].data_ptr(), s), "tq_encode")
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in times]
    total = sum(ms)
    res = {"stream_b2_80_layers_ms": round(total, 3),
           "stream_b2_layer_median_us": round(statistics.median(ms) * 1e3, 1),
           "stream_b2_hbm_frac": round(layers * n * (2 * D + P + 4) / (total * 1e-3) / 1e9
                                       / HBM_PEAK_GBPS, 4)}
    del pk, nm, xl
    return res


def ceiling_measurement(torch, stream, x, packed, norms, out, enc_ms, dec_ms):
    """The codec's byte mix moved by the no-arithmetic kernels of
    tq_ceiling.h over the whole 4 GiB cache (4, 3 and 2 bits; median of 10
    launches each), and the 4-bit encode and decode kernels' time against
    them (the 3- and 2-bit kernels are rated in ceiling_fractions)."""
    import ctypes
    from kv_cache_vector_amd import _lib
    L = _lib.load()
    f = L.tq_ceiling_stream
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    s = stream.cuda_stream
    calls = {}
    for bits in (4, 3, 2):
        pb = D * bits // 8
        sfx = "" if bits == BITS else "_b%d" % bits
        calls["encode" + sfx] = lambda pb=pb: f(0, pb, x.data_ptr(), None, N, packed.data_ptr(),
                                                norms.data_ptr(), s)
        calls["decode" + sfx] = lambda pb=pb: f(1, pb, packed.data_ptr(), norms.data_ptr(), N,
                                                out.data_ptr(), None, s)
    res = {}
    for name, fn in calls.items():
        assert fn() == 0, "tq_ceiling_stream"
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = statistics.median(ts)
        bits = int(name[-1]) if "_b" in name else BITS
        res["ceiling_%s_mix_ms" % name] = round(ms, 4)
        res["ceiling_%s_mix_GBps" % name] = round(N * (2 * D + D * bits // 8 + 4) / (ms * 1e-3) / 1e9, 1)
    res["encode_frac_of_ceiling"] = round(res["ceiling_encode_mix_ms"] / enc_ms, 4)
    res["decode_frac_of_ceiling"] = round(res["ceiling_decode_mix_ms"] / dec_ms, 4)
    return res


def ceiling_fractions(extra):
    """The 3- and 2-bit codec kernels' times (side measurements) against
    their byte mixes' no-arithmetic times."""
    res = {}
    for bits in (3, 2):
        for name in ("encode", "decode"):
            c, k = extra.get("ceiling_%s_b%d_mix_ms" % (name, bits)), extra.get("%s_b%d_ms" % (name, bits))
            if c and k:
                res["%s_b%d_frac_of_ceiling" % (name, bits)] = round(c / k, 4)
    return res


if __name__ == "__main__":
    sys.exit(main())
