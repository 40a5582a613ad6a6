"""Host-side contract of bench.py (no GPU needed): the one-GPU refusal, the
CPU-baseline record, the committed HBM-traffic record and the commands the
profile summaries give."""
import glob
import json
import os
import re
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""            # no JSON line for a run that did not happen


SMALL = dict(c4_tokens=256, c5_tokens=256, c3_tokens=64)   # the 70B layers, attention step, Student-t layer, shrunk


def test_cpu_baseline_record():
    rng = np.random.default_rng(0)
    layers = [rng.standard_normal((4096, bench.D)).astype(np.float16) for _ in range(3)]
    res, extra = bench.cpu_baseline(layers, budget_s=20.0, single_layer_budget_s=10.0, **SMALL)
    assert set(res) == {"value", "unit", "cores", "kind", "sample"}
    assert res["kind"] == "oracle" and res["unit"] == "GB/s"
    assert res["value"] > 0 and 1 <= res["cores"] <= 16
    assert "the whole cache (12288 vectors)" in res["sample"]   # every layer ran
    assert "over 4096 vectors of layer 0" in res["sample"]      # the 1-thread run
    # 70B-class layers 0/40/79 (2 x 8 heads x 256 tokens each) in full, and
    # 1% of the others' tokens (3 per K/V and head: 48 vectors each)
    assert "layers 0/40/79 in full plus a 0.01 sample of the others" in res["sample"]
    assert "all 15984 vectors (12288 in the full layers, 3696 in the 77 samples)" in res["sample"]
    assert "Student-t layer 0 (4096 vectors) at 3 / 2 bits" in res["sample"]
    assert "the 4,096-vector outlier workload on 1 thread" in res["sample"]
    assert "all 16 sequences" in res["sample"]                  # the whole attention step
    assert "hardware threads visible" in res["sample"]
    assert set(extra) == {"cpu_oracle_1thread_GBps", "cpu_oracle_70b_layers_b2_GBps",
                          "cpu_oracle_attn_batch16_32k_ms", "cpu_oracle_outlier_4096_ms",
                          "cpu_oracle_student_t_b3_GBps", "cpu_oracle_student_t_b2_GBps"}
    assert all(v > 0 for v in extra.values())


def test_cpu_baseline_budget_reports_the_subset():
    layers = [np.zeros((8192, bench.D), np.float16)]
    res, extra = bench.cpu_baseline(layers, budget_s=0.0, single_layer_budget_s=0.0,
                                    c4_budget_s=0.0, c5_budget_s=0.0, c3_budget_s=0.0, **SMALL)
    assert "the first" in res["sample"] and "of 8192 vectors" in res["sample"]
    # every leg finishes at least its first piece; the attention leg scales it to the step
    assert "of 16 sequences, scaled to 16" in res["sample"]


def test_70b_layer_sample_has_the_layer_scales():
    """The 1% sample of a 70B-class layer: 2 x 8 heads x round(0.01 T) rows,
    each (K/V, head) block scaled by that layer's factor."""
    from kv_cache_vector_amd import workloads as W
    x = W.llama70b_layer_sample(7, 0.01, tokens=131072).astype(np.float64)
    n = round(0.01 * 131072)
    assert x.shape == (2 * 8 * n, bench.D)
    sd = x.reshape(2, 8, n * bench.D).std(axis=2)
    np.testing.assert_allclose(sd, W.llama70b_head_scales(7), rtol=0.02)


def test_gpu_clocks_never_raises():
    r = bench.gpu_clocks()
    assert r is None or all(isinstance(v, int) for v in r.values())


def test_gpu_clocks_not_run_under_a_profiler(monkeypatch):
    """Under rocprofv3 (its library preloaded, ROCPROF_* set) no rocm-smi
    child is started: the profiler's library would start the GPU runtime in
    that child before its interpreter runs."""
    def no_child(*a, **k):
        raise AssertionError("rocm-smi started under a profiler")
    monkeypatch.setattr(subprocess, "run", no_child)
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so")
    assert bench.gpu_clocks() is None
    monkeypatch.delenv("LD_PRELOAD")
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp")
    assert bench.gpu_clocks() is None


def test_oracle_attention_pieces_match_one_call():
    """The per-sequence pieces of the attention leg compute what one call
    over the whole batch computes (the leg times real work)."""
    import oracle
    o = oracle.default()
    rng = np.random.default_rng(1)
    B, hq, hkv, bs, T = 2, 4, 1, 16, 64
    nblk = B * T // bs
    kp = rng.integers(0, 256, (nblk, bs, hkv, 64), dtype=np.uint8)
    vp = rng.integers(0, 256, (nblk, bs, hkv, 64), dtype=np.uint8)
    kn = rng.random((nblk, bs, hkv), dtype=np.float32) + 1
    vn = rng.random((nblk, bs, hkv), dtype=np.float32) + 1
    q = rng.standard_normal((B, hq, bench.D)).astype(np.float16)
    bt = rng.permutation(nblk).astype(np.int32).reshape(B, T // bs)
    cl = np.full(B, T, np.int32)
    whole = o.attn_decode(q, kp, kn, vp, vn, bt, cl, hkv, 4, 0, 0.1)
    for b in range(B):
        sel = np.zeros((B, hq), np.uint8)
        sel[b] = 1
        part = o.attn_decode(q, kp, kn, vp, vn, bt, cl, hkv, 4, 0, 0.1, sel=sel)
        assert np.array_equal(part[b].view(np.uint16), whole[b].view(np.uint16))


def test_traffic_record_matches_the_sources_or_is_withheld():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        rec = json.load(f)
    enc = bench.measured_traffic("encode_kernel<4>")
    dec = bench.measured_traffic("decode_kernel<4>")
    if rec["source_digest"] != bench.source_digest():
        # counters taken on other kernel sources are not reported
        assert enc is None and dec is None
        return
    for name, k in rec["kernels"].items():
        assert k["algorithmic"] == bench.N * bench.ALGO_BYTES
        assert k["read"] + k["written"] == k["bytes_per_launch"]
        # HBM bytes within 5% of the algorithmic bytes: no re-reads, no partial lines
        assert abs(k["bytes_per_launch"] / k["algorithmic"] - 1) < 0.05, name
    assert enc == rec["kernels"]["encode_kernel<4>"]["bytes_per_launch"]
    assert dec == rec["kernels"]["decode_kernel<4>"]["bytes_per_launch"]


def test_profile_commands_run_committed_files():
    summaries = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert summaries
    for path in summaries:
        with open(path) as f:
            text = f.read()
        cmds = [line.strip() for line in text.splitlines() if "rocprofv3 --" in line]
        assert cmds, path
        for cmd in cmds:
            for part in cmd.split(";"):
                if "rocprofv3 --" not in part:
                    continue
                # the profiled program follows "--" directly: python3 $R/<file>
                m = re.search(r" -- (\S+) \$R/(\S+)", part)
                assert m, (path, part)
                assert m.group(1) in ("python3", "python"), (path, part)
                assert os.path.isfile(os.path.join(ROOT, m.group(2))), (path, part)
                assert "_work" not in part, (path, part)
