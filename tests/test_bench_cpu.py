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


def test_cpu_baseline_record():
    x = np.random.default_rng(0).standard_normal((4096, bench.D)).astype(np.float16)
    res = bench.cpu_baseline(x, budget_s=5.0)
    assert set(res) == {"value", "unit", "cores", "kind", "sample"}
    assert res["kind"] == "oracle" and res["unit"] == "GB/s"
    assert res["value"] > 0 and 1 <= res["cores"] <= 16
    assert "4096 vectors" in res["sample"]      # the whole (bounded) sample ran


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
