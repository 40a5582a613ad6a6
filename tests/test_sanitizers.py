"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The oracle (gcc) and libtq's host code (hipcc, sanitizer flags on the host
compilation only) are built with both sanitizers, any report aborting the
process; then the oracle's pins and libtq's ABI and operator CPU tests run
against those builds in child processes that preload the matching
AddressSanitizer runtime.  The GPU kernels are not instrumented (GPU
sanitizers are not used here)."""
import glob
import os
import subprocess
import sys

import pytest

import oracle
from kv_cache_vector_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _env(runtime):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + (":" + pre if pre else "")   # the runtime must come first
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run(code, runtime, timeout=900):
    r = subprocess.run([sys.executable, "-c", code], env=_env(runtime), capture_output=True,
                       text=True, timeout=timeout, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def _instrumented(path):
    syms = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True,
                          text=True, check=True).stdout
    return "__asan_" in syms


def test_oracle_pins_under_sanitizers():
    path = oracle.build(force=True, sanitize=True)
    assert _instrumented(path)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle\n"
            "oracle._lib = oracle.Oracle(oracle.SAN_LIB_PATH)\n"
            "import pytest\n"
            "rc = pytest.main(['-q', '-p', 'no:cacheprovider', %r])\n"
            "assert oracle.default().path == oracle.SAN_LIB_PATH\n"
            "sys.exit(rc)\n" % (ROOT, TESTS, os.path.join(TESTS, "test_oracle_pins.py")))
    out = _run(code, oracle.asan_runtime())
    assert " passed" in out and " failed" not in out


def _libtq_san():
    """The sanitized libtq, rebuilt when any source is newer."""
    srcs = glob.glob(os.path.join(libbuild.CSRC, "*")) + \
        glob.glob(os.path.join(libbuild.INCLUDE, "*.h"))
    if not os.path.exists(libbuild.SAN_LIB) or \
            os.path.getmtime(libbuild.SAN_LIB) < max(os.path.getmtime(f) for f in srcs):
        libbuild.build(sanitize=True)
    return libbuild.SAN_LIB


def test_abi_and_operator_cpu_tests_under_sanitizers():
    path = _libtq_san()
    assert _instrumented(path)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "from kv_cache_vector_amd import _lib\n"
            "L = _lib.load(%r)\n"
            "import pytest\n"
            "rc = pytest.main(['-q', '-p', 'no:cacheprovider', %r, %r])\n"
            "assert _lib.load() is L and L._name == %r\n"
            "sys.exit(rc)\n" % (ROOT, TESTS, path, os.path.join(TESTS, "test_abi_cpu.py"),
                                os.path.join(TESTS, "test_torch_ops_cpu.py"), path))
    out = _run(code, libbuild.asan_runtime())
    assert " passed" in out and " failed" not in out


def test_a_planted_overflow_is_reported(tmp_path):
    """The set-up does catch memory errors: a copy of the oracle whose pack
    step clears one byte past its output, built and loaded the same way,
    aborts with an AddressSanitizer report."""
    src = oracle.source_text()
    bad = src.replace("memset(out, 0, (size_t)nbytes);", "memset(out, 0, (size_t)nbytes + 1);")
    assert bad != src
    c_path = str(tmp_path / "planted.c")
    so_path = str(tmp_path / "libplanted.so")
    with open(c_path, "w") as f:
        f.write(bad)
    subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-w", "-fPIC", "-shared"]
                   + oracle.SAN_FLAGS + ["-o", so_path, c_path, "-lm"], check=True)
    code = ("import sys; sys.path[:0] = [%r]\n"
            "import numpy as np, oracle\n"
            "o = oracle.Oracle(%r)\n"
            "o.pack(np.arange(128) %% 16, 4)\n" % (ROOT, so_path))
    r = subprocess.run([sys.executable, "-c", code], env=_env(oracle.asan_runtime()),
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr
