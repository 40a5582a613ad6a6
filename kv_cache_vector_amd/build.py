"""Build libtq.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m kv_cache_vector_amd.build

The library lands next to this file (kv_cache_vector_amd/libtq.so); the
Python binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtq.so")
SOURCES = ["tq_abi.cpp", "tq_codec.hip", "tq_attn.hip", "tq_ceiling.hip"]
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtq)")


def flags() -> list:
    return [
        "-O3", "-std=c++17", "-fPIC", "-Wall",
        "--offload-arch=" + ARCH,
        "-mcode-object-version=5",
        # packed-FP32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core results in ordinary VGPRs: the attention accumulators are
        # rescaled by VALU code, which otherwise copies them out of AGPRs per page
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I" + INCLUDE, "-I" + CSRC,
    ]


SAN_LIB = os.path.join(PKG, "libtq_san.so")
# Host code only (argument checks, codebook solver, tables, launches) with
# AddressSanitizer and UndefinedBehaviorSanitizer; the GPU code is built as
# usual.  Each sanitizer flag reaches the host compilation only.
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                  "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the ROCm clang's AddressSanitizer runtime, which a process
    loading libtq_san.so must preload."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "amdclang++"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build libtq.so, or with ``sanitize`` libtq_san.so (host code under
    AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests)."""
    cc = hipcc()
    objs = []
    tmpdir = os.path.join(PKG, "_build_san" if sanitize else "_build")
    os.makedirs(tmpdir, exist_ok=True)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc] + flags() + (SAN_HOST_FLAGS if sanitize else []) + lang + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in line and "unknown target feature" not in line
                        and line.strip())
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, msg))
        if verbose and msg:
            print(msg)
        objs.append(obj)
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + \
        (["-Xarch_host", "-shared-libsan"] if sanitize else []) + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
