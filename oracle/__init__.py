"""CPU oracle of the TurboQuant KV-cache codec -- TEST INFRASTRUCTURE ONLY.

The oracle is a plain C implementation in double precision (``tq_oracle.c``)
of what the codec computes.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the product
library (``kv_cache_vector_amd``) never does, and the two share no code.

This module compiles the C file with gcc (``build()``) and wraps it with
ctypes (numpy arrays in, numpy arrays out).  Marshalling only: every step of
the arithmetic lives in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtq_oracle.so")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p


SAN_LIB_PATH = os.path.join(_HERE, "libtq_oracle_san.so")
# gcc's AddressSanitizer runtime: a process that loads the sanitized build
# must have it preloaded (LD_PRELOAD), ahead of every other library
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle into ``oracle/libtq_oracle.so`` (gcc -O2, no
    fast-math), or with ``sanitize`` into ``oracle/libtq_oracle_san.so`` built
    with AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts)."""
    path = SAN_LIB_PATH if sanitize else _LIB_PATH
    if not force and os.path.exists(path) and \
            os.path.getmtime(path) >= os.path.getmtime(_SRC):
        return path
    tmp = path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wextra", "-fPIC",
           "-shared"] + (SAN_FLAGS if sanitize else []) + ["-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, path)
    return path


def asan_runtime() -> str:
    """Path of gcc's AddressSanitizer runtime library."""
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True)
    return r.stdout.strip()


def _bind(L: ctypes.CDLL) -> ctypes.CDLL:
    L.tqo_half_to_double.argtypes = [ctypes.c_uint16]
    L.tqo_half_to_double.restype = ctypes.c_double
    L.tqo_double_to_half.argtypes = [ctypes.c_double]
    L.tqo_double_to_half.restype = ctypes.c_uint16
    L.tqo_splitmix64_seq.argtypes = [ctypes.c_uint64, ctypes.c_int, _P]
    L.tqo_splitmix64_seq.restype = None
    L.tqo_signs.argtypes = [ctypes.c_uint64, ctypes.c_int, _P]
    L.tqo_hadamard.argtypes = [ctypes.c_int, _P]
    L.tqo_codebook.argtypes = [ctypes.c_int, _P, _P]
    L.tqo_codebook_distortion.argtypes = [ctypes.c_int]
    L.tqo_codebook_distortion.restype = ctypes.c_double
    L.tqo_quantize.argtypes = [ctypes.c_double, _P, ctypes.c_int]
    L.tqo_pack.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P]
    L.tqo_pack.restype = None
    L.tqo_unpack.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P]
    L.tqo_unpack.restype = None
    L.tqo_encode.argtypes = [_P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                             ctypes.c_uint64, _P, _P, _P]
    L.tqo_decode.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                             ctypes.c_uint64, _P, _P]
    L.tqo_attn_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_double, _P, _P, _P]
    L.tqo_attn_decode_kv.argtypes = [_P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_double, _P, _P, _P]
    L.tqo_packed_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    L.tqo_hybrid_packed_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    L.tqo_hybrid_encode.argtypes = [_P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint64, _P, _P, _P, _P]
    L.tqo_hybrid_decode.argtypes = [_P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint64, _P, _P, _P]
    return L


HYBRID_MODES = {"tq35": 35, "tq25": 25}


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """ctypes view of one compiled copy of the oracle (numpy in, numpy out)."""

    def __init__(self, so_path: str):
        self.path = so_path
        self.L = _bind(ctypes.CDLL(so_path))

    def half_to_double(self, bits_u16) -> np.ndarray:
        b = _c(bits_u16, np.uint16).ravel()
        f = self.L.tqo_half_to_double
        return np.array([f(int(v)) for v in b], dtype=np.float64)

    def double_to_half(self, x) -> np.ndarray:
        x = _c(x, np.float64).ravel()
        f = self.L.tqo_double_to_half
        return np.array([f(float(v)) for v in x], dtype=np.uint16)

    def splitmix64(self, seed: int, n: int) -> np.ndarray:
        out = np.zeros(n, dtype=np.uint64)
        self.L.tqo_splitmix64_seq(ctypes.c_uint64(seed), n, _ptr(out))
        return out

    def signs(self, seed: int, d: int = 128) -> np.ndarray:
        out = np.zeros(d, dtype=np.int8)
        rc = self.L.tqo_signs(ctypes.c_uint64(seed), d, _ptr(out))
        assert rc == 0
        return out

    def hadamard(self, d: int = 128) -> np.ndarray:
        out = np.zeros((d, d), dtype=np.int8)
        rc = self.L.tqo_hadamard(d, _ptr(out))
        assert rc == 0
        return out

    def codebook(self, bits: int):
        L = 1 << bits
        c = np.zeros(L, dtype=np.float64)
        t = np.zeros(L - 1, dtype=np.float64)
        it = self.L.tqo_codebook(bits, _ptr(c), _ptr(t))
        assert it > 0
        return c, t

    def codebook_distortion(self, bits: int) -> float:
        return self.L.tqo_codebook_distortion(bits)

    def quantize_many(self, z, bits: int) -> np.ndarray:
        _, t = self.codebook(bits)
        f = self.L.tqo_quantize
        L = 1 << bits
        return np.array([f(float(v), _ptr(t), L) for v in np.ravel(z)], dtype=np.uint8)

    def pack(self, codes, bits: int) -> np.ndarray:
        codes = _c(codes, np.uint8)
        d = codes.shape[-1]
        out = np.zeros(d * bits // 8, dtype=np.uint8)
        self.L.tqo_pack(_ptr(codes), d, bits, _ptr(out))
        return out

    def unpack(self, packed, d: int, bits: int) -> np.ndarray:
        packed = _c(packed, np.uint8)
        out = np.zeros(d, dtype=np.uint8)
        self.L.tqo_unpack(_ptr(packed), d, bits, _ptr(out))
        return out

    def packed_bytes(self, d: int, bits: int) -> int:
        return self.L.tqo_packed_bytes(d, bits)

    def encode(self, x_f16, bits: int, seed: int, want_z: bool = False):
        """x_f16: array [..., d] of float16 (or its uint16 bit patterns).

        Returns (packed [..., d*bits/8] u8, norms [...] f32[, z [..., d] f64])."""
        x = np.asarray(x_f16)
        if x.dtype == np.float16:
            x = x.view(np.uint16)
        x = _c(x, np.uint16)
        d = x.shape[-1]
        lead = x.shape[:-1]
        n = int(np.prod(lead)) if lead else 1
        P = d * bits // 8
        packed = np.zeros(lead + (P,), dtype=np.uint8)
        norms = np.zeros(lead, dtype=np.float32)
        z = np.zeros(lead + (d,), dtype=np.float64) if want_z else None
        rc = self.L.tqo_encode(_ptr(x), n, d, bits, ctypes.c_uint64(seed), _ptr(packed),
                               _ptr(norms), _ptr(z))
        if rc != 0:
            raise ValueError("tqo_encode rejected its arguments (rc=%d)" % rc)
        return (packed, norms, z) if want_z else (packed, norms)

    def decode(self, packed, norms, d: int, bits: int, seed: int, want_f64: bool = False):
        """Returns the float16 decode [..., d] (and the unrounded float64 values)."""
        packed = _c(packed, np.uint8)
        norms = _c(norms, np.float32)
        lead = norms.shape
        n = int(np.prod(lead)) if lead else 1
        out = np.zeros(lead + (d,), dtype=np.uint16)
        xh = np.zeros(lead + (d,), dtype=np.float64) if want_f64 else None
        rc = self.L.tqo_decode(_ptr(packed), _ptr(norms), n, d, bits, ctypes.c_uint64(seed),
                               _ptr(out), _ptr(xh))
        if rc != 0:
            raise ValueError("tqo_decode rejected its arguments (rc=%d)" % rc)
        out = out.view(np.float16)
        return (out, xh) if want_f64 else out

    def attn_decode(self, q_f16, k_packed, k_norms, v_packed, v_norms, block_tables,
                    context_lens, num_kv_heads: int, bits: int, seed: int, scale: float,
                    sel=None, want_f64: bool = False, v_bits: int | None = None):
        """Plain paged decode attention.  q [B, Hq, d] float16; caches
        [num_blocks, block_size, Hkv, P] u8 and [num_blocks, block_size, Hkv] f32;
        block_tables [B, max_blocks] int32; context_lens [B] int32.
        sel (optional bool [B, Hq]) restricts the (b, h) pairs computed.
        v_bits (default: bits) is the width of the value codes."""
        q = np.asarray(q_f16)
        if q.dtype == np.float16:
            q = q.view(np.uint16)
        q = _c(q, np.uint16)
        B, Hq, d = q.shape
        k_packed = _c(k_packed, np.uint8)
        v_packed = _c(v_packed, np.uint8)
        k_norms = _c(k_norms, np.float32)
        v_norms = _c(v_norms, np.float32)
        nblk, bs, hkv = k_norms.shape
        assert hkv == num_kv_heads
        bt = _c(block_tables, np.int32)
        cl = _c(context_lens, np.int32)
        max_blocks = bt.shape[1] if bt.ndim == 2 else 0
        s = None if sel is None else _c(sel, np.uint8)
        out = np.zeros((B, Hq, d), dtype=np.uint16)
        of = np.zeros((B, Hq, d), dtype=np.float64) if want_f64 else None
        vb = bits if v_bits is None else v_bits
        rc = self.L.tqo_attn_decode_kv(_ptr(q), _ptr(k_packed), _ptr(k_norms), _ptr(v_packed),
                                       _ptr(v_norms), _ptr(bt), _ptr(cl), B, Hq, num_kv_heads,
                                       d, bits, vb, ctypes.c_uint64(seed), bs, max_blocks, nblk,
                                       float(scale), _ptr(s), _ptr(out), _ptr(of))
        if rc != 0:
            raise ValueError("tqo_attn_decode_kv rejected its arguments (rc=%d)" % rc)
        out = out.view(np.float16)
        return (out, of) if want_f64 else out


def _hybrid_mode(mode) -> int:
    if mode not in HYBRID_MODES:
        raise ValueError("mode must be one of %s" % sorted(HYBRID_MODES))
    return HYBRID_MODES[mode]


def _hybrid_methods():
    def hybrid_packed_bytes(self, d: int, mode: str) -> int:
        return self.L.tqo_hybrid_packed_bytes(d, _hybrid_mode(mode))

    def hybrid_encode(self, x_f16, mode: str, seed: int, perm, want_z: bool = False,
                      want_t: bool = False):
        """Hybrid-mode encode of x [..., d] binary16 with channel permutation
        perm [d].  Returns packed [..., row] u8 (and z, t [..., d] f64)."""
        x = np.asarray(x_f16)
        if x.dtype == np.float16:
            x = x.view(np.uint16)
        x = _c(x, np.uint16)
        d = x.shape[-1]
        lead = x.shape[:-1]
        n = int(np.prod(lead)) if lead else 1
        row = self.hybrid_packed_bytes(d, mode)
        if row == 0:
            raise ValueError("unsupported head_dim %d" % d)
        packed = np.zeros(lead + (row,), dtype=np.uint8)
        z = np.zeros(lead + (d,), dtype=np.float64) if want_z else None
        t = np.zeros(lead + (d,), dtype=np.float64) if want_t else None
        pm = _c(perm, np.int32)
        rc = self.L.tqo_hybrid_encode(_ptr(x), n, d, _hybrid_mode(mode), ctypes.c_uint64(seed),
                                      _ptr(pm), _ptr(packed), _ptr(z), _ptr(t))
        if rc != 0:
            raise ValueError("tqo_hybrid_encode rejected its arguments (rc=%d)" % rc)
        res = (packed,)
        if want_z:
            res += (z,)
        if want_t:
            res += (t,)
        return res if len(res) > 1 else packed

    def hybrid_decode(self, packed, d: int, mode: str, seed: int, perm, want_f64: bool = False):
        """Returns the binary16 decode [..., d] (and the unrounded doubles)."""
        packed = _c(packed, np.uint8)
        lead = packed.shape[:-1]
        n = int(np.prod(lead)) if lead else 1
        out = np.zeros(lead + (d,), dtype=np.uint16)
        xh = np.zeros(lead + (d,), dtype=np.float64) if want_f64 else None
        pm = _c(perm, np.int32)
        rc = self.L.tqo_hybrid_decode(_ptr(packed), n, d, _hybrid_mode(mode),
                                      ctypes.c_uint64(seed), _ptr(pm), _ptr(out), _ptr(xh))
        if rc != 0:
            raise ValueError("tqo_hybrid_decode rejected its arguments (rc=%d)" % rc)
        out = out.view(np.float16)
        return (out, xh) if want_f64 else out

    return hybrid_packed_bytes, hybrid_encode, hybrid_decode


(Oracle.hybrid_packed_bytes, Oracle.hybrid_encode, Oracle.hybrid_decode) = _hybrid_methods()


def default() -> Oracle:
    """The oracle built from ``tq_oracle.c`` as committed."""
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = Oracle(_LIB_PATH)
    return _lib


def build_variant(src_text: str, out_path: str) -> Oracle:
    """Compile a modified copy of the oracle source (used by the tests that
    plant a mistake in the oracle and check that some pin catches it)."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-w", "-fPIC", "-shared",
                    "-o", out_path, c_path, "-lm"], check=True)
    return Oracle(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def __getattr__(name):
    # module-level shortcuts: oracle.encode(...) == oracle.default().encode(...)
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
