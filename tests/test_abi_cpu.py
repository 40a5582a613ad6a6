"""libtq on the CPU: the library loads, exports every entry point include/tq.h
declares, and its host-only parts behave (codebook and sign hooks against the
oracle, argument checks that return before anything is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from kv_cache_vector_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")

OK, INVAL, UNSUP, MISAL, WS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.SYMBOLS) == names


def test_version_and_status_strings(L):
    assert L.tq_abi_version() == 1
    for s, name in _lib.STATUS_NAMES.items():
        assert _lib.tq_status_string(s) == name


def test_packed_bytes(L):
    assert [_lib.tq_packed_bytes(128, b) for b in (2, 3, 4)] == [32, 48, 64]
    assert [_lib.tq_packed_bytes(64, b) for b in (2, 3, 4)] == [16, 24, 32]
    assert [_lib.tq_packed_bytes(256, b) for b in (2, 3, 4)] == [64, 96, 128]
    assert _lib.tq_packed_bytes(128, 5) == 0
    assert _lib.tq_packed_bytes(96, 4) == 0
    assert _lib.tq_packed_bytes(32, 4) == 0
    assert _lib.tq_packed_bytes(512, 4) == 0
    assert _lib.tq_packed_bytes(128, 1) == 0


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_hook_matches_oracle(L, bits):
    """libtq solves the Lloyd-Max conditions with its own solver (extended
    precision, iterating on the decision points); the oracle iterates on the
    levels in double.  Both must land on the same f32 values."""
    lv, th = _lib.tq_codebook(bits)
    c, t = oracle.codebook(bits)
    assert np.array_equal(np.array(lv, np.float32), c.astype(np.float32))
    assert np.array_equal(np.array(th, np.float32), t.astype(np.float32))
    lvf = np.array(lv, np.float32)
    assert np.all(np.abs(lvf.astype(np.float64) - c) <= 0.5 * np.spacing(np.abs(lvf)))
    assert th[len(th) // 2] == 0.0


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("seed", [0, 1, 42, 2 ** 64 - 1])
def test_sign_hook_matches_oracle(L, seed, d):
    words = _lib.tq_signs(seed, d)
    assert len(words) == d // 32
    s = oracle.signs(seed, d)
    bits = np.array([(words[i // 32] >> (i % 32)) & 1 for i in range(d)])
    assert np.array_equal(bits, (s < 0).astype(int))


def test_hook_errors(L):
    buf = (ctypes.c_float * 16)()
    assert L.tq_codebook(5, buf, buf) == UNSUP
    assert L.tq_codebook(4, None, buf) == INVAL
    assert L.tq_signs(0, 96, buf) == UNSUP
    assert L.tq_signs(0, 512, buf) == UNSUP
    assert L.tq_signs(0, 128, None) == INVAL


# Fake device addresses: every call below must be rejected (or be a no-op)
# before anything touches them or the GPU.
A = 0x10000000
B = 0x20000000
C = 0x30000000


def test_encode_argument_errors(L):
    e = L.tq_encode
    assert e(A, 10, 128, 5, 0, B, C, None) == UNSUP
    assert e(A, 10, 96, 4, 0, B, C, None) == UNSUP
    assert e(A, 10, 0, 4, 0, B, C, None) == INVAL
    assert e(A, -1, 128, 4, 0, B, C, None) == INVAL
    assert e(A, 0, 128, 4, 0, B, C, None) == OK          # n == 0: nothing to do
    assert e(None, 0, 128, 4, 0, None, None, None) == OK
    assert e(None, 10, 128, 4, 0, B, C, None) == INVAL
    assert e(A, 10, 128, 4, 0, None, C, None) == INVAL
    assert e(A, 10, 128, 4, 0, B, None, None) == INVAL
    assert e(A + 8, 10, 128, 4, 0, B, C, None) == MISAL
    assert e(A, 10, 128, 4, 0, B + 4, C, None) == MISAL
    assert e(A, 10, 128, 4, 0, B, C + 2, None) == MISAL
    # overlapping input and output ranges
    assert e(A, 10, 128, 4, 0, A + 256, C, None) == INVAL
    assert e(A, 10, 128, 4, 0, B, B + 9 * 64, None) == INVAL
    # the ranges scale with head_dim: 10 vectors of 256 are 5120 bytes
    assert e(A, 10, 256, 4, 0, A + 5120 - 16, C, None) == INVAL
    assert e(A, 10, 256, 4, 0, B, B + 9 * 128, None) == INVAL
    assert e(A, 10, 64, 4, 0, B, B + 9 * 32, None) == INVAL
    assert e(A, 10, 512, 4, 0, B, C, None) == UNSUP
    assert e(A, 10, 32, 4, 0, B, C, None) == UNSUP


def test_decode_argument_errors(L):
    d = L.tq_decode
    assert d(B, C, 10, 128, 1, 0, A, None) == UNSUP
    assert d(B, C, -5, 128, 4, 0, A, None) == INVAL
    assert d(B, C, 0, 128, 4, 0, A, None) == OK
    assert d(None, C, 10, 128, 4, 0, A, None) == INVAL
    assert d(B, C, 10, 128, 4, 0, A + 2, None) == MISAL
    assert d(B, C, 10, 128, 4, 0, B + 64, None) == INVAL   # output overlaps codes
    assert d(B, C, 10, 256, 4, 0, C - 5120 + 16, None) == INVAL   # output overlaps norms
    assert d(B, C, 10, 96, 4, 0, A, None) == UNSUP


def test_paged_encode_argument_errors(L):
    p = L.tq_encode_paged
    assert p(A, B, 4, 128, 6, 0, C, C + 4096, 100, None) == UNSUP
    assert p(A, B, 4, 128, 4, 0, C, C + 1 << 20, -1, None) == INVAL
    assert p(A, B, 0, 128, 4, 0, C, C + 4096, 100, None) == OK
    assert p(A, None, 4, 128, 4, 0, C, C + 8192, 100, None) == INVAL
    assert p(A, B + 4, 4, 128, 4, 0, C, C + 8192, 100, None) == MISAL
    assert p(A, B, 4, 128, 4, 0, C, C + 64, 100, None) == INVAL   # packed overlaps norms
    assert p(A, B, 4, 256, 4, 0, C, C + 128 * 99, 100, None) == INVAL
    assert p(A, B, 4, 96, 4, 0, C, C + 1 << 20, 100, None) == UNSUP


def test_attention_argument_errors(L):
    ws = L.tq_attn_workspace_bytes(16, 32, 8, 128, 16, 2048)
    assert ws > 0 and ws % 16 == 0
    assert L.tq_attn_workspace_bytes(16, 32, 8, 96, 16, 2048) == 0
    assert L.tq_attn_workspace_bytes(16, 30, 8, 128, 16, 2048) == 0
    # group sizes: at most 16 query heads per kv head, 8 at head_dim 256
    assert L.tq_attn_workspace_bytes(16, 128, 8, 128, 16, 2048) > 0
    assert L.tq_attn_workspace_bytes(16, 136, 8, 128, 16, 2048) == 0
    assert L.tq_attn_workspace_bytes(16, 64, 8, 256, 16, 2048) > 0
    assert L.tq_attn_workspace_bytes(16, 72, 8, 256, 16, 2048) == 0
    # one f32 entry of 2 + head_dim floats per (sequence, query head, split)
    for d in (64, 256):
        wd = L.tq_attn_workspace_bytes(16, 32, 8, d, 16, 2048)
        assert wd > 0 and wd % 16 == 0
        assert wd % (16 * 32 * (2 + d) * 4) == 0
    a = L.tq_attn_decode

    def call(**kw):
        args = dict(q=A, kp=B, kn=B + (1 << 24), vp=C, vn=C + (1 << 24), bt=A + (1 << 24),
                    cl=A + (1 << 25), batch=16, hq=32, hkv=8, d=128, bits=4, seed=0, bs=16,
                    maxb=2048, nblk=32768, scale=0.088, out=A + (1 << 26), ws=0x40000000,
                    wsb=ws)
        args.update(kw)
        return a(args["q"], args["kp"], args["kn"], args["vp"], args["vn"], args["bt"],
                 args["cl"], args["batch"], args["hq"], args["hkv"], args["d"], args["bits"],
                 args["seed"], args["bs"], args["maxb"], args["nblk"], args["scale"],
                 args["out"], args["ws"], args["wsb"], None)

    assert call(bits=5) == UNSUP
    assert call(d=96) == UNSUP
    assert call(d=512) == UNSUP
    assert call(d=64, batch=0) == OK
    assert call(d=256, hq=8 * 9) == UNSUP          # head_dim 256: at most 8 query heads per kv head
    assert call(d=256, hq=8 * 8, batch=0) == OK
    # launch extents: sequences on the grid's y axis, tokens per sequence in an int
    assert call(batch=65536) == UNSUP
    assert call(maxb=(2 ** 31 - 1) // 16 + 1) == UNSUP
    assert call(batch=65535, hq=2049 * 16, hkv=2049) == UNSUP     # batch * hq > 2^31 - 1
    assert L.tq_attn_workspace_bytes(65536, 32, 8, 128, 16, 2048) == 0
    assert L.tq_attn_workspace_bytes(16, 32, 8, 128, 16, (2 ** 31 - 1) // 16 + 1) == 0
    assert call(bs=32) == UNSUP
    assert call(hq=30) == INVAL
    assert call(hq=8 * 17) == UNSUP                 # 17 query heads per kv head
    assert call(hq=8 * 17, bits=2) == UNSUP
    assert call(batch=-1) == INVAL
    assert call(scale=float("nan")) == INVAL
    assert call(batch=0) == OK
    assert call(q=None) == INVAL
    assert call(out=A + (1 << 26) + 2) == MISAL
    assert call(ws=None) == WS
    assert call(wsb=ws - 16) == WS
    assert call(out=A) == INVAL                     # output overlaps the query
    assert call(out=B + 1024) == INVAL              # output overlaps the packed keys
    assert call(out=A + (1 << 24)) == INVAL         # output overlaps the block tables
    assert call(ws=C + (1 << 24)) == INVAL          # workspace overlaps the value norms
    assert call(ws=A + (1 << 25)) == INVAL          # workspace overlaps the context lengths
    assert call(ws=A + (1 << 26)) == INVAL          # workspace overlaps the output

    # keys and values at different widths
    kv = L.tq_attn_decode_kv

    def call_kv(kb, vb, **kw):
        args = dict(q=A, kp=B, kn=B + (1 << 24), vp=C, vn=C + (1 << 24), bt=A + (1 << 24),
                    cl=A + (1 << 25), batch=16, hq=32, hkv=8, d=128, seed=0, bs=16,
                    maxb=2048, nblk=32768, scale=0.088, out=A + (1 << 26), ws=0x40000000,
                    wsb=ws)
        args.update(kw)
        return kv(args["q"], args["kp"], args["kn"], args["vp"], args["vn"], args["bt"],
                  args["cl"], args["batch"], args["hq"], args["hkv"], args["d"], kb, vb,
                  args["seed"], args["bs"], args["maxb"], args["nblk"], args["scale"],
                  args["out"], args["ws"], args["wsb"], None)

    assert call_kv(4, 5) == UNSUP
    assert call_kv(1, 2) == UNSUP
    assert call_kv(4, 2, d=96) == UNSUP
    assert call_kv(4, 2, d=64, batch=0) == OK
    assert call_kv(4, 2, batch=0) == OK
    assert call_kv(2, 4, q=None) == INVAL
    assert call_kv(3, 4, wsb=ws - 16) == WS


def test_noalloc_attention_argument_errors(L):
    """The allocation-free attention entry point checks its arguments like
    tq_attn_decode_kv, and refuses shapes whose partial state does not fit its
    fixed array, all before anything touches the GPU."""
    f = L.tq_attn_decode_kv_noalloc

    def call(kb=4, vb=4, **kw):
        args = dict(q=A, kp=B, kn=B + (1 << 24), vp=C, vn=C + (1 << 24), bt=A + (1 << 24),
                    cl=A + (1 << 25), batch=16, hq=32, hkv=8, d=128, seed=0, bs=16,
                    maxb=2048, nblk=32768, scale=0.088, out=A + (1 << 26))
        args.update(kw)
        return f(args["q"], args["kp"], args["kn"], args["vp"], args["vn"], args["bt"],
                 args["cl"], args["batch"], args["hq"], args["hkv"], args["d"], kb, vb,
                 args["seed"], args["bs"], args["maxb"], args["nblk"], args["scale"],
                 args["out"], None)

    assert call(kb=5) == UNSUP
    assert call(d=96) == UNSUP
    assert call(batch=0) == OK
    assert call(q=None) == INVAL
    assert call(out=A + (1 << 26) + 2) == MISAL
    assert call(out=A) == INVAL                     # output overlaps the query
    assert call(bs=32) == UNSUP
    # the fixed array: 32 MiB per GPU
    assert _lib.TQ_ATTN_NOALLOC_WORKSPACE_BYTES == 32 << 20
    need = L.tq_attn_workspace_bytes(512, 64, 8, 128, 16, 1024)
    assert need > _lib.TQ_ATTN_NOALLOC_WORKSPACE_BYTES
    assert call(batch=512, hq=64, maxb=1024, nblk=512 * 1024, out=0x70000000) == WS
    header = open(HEADER).read()
    assert "#define TQ_ATTN_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)" in header


def test_every_header_symbol_is_exported(L):
    """libtq exports every function any include/*.h declares (the codec ABI
    and the measurement hook of tq_ceiling.h)."""
    import glob
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names = sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))
        assert names, h
        for n in names:
            assert hasattr(L, n), (h, n)


def test_ceiling_hook_argument_errors(L):
    f = L.tq_ceiling_stream
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert f(2, 64, A, None, 10, B, C, None) == 1          # no such mode
    assert f(0, 40, A, None, 10, B, C, None) == 1          # packed bytes of no width
    assert f(0, 64, A, None, -1, B, C, None) == 1
    assert f(0, 64, A, None, 0, B, C, None) == 0           # nothing to do
    assert f(0, 64, A, None, 10, B, None, None) == 1       # encode mix needs the norm output
    assert f(1, 64, A, None, 10, B, None, None) == 1       # decode mix needs the norm input


def test_hybrid_argument_errors(L):
    """The hybrid entry points check their arguments on the host, including
    the channel permutation, before anything touches the GPU."""
    assert L.tq_hybrid_packed_bytes(128, 35) == 68 and L.tq_hybrid_packed_bytes(128, 25) == 52
    assert L.tq_hybrid_packed_bytes(64, 35) == 0 and L.tq_hybrid_packed_bytes(128, 40) == 0
    ident = np.arange(128, dtype=np.int32)
    dup = ident.copy()
    dup[5] = 4
    out_of_range = ident.copy()
    out_of_range[0] = 128
    e, dcd = L.tq_hybrid_encode, L.tq_hybrid_decode
    p = ident.ctypes.data
    assert e(A, 10, 128, 30, 0, p, B, None) == UNSUP
    assert e(A, 10, 64, 35, 0, p, B, None) == UNSUP
    assert e(A, -1, 128, 35, 0, p, B, None) == INVAL
    assert e(A, 0, 128, 35, 0, p, B, None) == OK
    assert e(A, 10, 128, 35, 0, dup.ctypes.data, B, None) == INVAL
    assert e(A, 10, 128, 35, 0, out_of_range.ctypes.data, B, None) == INVAL
    assert e(None, 10, 128, 35, 0, p, B, None) == INVAL
    assert e(A + 8, 10, 128, 35, 0, p, B, None) == MISAL
    assert e(A, 10, 128, 35, 0, p, B + 2, None) == MISAL
    assert e(A, 10, 128, 35, 0, p, A + 1024, None) == INVAL      # rows overlap the input
    assert dcd(B, 10, 128, 25, 0, p, A + 4, None) == MISAL
    assert dcd(B, 10, 128, 25, 0, dup.ctypes.data, A, None) == INVAL
    assert dcd(B, 10, 128, 25, 0, p, B + 64, None) == INVAL       # output overlaps the rows
    assert dcd(B, 0, 128, 25, 0, None, A, None) == OK
