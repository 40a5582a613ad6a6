"""ctypes binding of libtq (include/tq.h): the same entry points, same names.

Argument marshalling only -- every step of the codec runs in libtq's HIP
kernels.  The library is loaded from this package's directory; if it is
missing, ``load()`` raises (there is no other implementation to fall back to).
torch is imported first so that libtq binds to the HIP runtime torch already
loaded, and device pointers and streams from torch are valid in libtq.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK = 0
STATUS_NAMES = {0: "TQ_OK", 1: "TQ_ERR_INVALID_ARG", 2: "TQ_ERR_UNSUPPORTED",
                3: "TQ_ERR_MISALIGNED", 4: "TQ_ERR_WORKSPACE", 5: "TQ_ERR_HIP"}

# every symbol include/tq.h declares
SYMBOLS = ("tq_status_string", "tq_abi_version", "tq_packed_bytes", "tq_encode", "tq_decode",
           "tq_encode_paged", "tq_attn_workspace_bytes", "tq_attn_decode", "tq_attn_decode_kv",
           "tq_attn_decode_kv_noalloc", "tq_hybrid_packed_bytes", "tq_hybrid_encode",
           "tq_hybrid_decode", "tq_codebook", "tq_signs")

# bytes of the library-owned workspace of tq_attn_decode_kv_noalloc, per GPU
# (TQ_ATTN_NOALLOC_WORKSPACE_BYTES in include/tq.h)
TQ_ATTN_NOALLOC_WORKSPACE_BYTES = 32 << 20

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_U64 = ctypes.c_uint64
_lock = threading.Lock()
_lib = None


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, STATUS_NAMES.get(status, status)))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open libtq.so (once).  Raises FileNotFoundError when it was not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise FileNotFoundError(
                "libtq.so not found at %s: build it with `python -m kv_cache_vector_amd.build`"
                % path)
        import torch  # noqa: F401  -- binds libtq to torch's HIP runtime
        L = ctypes.CDLL(path)
        L.tq_status_string.argtypes = [_I]
        L.tq_status_string.restype = ctypes.c_char_p
        L.tq_abi_version.argtypes = []
        L.tq_packed_bytes.argtypes = [_I, _I]
        L.tq_packed_bytes.restype = ctypes.c_size_t
        L.tq_encode.argtypes = [_P, _I64, _I, _I, _U64, _P, _P, _P]
        L.tq_decode.argtypes = [_P, _P, _I64, _I, _I, _U64, _P, _P]
        L.tq_encode_paged.argtypes = [_P, _P, _I64, _I, _I, _U64, _P, _P, _I64, _P]
        L.tq_attn_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
        L.tq_attn_workspace_bytes.restype = ctypes.c_size_t
        L.tq_attn_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _U64, _I,
                                     _I, _I64, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
        L.tq_attn_decode_kv.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _U64,
                                        _I, _I, _I64, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
        L.tq_attn_decode_kv_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                                _I, _U64, _I, _I, _I64, ctypes.c_float, _P, _P]
        L.tq_hybrid_packed_bytes.argtypes = [_I, _I]
        L.tq_hybrid_packed_bytes.restype = ctypes.c_size_t
        L.tq_hybrid_encode.argtypes = [_P, _I64, _I, _I, _U64, _P, _P, _P]
        L.tq_hybrid_decode.argtypes = [_P, _I64, _I, _I, _U64, _P, _P, _P]
        L.tq_codebook.argtypes = [_I, _P, _P]
        L.tq_signs.argtypes = [_U64, _I, _P]
        _lib = L
        return L


def check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where)


# thin same-name wrappers (integers are device addresses; stream is a hipStream_t)

def tq_packed_bytes(head_dim: int, bits: int) -> int:
    return load().tq_packed_bytes(head_dim, bits)


def tq_encode(x_f16, n, head_dim, bits, seed, packed, norms, stream) -> int:
    return load().tq_encode(x_f16, n, head_dim, bits, seed, packed, norms, stream)


def tq_decode(packed, norms, n, head_dim, bits, seed, out_f16, stream) -> int:
    return load().tq_decode(packed, norms, n, head_dim, bits, seed, out_f16, stream)


def tq_encode_paged(x_f16, slots, n, head_dim, bits, seed, cache_packed, cache_norms,
                    num_slots, stream) -> int:
    return load().tq_encode_paged(x_f16, slots, n, head_dim, bits, seed, cache_packed,
                                  cache_norms, num_slots, stream)


def tq_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq) -> int:
    return load().tq_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                          block_size, max_blocks_per_seq)


def tq_attn_decode(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                   batch, num_q_heads, num_kv_heads, head_dim, bits, seed, block_size,
                   max_blocks_per_seq, num_blocks, scale, out_f16, workspace, workspace_bytes,
                   stream) -> int:
    return load().tq_attn_decode(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables,
                                 context_lens, batch, num_q_heads, num_kv_heads, head_dim, bits,
                                 seed, block_size, max_blocks_per_seq, num_blocks, scale,
                                 out_f16, workspace, workspace_bytes, stream)


def tq_attn_decode_kv(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                      batch, num_q_heads, num_kv_heads, head_dim, k_bits, v_bits, seed,
                      block_size, max_blocks_per_seq, num_blocks, scale, out_f16, workspace,
                      workspace_bytes, stream) -> int:
    return load().tq_attn_decode_kv(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables,
                                    context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                    k_bits, v_bits, seed, block_size, max_blocks_per_seq,
                                    num_blocks, scale, out_f16, workspace, workspace_bytes,
                                    stream)


def tq_attn_decode_kv_noalloc(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables,
                              context_lens, batch, num_q_heads, num_kv_heads, head_dim, k_bits,
                              v_bits, seed, block_size, max_blocks_per_seq, num_blocks, scale,
                              out_f16, stream) -> int:
    return load().tq_attn_decode_kv_noalloc(q_f16, k_packed, k_norms, v_packed, v_norms,
                                            block_tables, context_lens, batch, num_q_heads,
                                            num_kv_heads, head_dim, k_bits, v_bits, seed,
                                            block_size, max_blocks_per_seq, num_blocks, scale,
                                            out_f16, stream)


def tq_hybrid_packed_bytes(head_dim, mode) -> int:
    return load().tq_hybrid_packed_bytes(head_dim, mode)


def tq_hybrid_encode(x_f16, n, head_dim, mode, seed, perm, packed, stream) -> int:
    """perm: a HOST pointer (or None) to head_dim int32."""
    return load().tq_hybrid_encode(x_f16, n, head_dim, mode, seed, perm, packed, stream)


def tq_hybrid_decode(packed, n, head_dim, mode, seed, perm, out_f16, stream) -> int:
    return load().tq_hybrid_decode(packed, n, head_dim, mode, seed, perm, out_f16, stream)


def tq_codebook(bits: int):
    """(levels, thresholds) as Python float lists (f32 values)."""
    L = 1 << bits
    lv = (ctypes.c_float * L)()
    th = (ctypes.c_float * max(L - 1, 1))()
    check(load().tq_codebook(bits, lv, th), "tq_codebook")
    return list(lv), list(th)[: L - 1]


def tq_signs(seed: int, head_dim: int = 128):
    """The sign mask words (bit i of word i//32 set iff sigma_i = -1)."""
    m = (ctypes.c_uint32 * (head_dim // 32))()
    check(load().tq_signs(seed, head_dim, m), "tq_signs")
    return list(m)


def tq_status_string(status: int) -> str:
    return load().tq_status_string(status).decode()
