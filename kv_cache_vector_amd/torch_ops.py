"""libtq's entry points as torch custom operators (namespace kv_cache_vector).

Registered with torch.library.custom_op, each with a fake (meta) kernel that
gives output shapes and dtypes without running anything, so torch.compile
traces calls to them without graph breaks (aither-kvcache PyPI page, "API
Reference": the codec and the paged attention exposed as registered torch
operators).

    torch.ops.kv_cache_vector.tq_encode(x, bits, seed) -> (packed, norms)
    torch.ops.kv_cache_vector.tq_decode(packed, norms, bits, seed) -> x_hat
    torch.ops.kv_cache_vector.tq_encode_paged_(x, slots, cache_packed,
                                               cache_norms, bits, seed) -> ()
    torch.ops.kv_cache_vector.tq_attn_decode(q, k_packed, k_norms, v_packed,
                                             v_norms, block_tables,
                                             context_lens, bits, seed, scale,
                                             v_bits=-1) -> out
      (v_bits: width of the value codes; -1 means the same as the keys')
    torch.ops.kv_cache_vector.tq_hybrid_encode(x, mode, seed, perm) -> packed
    torch.ops.kv_cache_vector.tq_hybrid_decode(packed, mode, seed, perm) -> x_hat
      (hybrid modes: mode 35 or 25, head_dim 128, perm a host int32 tensor)

Every operator takes head_dim 64, 128 or 256, read off the tensors' last
dimension (the attention operator: at most 8 query heads per kv head at 256).
Seeds are unsigned 64-bit values; the schema's int is signed, so seeds at or
above 2^63 travel as their two's-complement int64 and are converted back.
The real kernels take GPU tensors only and call libtq on the current stream;
there is no host implementation.
"""
from __future__ import annotations

import torch

from . import _lib

CODEC_HEAD_DIMS = (64, 128, 256)
_U64 = 1 << 64


def seed_to_i64(seed: int) -> int:
    s = int(seed) % _U64
    return s - _U64 if s >= (1 << 63) else s


def _seed_u64(seed: int) -> int:
    return int(seed) % _U64


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _gpu(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (libtq has no host implementation)" % name)


def _packed_dim(head_dim: int, bits: int) -> int:
    # codes of one vector: head_dim * bits / 8 bytes (same rule as tq_packed_bytes)
    if head_dim not in CODEC_HEAD_DIMS or bits not in (2, 3, 4):
        raise ValueError("unsupported (head_dim=%d, bits=%d)" % (head_dim, bits))
    return head_dim * bits // 8


def _decoded_dim(packed: torch.Tensor, bits: int) -> int:
    # head_dim of packed rows of `bits`-bit codes
    if packed.dtype != torch.uint8 or packed.dim() < 1 or bits not in (2, 3, 4):
        raise ValueError("packed must be uint8 [..., head_dim*bits/8], bits 2, 3 or 4")
    D = packed.shape[-1] * 8 // bits
    if packed.shape[-1] * 8 % bits or D not in CODEC_HEAD_DIMS:
        raise ValueError("packed rows of %d bytes match no head_dim in %s at %d bits"
                         % (packed.shape[-1], CODEC_HEAD_DIMS, bits))
    return D


# ---------------------------------------------------------------------------
# encode / decode

@torch.library.custom_op("kv_cache_vector::tq_encode", mutates_args=())
def tq_encode(x: torch.Tensor, bits: int, seed: int) -> tuple[torch.Tensor, torch.Tensor]:
    _gpu(x, "x")
    if x.dtype != torch.float16 or x.dim() < 1:
        raise ValueError("x must be float16 [..., head_dim]")
    D = x.shape[-1]
    P = _packed_dim(D, bits)
    x = x.contiguous()
    lead = tuple(x.shape[:-1])
    n = x.numel() // D
    packed = torch.empty(lead + (P,), dtype=torch.uint8, device=x.device)
    norms = torch.empty(lead, dtype=torch.float32, device=x.device)
    _lib.check(_lib.tq_encode(x.data_ptr(), n, D, bits, _seed_u64(seed),
                              packed.data_ptr(), norms.data_ptr(), _stream(x.device)),
               "tq_encode")
    return packed, norms


@tq_encode.register_fake
def _(x, bits, seed):
    P = _packed_dim(x.shape[-1], bits)
    lead = tuple(x.shape[:-1])
    return x.new_empty(lead + (P,), dtype=torch.uint8), x.new_empty(lead, dtype=torch.float32)


@torch.library.custom_op("kv_cache_vector::tq_decode", mutates_args=())
def tq_decode(packed: torch.Tensor, norms: torch.Tensor, bits: int, seed: int) -> torch.Tensor:
    _gpu(packed, "packed")
    _gpu(norms, "norms")
    D = _decoded_dim(packed, bits)
    if norms.dtype != torch.float32 or tuple(norms.shape) != tuple(packed.shape[:-1]):
        raise ValueError("norms must be float32 with packed's leading shape")
    packed = packed.contiguous()
    norms = norms.contiguous()
    out = torch.empty(tuple(norms.shape) + (D,), dtype=torch.float16, device=packed.device)
    _lib.check(_lib.tq_decode(packed.data_ptr(), norms.data_ptr(), norms.numel(), D,
                              bits, _seed_u64(seed), out.data_ptr(), _stream(packed.device)),
               "tq_decode")
    return out


@tq_decode.register_fake
def _(packed, norms, bits, seed):
    return norms.new_empty(tuple(norms.shape) + (_decoded_dim(packed, bits),),
                           dtype=torch.float16)


# ---------------------------------------------------------------------------
# paged write

@torch.library.custom_op("kv_cache_vector::tq_encode_paged_",
                         mutates_args=("cache_packed", "cache_norms"))
def tq_encode_paged_(x: torch.Tensor, slots: torch.Tensor, cache_packed: torch.Tensor,
                     cache_norms: torch.Tensor, bits: int, seed: int) -> None:
    for t, name in ((x, "x"), (slots, "slots"), (cache_packed, "cache_packed"),
                    (cache_norms, "cache_norms")):
        _gpu(t, name)
    if x.dtype != torch.float16 or x.dim() < 1:
        raise ValueError("x must be float16 [..., head_dim]")
    D = x.shape[-1]
    P = _packed_dim(D, bits)
    if slots.dtype != torch.int64 or slots.numel() != x.numel() // D:
        raise ValueError("slots must be int64 with one entry per vector")
    if not (cache_packed.is_contiguous() and cache_norms.is_contiguous()):
        raise ValueError("the cache tensors must be contiguous")
    if cache_packed.dtype != torch.uint8 or cache_packed.shape[-1] != P:
        raise ValueError("cache_packed must be uint8 [..., %d]" % P)
    if cache_norms.dtype != torch.float32:
        raise ValueError("cache_norms must be float32")
    num_slots = cache_norms.numel()
    if cache_packed.numel() != num_slots * P:
        raise ValueError("cache_packed and cache_norms disagree on the number of rows")
    x = x.contiguous()
    slots = slots.contiguous()
    _lib.check(_lib.tq_encode_paged(x.data_ptr(), slots.data_ptr(), slots.numel(), D,
                                    bits, _seed_u64(seed), cache_packed.data_ptr(),
                                    cache_norms.data_ptr(), num_slots, _stream(x.device)),
               "tq_encode_paged")


@tq_encode_paged_.register_fake
def _(x, slots, cache_packed, cache_norms, bits, seed):
    return None


# ---------------------------------------------------------------------------
# decode attention

def check_attn_args(q, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                    bits: int, v_bits: int, out=None):
    """Validate the arguments of a decode-attention call before anything is
    launched: dtypes, shapes, one device for every tensor, and (when given) an
    output tensor the kernel may write batch * num_q_heads * head_dim binary16
    values into.  Works on tensors of any device (no GPU needed).  Returns
    (B, Hq, D, num_blocks, block_size, Hkv, max_blocks)."""
    if q.dim() != 3 or q.dtype != torch.float16:
        raise ValueError("query must be float16 [batch, num_q_heads, head_dim]")
    B, Hq, D = q.shape
    P = _packed_dim(D, bits)
    PV = _packed_dim(D, v_bits)
    if k_packed.dim() != 4:
        raise ValueError("k_packed must be [num_blocks, block_size, num_kv_heads, P]")
    nblk, bs, hkv, Pk = k_packed.shape
    if Pk != P or tuple(v_packed.shape) != (nblk, bs, hkv, PV):
        raise ValueError("k_packed / v_packed shape mismatch")
    if tuple(k_norms.shape) != (nblk, bs, hkv) or tuple(v_norms.shape) != (nblk, bs, hkv):
        raise ValueError("norms must be [num_blocks, block_size, num_kv_heads]")
    if k_packed.dtype != torch.uint8 or v_packed.dtype != torch.uint8 or \
            k_norms.dtype != torch.float32 or v_norms.dtype != torch.float32:
        raise ValueError("codes must be uint8 and norms float32")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise ValueError("block_tables [batch, max_blocks], context_lens [batch]")
    for t, name in ((k_packed, "k_packed"), (k_norms, "k_norms"), (v_packed, "v_packed"),
                    (v_norms, "v_norms"), (block_tables, "block_tables"),
                    (context_lens, "context_lens")):
        if t.device != q.device:
            raise ValueError("%s is on %s, the query on %s" % (name, t.device, q.device))
    if out is not None:
        if out.dtype != torch.float16 or tuple(out.shape) != (B, Hq, D):
            raise ValueError("out must be float16 [%d, %d, %d]" % (B, Hq, D))
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        if out.device != q.device:
            raise ValueError("out is on %s, the query on %s" % (out.device, q.device))
    return B, Hq, D, nblk, bs, hkv, block_tables.shape[1]


def attn_decode_into(out, q, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                     bits: int, v_bits: int, seed: int, scale: float) -> torch.Tensor:
    """Run tq_attn_decode_kv on the current stream, writing `out`.  The
    workspace comes from torch's caching allocator on every call, so calls on
    different streams never share one (the allocator orders its reuse on the
    stream that allocated it)."""
    for t, name in ((q, "query"), (k_packed, "k_packed"), (k_norms, "k_norms"),
                    (v_packed, "v_packed"), (v_norms, "v_norms"),
                    (block_tables, "block_tables"), (context_lens, "context_lens"), (out, "out")):
        _gpu(t, name)
    B, Hq, D, nblk, bs, hkv, maxb = check_attn_args(q, k_packed, k_norms, v_packed, v_norms,
                                                    block_tables, context_lens, bits, v_bits,
                                                    out)
    q, k_packed, v_packed = q.contiguous(), k_packed.contiguous(), v_packed.contiguous()
    k_norms, v_norms = k_norms.contiguous(), v_norms.contiguous()
    block_tables, context_lens = block_tables.contiguous(), context_lens.contiguous()
    nbytes = _lib.tq_attn_workspace_bytes(B, Hq, hkv, D, bs, maxb)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _lib.check(_lib.tq_attn_decode_kv(
        q.data_ptr(), k_packed.data_ptr(), k_norms.data_ptr(), v_packed.data_ptr(),
        v_norms.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, hkv,
        D, bits, v_bits, _seed_u64(seed), bs, maxb, nblk, float(scale), out.data_ptr(),
        ws.data_ptr(), ws.numel(), _stream(q.device)), "tq_attn_decode_kv")
    return out


@torch.library.custom_op("kv_cache_vector::tq_attn_decode", mutates_args=())
def tq_attn_decode(q: torch.Tensor, k_packed: torch.Tensor, k_norms: torch.Tensor,
                   v_packed: torch.Tensor, v_norms: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, bits: int, seed: int,
                   scale: float, v_bits: int = -1) -> torch.Tensor:
    vb = bits if v_bits < 0 else v_bits
    _gpu(q, "query")
    out = torch.empty_like(q, memory_format=torch.contiguous_format)
    return attn_decode_into(out, q, k_packed, k_norms, v_packed, v_norms, block_tables,
                            context_lens, bits, vb, seed, scale)


@tq_attn_decode.register_fake
def _(q, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens, bits, seed, scale,
      v_bits=-1):
    check_attn_args(q, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens, bits,
                    bits if v_bits < 0 else v_bits)
    return torch.empty_like(q, memory_format=torch.contiguous_format)


# ---------------------------------------------------------------------------
# hybrid modes (tq35 / tq25), head_dim 128; perm is a host int32 tensor of
# the 128 channels (group A = perm[:64])

def _hybrid_row(mode) -> int:
    # comparisons, not a dict lookup: under torch.compile mode may be a
    # symbolic int, which cannot be hashed
    if mode == 35:
        return 68
    if mode == 25:
        return 52
    raise ValueError("mode must be 35 (tq35) or 25 (tq25)")


def _host_perm(perm: torch.Tensor) -> torch.Tensor:
    if perm.device.type != "cpu" or perm.dtype != torch.int32 or tuple(perm.shape) != (128,):
        raise ValueError("perm must be a host int32 tensor of 128 channels")
    return perm.contiguous()


@torch.library.custom_op("kv_cache_vector::tq_hybrid_encode", mutates_args=())
def tq_hybrid_encode(x: torch.Tensor, mode: int, seed: int, perm: torch.Tensor) -> torch.Tensor:
    _gpu(x, "x")
    if x.dtype != torch.float16 or x.dim() < 1 or x.shape[-1] != 128:
        raise ValueError("x must be float16 [..., 128]")
    row = _hybrid_row(mode)
    perm = _host_perm(perm)
    x = x.contiguous()
    packed = torch.empty(tuple(x.shape[:-1]) + (row,), dtype=torch.uint8, device=x.device)
    _lib.check(_lib.tq_hybrid_encode(x.data_ptr(), x.numel() // 128, 128, mode, _seed_u64(seed),
                                     perm.data_ptr(), packed.data_ptr(), _stream(x.device)),
               "tq_hybrid_encode")
    return packed


@tq_hybrid_encode.register_fake
def _(x, mode, seed, perm):
    if x.shape[-1] != 128:
        raise ValueError("x must be [..., 128]")
    return x.new_empty(tuple(x.shape[:-1]) + (_hybrid_row(mode),), dtype=torch.uint8)


@torch.library.custom_op("kv_cache_vector::tq_hybrid_decode", mutates_args=())
def tq_hybrid_decode(packed: torch.Tensor, mode: int, seed: int,
                     perm: torch.Tensor) -> torch.Tensor:
    _gpu(packed, "packed")
    row = _hybrid_row(mode)
    if packed.dtype != torch.uint8 or packed.dim() < 1 or packed.shape[-1] != row:
        raise ValueError("packed must be uint8 [..., %d]" % row)
    perm = _host_perm(perm)
    packed = packed.contiguous()
    out = torch.empty(tuple(packed.shape[:-1]) + (128,), dtype=torch.float16,
                      device=packed.device)
    _lib.check(_lib.tq_hybrid_decode(packed.data_ptr(), packed.numel() // row, 128, mode,
                                     _seed_u64(seed), perm.data_ptr(), out.data_ptr(),
                                     _stream(packed.device)), "tq_hybrid_decode")
    return out


@tq_hybrid_decode.register_fake
def _(packed, mode, seed, perm):
    if packed.shape[-1] != _hybrid_row(mode):
        raise ValueError("packed rows of %d bytes are not mode %d's" % (packed.shape[-1], mode))
    return packed.new_empty(tuple(packed.shape[:-1]) + (128,), dtype=torch.float16)
