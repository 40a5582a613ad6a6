"""torch-facing wrappers over libtq, shaped like the Python objects the pages
describe (aither-kvcache PyPI page, "API Reference": TurboQuant(head_dim,
bits, seed, device) with encode / decode / compression_ratio / validate /
benchmark, and TQPagedAttention(tq, num_query_heads).forward(...)).

torch provides device memory and the current stream; every step of the codec
runs in libtq's HIP kernels.  CPU tensors are rejected: there is no host
implementation in the product.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from . import torch_ops  # registers torch.ops.kv_cache_vector.*

HEAD_DIM = 128


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require_gpu(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (libtq has no host implementation)" % name)


class TurboQuant:
    """TurboQuant codec: [..., head_dim] fp16 <-> ([..., head_dim*bits/8] uint8, [...] f32),
    head_dim 64, 128 or 256."""

    def __init__(self, head_dim: int = HEAD_DIM, bits: int = 4, seed: int = 42,
                 device="cuda"):
        if _lib.tq_packed_bytes(head_dim, bits) == 0:
            raise ValueError("unsupported (head_dim=%d, bits=%d)" % (head_dim, bits))
        self.head_dim = head_dim
        self.bits = bits
        self.seed = int(seed) & (2 ** 64 - 1)
        self.device = torch.device(device)
        if self.device.type != "cuda":
            raise ValueError("TurboQuant runs on the GPU only")

    @property
    def packed_dim(self) -> int:
        return self.head_dim * self.bits // 8

    def compression_ratio(self) -> float:
        """Bytes of fp16 against bytes of codes plus the f32 norm."""
        return 2.0 * self.head_dim / (self.packed_dim + 4)

    def encode(self, x: torch.Tensor):
        """x [..., head_dim] fp16 -> (packed [..., head_dim*bits/8] uint8, norms [...] f32),
        through torch.ops.kv_cache_vector.tq_encode."""
        _require_gpu(x, "x")
        if x.dtype != torch.float16 or x.shape[-1] != self.head_dim:
            raise ValueError("x must be float16 [..., %d]" % self.head_dim)
        return torch.ops.kv_cache_vector.tq_encode(x, self.bits, torch_ops.seed_to_i64(self.seed))

    def decode(self, packed: torch.Tensor, norms: torch.Tensor) -> torch.Tensor:
        """Inverse of encode, through torch.ops.kv_cache_vector.tq_decode."""
        _require_gpu(packed, "packed")
        _require_gpu(norms, "norms")
        if packed.dtype != torch.uint8 or packed.shape[-1] != self.packed_dim:
            raise ValueError("packed must be uint8 [..., %d]" % self.packed_dim)
        if norms.dtype != torch.float32 or tuple(norms.shape) != tuple(packed.shape[:-1]):
            raise ValueError("norms must be float32 with packed's leading shape")
        return torch.ops.kv_cache_vector.tq_decode(packed, norms, self.bits,
                                                   torch_ops.seed_to_i64(self.seed))

    def encode_into(self, x: torch.Tensor, slots: torch.Tensor, cache_packed: torch.Tensor,
                    cache_norms: torch.Tensor) -> None:
        """Encode x [n, head_dim] into rows `slots` [n] (int64) of a paged cache
        ([num_blocks, block_size, Hkv, P] uint8 and [num_blocks, block_size, Hkv]
        f32, rows counted as (block*block_size + offset)*Hkv + kv_head)."""
        for t, name in ((x, "x"), (slots, "slots"), (cache_packed, "cache_packed"),
                        (cache_norms, "cache_norms")):
            _require_gpu(t, name)
        if x.dtype != torch.float16 or x.shape[-1] != self.head_dim:
            raise ValueError("x must be float16 [..., %d]" % self.head_dim)
        if slots.dtype != torch.int64 or slots.numel() != x.numel() // self.head_dim:
            raise ValueError("slots must be int64 with one entry per vector")
        if not (cache_packed.is_contiguous() and cache_norms.is_contiguous()):
            raise ValueError("the cache tensors must be contiguous")
        if cache_packed.shape[-1] != self.packed_dim or cache_packed.dtype != torch.uint8:
            raise ValueError("cache_packed must be uint8 [..., %d]" % self.packed_dim)
        num_slots = cache_norms.numel()
        if cache_packed.numel() != num_slots * self.packed_dim:
            raise ValueError("cache_packed and cache_norms disagree on the number of rows")
        x = x.contiguous()
        slots = slots.contiguous()
        _lib.check(_lib.tq_encode_paged(x.data_ptr(), slots.data_ptr(), slots.numel(),
                                        self.head_dim, self.bits, self.seed,
                                        cache_packed.data_ptr(), cache_norms.data_ptr(),
                                        num_slots, _stream(x.device)), "tq_encode_paged")

    def validate(self, num_vectors: int = 10000, seed: int = 0) -> dict:
        """Round-trip MSE on N(0,1) vectors, per coordinate of the unit vector
        (||x - xhat||^2 / ||x||^2), next to the 4^-bits lower bound."""
        g = torch.Generator(device=self.device).manual_seed(seed)
        x = torch.randn(num_vectors, self.head_dim, generator=g, device=self.device).half()
        y = self.decode(*self.encode(x)).float()
        xf = x.float()
        mse = float((((xf - y) ** 2).sum(1) / (xf ** 2).sum(1)).mean())
        bound = 4.0 ** (-self.bits)
        return {"mse": mse, "lower_bound": bound, "ratio_to_bound": mse / bound,
                "num_vectors": num_vectors, "bits": self.bits}

    def benchmark(self, num_vectors: int = 32768, iters: int = 20) -> dict:
        """Kernel time of encode and decode on random fp16 vectors."""
        x = torch.randn(num_vectors, self.head_dim, device=self.device).half()
        packed, norms = self.encode(x)
        out = self.decode(packed, norms)
        res = {}
        for name, fn in (("encode", lambda: self.encode(x)),
                         ("decode", lambda: self.decode(packed, norms))):
            fn()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(iters):
                fn()
            e.record()
            e.synchronize()
            ms = s.elapsed_time(e) / iters
            res[name + "_ms"] = ms
            res[name + "_fp16_GBps"] = num_vectors * self.head_dim * 2 / ms / 1e6
        del out
        return res


class TQPagedAttention:
    """Single-token decode attention straight from the packed, paged cache.
    Keys are in `tq`'s format; values in `v_tq`'s (default: the same codec).
    A separate value codec may use another bit width (e.g. 4-bit keys, 2-bit
    values) but must share the seed, i.e. the rotation."""

    def __init__(self, tq: TurboQuant, num_query_heads: int, scale: float | None = None,
                 v_tq: TurboQuant | None = None):
        self.tq = tq
        self.v_tq = tq if v_tq is None else v_tq
        if self.v_tq.seed != tq.seed or self.v_tq.head_dim != tq.head_dim:
            raise ValueError("keys and values must share head_dim and seed")
        self.num_query_heads = num_query_heads
        self.scale = (1.0 / math.sqrt(tq.head_dim)) if scale is None else float(scale)
        self._ws = {}

    def workspace(self, batch: int, num_kv_heads: int, max_blocks: int, block_size: int,
                  device) -> torch.Tensor:
        nbytes = _lib.tq_attn_workspace_bytes(batch, self.num_query_heads, num_kv_heads,
                                              self.tq.head_dim, block_size, max_blocks)
        key = (str(device), nbytes)
        ws = self._ws.get(key)
        if ws is None:
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
            self._ws = {key: ws}
        return ws

    def forward(self, query, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                block_size: int = 16, out: torch.Tensor | None = None) -> torch.Tensor:
        for t, name in ((query, "query"), (k_packed, "k_packed"), (k_norms, "k_norms"),
                        (v_packed, "v_packed"), (v_norms, "v_norms"),
                        (block_tables, "block_tables"), (context_lens, "context_lens")):
            _require_gpu(t, name)
        tq = self.tq
        B, Hq, D = query.shape
        if Hq != self.num_query_heads or D != tq.head_dim or query.dtype != torch.float16:
            raise ValueError("query must be float16 [batch, %d, %d]" % (self.num_query_heads,
                                                                         tq.head_dim))
        if k_packed.dim() != 4 or k_packed.shape[1] != block_size:
            raise ValueError("k_packed must be [num_blocks, block_size, num_kv_heads, P]")
        nblk, _, hkv, P = k_packed.shape
        if P != tq.packed_dim or \
                tuple(v_packed.shape) != (nblk, block_size, hkv, self.v_tq.packed_dim):
            raise ValueError("k_packed / v_packed shape mismatch")
        if tuple(k_norms.shape) != (nblk, block_size, hkv) or \
                tuple(v_norms.shape) != (nblk, block_size, hkv):
            raise ValueError("norms must be [num_blocks, block_size, num_kv_heads]")
        if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
            raise ValueError("block_tables and context_lens must be int32")
        if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
            raise ValueError("block_tables [batch, max_blocks], context_lens [batch]")
        query, k_packed, v_packed = query.contiguous(), k_packed.contiguous(), v_packed.contiguous()
        k_norms, v_norms = k_norms.contiguous(), v_norms.contiguous()
        block_tables, context_lens = block_tables.contiguous(), context_lens.contiguous()
        maxb = block_tables.shape[1]
        if out is None:
            out = torch.empty_like(query)
        ws = self.workspace(B, hkv, maxb, block_size, query.device)
        _lib.check(_lib.tq_attn_decode_kv(
            query.data_ptr(), k_packed.data_ptr(), k_norms.data_ptr(), v_packed.data_ptr(),
            v_norms.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, hkv,
            tq.head_dim, tq.bits, self.v_tq.bits, tq.seed, block_size, maxb, nblk, self.scale,
            out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(query.device)),
            "tq_attn_decode_kv")
        return out

    __call__ = forward
