"""torch-facing wrappers over libtq, shaped like the Python objects the pages
describe (aither-kvcache PyPI page, "API Reference": TurboQuant(head_dim,
bits, seed, device) with encode / decode / compression_ratio / validate /
benchmark, HybridTurboQuant(head_dim, mode, seed, device) with
calibrate_uniform / calibrate / encode / decode / validate /
compression_ratio / packed_dim_for_mode, and
TQPagedAttention(tq, num_query_heads).forward(...)).

torch provides device memory and the current stream; every step of the codec
runs in libtq's HIP kernels.  CPU tensors are rejected: there is no host
implementation in the product.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _lib
from . import torch_ops  # registers torch.ops.kv_cache_vector.*

HEAD_DIM = 128


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require_gpu(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (libtq has no host implementation)" % name)


def verify_slots(slots: torch.Tensor, num_slots: int) -> None:
    """Raise ValueError unless the non-negative entries of `slots` are
    distinct and below num_slots (negative entries mark skipped vectors):
    the paged write's contract, which its kernel does not check (an
    out-of-range slot is skipped, duplicates race)."""
    s = slots.reshape(-1)
    s = s[s >= 0]
    if s.numel() == 0:
        return
    top = int(s.max())
    if top >= num_slots:
        raise ValueError("slot %d is past the cache's %d rows" % (top, num_slots))
    if torch.unique(s).numel() != s.numel():
        raise ValueError("slots must be distinct (duplicate rows would race)")


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
                    cache_norms: torch.Tensor, check_slots: bool = False) -> None:
        """Encode x [n, head_dim] into rows `slots` [n] (int64) of a paged cache
        ([num_blocks, block_size, Hkv, P] uint8 and [num_blocks, block_size, Hkv]
        f32, rows counted as (block*block_size + offset)*Hkv + kv_head).  A
        negative slot skips its vector.  The kernel takes the other slots as
        distinct and in range; check_slots=True verifies that first (reading
        the slots back: a device synchronisation)."""
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
        if check_slots:
            verify_slots(slots, num_slots)
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

    def forward(self, query, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                block_size: int = 16, out: torch.Tensor | None = None) -> torch.Tensor:
        """softmax(scale * q K^T) V over each sequence's first context_lens[b]
        cached tokens.  Every argument is validated before the launch
        (torch_ops.check_attn_args); `out`, when given, must be a contiguous
        float16 [batch, num_query_heads, head_dim] tensor on the query's
        device.  The workspace is taken from torch's caching allocator per
        call, on the current stream."""
        tq = self.tq
        if query.dim() != 3 or query.shape[1] != self.num_query_heads or \
                query.shape[2] != tq.head_dim:
            raise ValueError("query must be float16 [batch, %d, %d]" % (self.num_query_heads,
                                                                         tq.head_dim))
        if k_packed.dim() != 4 or k_packed.shape[1] != block_size:
            raise ValueError("k_packed must be [num_blocks, block_size, num_kv_heads, P]")
        torch_ops.check_attn_args(query, k_packed, k_norms, v_packed, v_norms, block_tables,
                                  context_lens, tq.bits, self.v_tq.bits, out)
        if out is None:
            _require_gpu(query, "query")
            out = torch.empty_like(query, memory_format=torch.contiguous_format)
        return torch_ops.attn_decode_into(out, query, k_packed, k_norms, v_packed, v_norms,
                                          block_tables, context_lens, tq.bits, self.v_tq.bits,
                                          tq.seed, self.scale)

    __call__ = forward


class HybridTurboQuant:
    """Hybrid modes tq35 / tq25 (aither-kvcache PyPI page, "Hybrid modes
    (tq35/tq25)" and "API Reference"): [..., 128] fp16 <-> [..., row] uint8
    with the norms inside the row (68 bytes for tq35, 52 for tq25).

    The channels are split into two groups of 64 by calibration (group A,
    coded with the more bits, holds the channels with the largest mean square
    in `calibrate`; `calibrate_uniform` keeps channels 0-63 / 64-127); each
    group is a TurboQuant vector of dimension 64 at (3, 2) or (2, 1) bits, and
    the residual is kept as a 128-bit sign sketch plus its norm (QJL), which
    makes inner products with the decoded vectors unbiased."""

    MODES = {"tq35": 35, "tq25": 25}

    def __init__(self, head_dim: int = HEAD_DIM, mode: str = "tq35", seed: int = 42,
                 device="cuda"):
        if mode not in self.MODES:
            raise ValueError("mode must be one of %s" % sorted(self.MODES))
        if self.packed_dim_for_mode(head_dim, mode) == 0:
            raise ValueError("hybrid modes take head_dim 128")
        self.head_dim = head_dim
        self.mode = mode
        self.seed = int(seed) & (2 ** 64 - 1)
        self.device = torch.device(device)
        if self.device.type != "cuda":
            raise ValueError("HybridTurboQuant runs on the GPU only")
        self.num_kv_heads = 1
        self._perm = np.arange(head_dim, dtype=np.int32)

    @staticmethod
    def packed_dim_for_mode(head_dim: int, mode: str) -> int:
        """Bytes of one packed row (norms included); 0 when unsupported."""
        if mode not in HybridTurboQuant.MODES:
            return 0
        return _lib.tq_hybrid_packed_bytes(head_dim, HybridTurboQuant.MODES[mode])

    @property
    def packed_dim(self) -> int:
        return self.packed_dim_for_mode(self.head_dim, self.mode)

    @property
    def perm(self) -> np.ndarray:
        """Channel permutation: perm[0..63] is group A, perm[64..127] group B."""
        return self._perm.copy()

    def compression_ratio(self) -> float:
        return 2.0 * self.head_dim / self.packed_dim

    def calibrate_uniform(self, num_kv_heads: int = 1) -> None:
        """Data-free split: channels 0-63 in group A, 64-127 in group B (the
        same for every one of the num_kv_heads heads)."""
        if num_kv_heads < 1:
            raise ValueError("num_kv_heads must be positive")
        self.num_kv_heads = num_kv_heads
        self._perm = np.arange(self.head_dim, dtype=np.int32)

    def calibrate(self, sample_vectors: torch.Tensor) -> None:
        """Group A = the 64 channels with the largest mean square over the
        sample (ties to the lower channel), both groups in ascending channel
        order."""
        if sample_vectors.shape[-1] != self.head_dim:
            raise ValueError("sample_vectors must be [..., %d]" % self.head_dim)
        ms = sample_vectors.reshape(-1, self.head_dim).float().pow(2).mean(0).cpu().numpy()
        order = np.lexsort((np.arange(self.head_dim), -ms))     # largest first, lower index on ties
        h = self.head_dim // 2
        self._perm = np.concatenate([np.sort(order[:h]), np.sort(order[h:])]).astype(np.int32)

    def encode(self, x: torch.Tensor) -> torch.Tensor:
        """x [..., 128] fp16 -> packed [..., packed_dim] uint8 (norms embedded)."""
        _require_gpu(x, "x")
        if x.dtype != torch.float16 or x.shape[-1] != self.head_dim:
            raise ValueError("x must be float16 [..., %d]" % self.head_dim)
        return torch.ops.kv_cache_vector.tq_hybrid_encode(
            x, self.MODES[self.mode], torch_ops.seed_to_i64(self.seed),
            torch.from_numpy(self._perm))

    def decode(self, packed: torch.Tensor) -> torch.Tensor:
        """packed [..., packed_dim] uint8 -> [..., 128] fp16."""
        _require_gpu(packed, "packed")
        if packed.dtype != torch.uint8 or packed.shape[-1] != self.packed_dim:
            raise ValueError("packed must be uint8 [..., %d]" % self.packed_dim)
        return torch.ops.kv_cache_vector.tq_hybrid_decode(
            packed, self.MODES[self.mode], torch_ops.seed_to_i64(self.seed),
            torch.from_numpy(self._perm))

    def validate(self, num_vectors: int = 10000, seed: int = 0) -> dict:
        """Round-trip MSE per coordinate of the unit vector on N(0,1) vectors,
        and the relative bias of the inner products <x, xhat> against ||x||^2
        (the direction in which the TurboQuant part alone shrinks; the QJL
        sketch makes the estimate unbiased)."""
        g = torch.Generator(device=self.device).manual_seed(seed)
        x = torch.randn(num_vectors, self.head_dim, generator=g, device=self.device).half()
        xh = self.decode(self.encode(x)).float()
        xf = x.float()
        mse = float((((xf - xh) ** 2).sum(1) / (xf ** 2).sum(1)).mean())
        xx = (xf * xf).sum(1)
        bias = float(((xf * xh).sum(1) - xx).mean() / xx.mean())
        return {"mse": mse, "inner_product_bias": bias, "num_vectors": num_vectors,
                "mode": self.mode}
