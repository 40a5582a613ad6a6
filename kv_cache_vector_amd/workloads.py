"""Seeded synthetic KV-cache workloads (host side, numpy).

These generators produce inputs only: fp16 key/value vectors, queries, block
tables and context lengths.  They contain none of the codec's arithmetic, so
the test-suite can feed the very same bytes to the GPU library and to the CPU
oracle.  Every array is drawn with ``numpy.random.default_rng(seed)`` in
float32 and rounded to float16 with round-to-nearest-even.

Shapes and value distributions follow the caches the pages discuss: head_dim
128 key/value vectors of grouped-query-attention models (8 KV heads), stored
in 16-token pages (aither-kvcache PyPI page, "Paged KV cache"); keys and
values carry a few large outlier channels, which the random rotation is there
to spread out (qbc.network blog, "What TurboQuant is").
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128


def _f16(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float16)


# ---------------------------------------------------------------------------
# small parity workload: 1 layer x 8 KV heads x 512 tokens, N(0,1) with
# channels 7 and 93 scaled x20 in every vector
# ---------------------------------------------------------------------------

def outlier_channels_fixed(n_tokens: int = 512, n_heads: int = 8, seed: int = 1,
                           channels=(7, 93), factor: float = 20.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_heads * n_tokens, HEAD_DIM), dtype=np.float32)
    x[:, list(channels)] *= factor
    return _f16(x)


# ---------------------------------------------------------------------------
# Llama-3-8B-shaped cache: [32 layers, {K,V}, batch 4, 8 heads, 8192 tokens, 128]
# ---------------------------------------------------------------------------

LLAMA8B = dict(layers=32, kv=2, batch=4, heads=8, tokens=8192)


def llama8b_layer(layer: int, dist: str = "gauss_outliers", tokens: int = 8192,
                  batch: int = 4, heads: int = 8, outlier_p: float = 0.01,
                  outlier_factor: float = 15.0, seed_base: int | None = None) -> np.ndarray:
    """One layer of the 8B-shaped cache, flattened to [2*batch*heads*tokens, 128].

    dist="gauss_outliers": N(0,1); per (K/V, head) every channel is an
      outlier with probability ``outlier_p`` and is then scaled by
      ``outlier_factor`` for all batch entries and tokens.  Data seed 100+layer.
    dist="student_t": iid Student-t with 4 degrees of freedom divided by
      sqrt(2) (unit variance), no outliers.  Data seed 200+layer.
    """
    if dist == "gauss_outliers":
        rng = np.random.default_rng((100 if seed_base is None else seed_base) + layer)
        mask = rng.random((2, 1, heads, 1, HEAD_DIM)) < outlier_p
        x = rng.standard_normal((2, batch, heads, tokens, HEAD_DIM), dtype=np.float32)
        x = np.where(mask, x * np.float32(outlier_factor), x)
    elif dist == "student_t":
        rng = np.random.default_rng((200 if seed_base is None else seed_base) + layer)
        x = rng.standard_t(4.0, size=(2, batch, heads, tokens, HEAD_DIM)).astype(np.float32)
        x *= np.float32(1.0 / np.sqrt(2.0))
    else:
        raise ValueError(dist)
    return _f16(x.reshape(-1, HEAD_DIM))


# ---------------------------------------------------------------------------
# 70B-class GQA cache at 128K context: [80 layers, {K,V}, 1, 8 heads, 131072, 128]
# ---------------------------------------------------------------------------

LLAMA70B_128K = dict(layers=80, kv=2, batch=1, heads=8, tokens=131072)


def llama70b_layer(layer: int, tokens: int = 131072, heads: int = 8) -> np.ndarray:
    """N(0,1) scaled per (K/V, head) by a factor drawn uniformly in [0.5, 2].
    Data seed 300+layer.  Returns [2*heads*tokens, 128]."""
    rng = np.random.default_rng(300 + layer)
    scale = rng.uniform(0.5, 2.0, size=(2, heads, 1, 1)).astype(np.float32)
    x = rng.standard_normal((2, heads, tokens, HEAD_DIM), dtype=np.float32) * scale
    return _f16(x.reshape(-1, HEAD_DIM))


# ---------------------------------------------------------------------------
# decode-attention workload: batch 16, 32 query heads / 8 KV heads,
# 32768 cached tokens per sequence in 16-token pages
# ---------------------------------------------------------------------------

def attn_workload(batch: int = 16, num_q_heads: int = 32, num_kv_heads: int = 8,
                  context: int = 32768, block_size: int = 16, seed: int = 500,
                  perm_seed: int = 501, ragged: bool = False, outlier_p: float = 0.01,
                  outlier_factor: float = 15.0, extra_blocks: int = 0):
    """Returns a dict with
      q            [B, Hq, 128] fp16, N(0,1)
      k, v         [num_blocks, block_size, Hkv, 128] fp16 -- the cache content
                   in physical (paged) order, N(0,1) with Bernoulli(outlier_p)
                   outlier channels (x outlier_factor) per (sequence, kv head)
      block_tables [B, max_blocks] int32 -- a seeded random permutation of the
                   physical blocks
      context_lens [B] int32 -- all equal to ``context`` unless ragged=True,
                   in which case they are drawn in [1, context] and include 1
                   and lengths that are not multiples of the block size.
    """
    rng = np.random.default_rng(seed)
    max_blocks = (context + block_size - 1) // block_size
    nblk = batch * max_blocks + extra_blocks
    q = rng.standard_normal((batch, num_q_heads, HEAD_DIM), dtype=np.float32)
    # logical [B, Hkv, T, 128] -> physical pages
    mask = rng.random((2, batch, num_kv_heads, 1, HEAD_DIM)) < outlier_p
    kv = rng.standard_normal((2, batch, num_kv_heads, max_blocks * block_size, HEAD_DIM),
                             dtype=np.float32)
    kv = np.where(mask, kv * np.float32(outlier_factor), kv)
    prng = np.random.default_rng(perm_seed)
    perm = prng.permutation(nblk)[: batch * max_blocks].astype(np.int32)
    block_tables = perm.reshape(batch, max_blocks)
    pages = np.zeros((2, nblk, block_size, num_kv_heads, HEAD_DIM), dtype=np.float32)
    if extra_blocks:
        pages[:] = rng.standard_normal(pages.shape, dtype=np.float32)
    # token t of sequence b lives in block block_tables[b, t // bs], row t % bs
    logical = kv.reshape(2, batch, num_kv_heads, max_blocks, block_size, HEAD_DIM)
    logical = logical.transpose(0, 1, 3, 4, 2, 5)  # [2, B, max_blocks, bs, Hkv, 128]
    pages[:, block_tables.reshape(-1)] = logical.reshape(2, batch * max_blocks, block_size,
                                                         num_kv_heads, HEAD_DIM)
    if ragged:
        cl = rng.integers(1, context + 1, size=batch).astype(np.int32)
        cl[0] = 1
        if batch > 1:
            cl[1] = context
        if batch > 2:
            cl[2] = min(context, block_size + 1)
        if batch > 3:
            cl[3] = max(1, context - 3)
    else:
        cl = np.full(batch, context, dtype=np.int32)
    return dict(q=_f16(q), k=_f16(pages[0]), v=_f16(pages[1]), block_tables=block_tables,
                context_lens=cl, block_size=block_size, num_kv_heads=num_kv_heads)


def gaussian(n: int, seed: int) -> np.ndarray:
    """n plain N(0,1) vectors of dimension 128 (fp16)."""
    rng = np.random.default_rng(seed)
    return _f16(rng.standard_normal((n, HEAD_DIM), dtype=np.float32))
