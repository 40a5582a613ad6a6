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


def llama70b_head_scales(layer: int, heads: int = 8) -> np.ndarray:
    """The per-(K/V, head) scale factors of one 70B-class layer, [2, heads]
    (the first draw of the layer's data seed 300+layer)."""
    rng = np.random.default_rng(300 + layer)
    return rng.uniform(0.5, 2.0, size=(2, heads)).astype(np.float32)


def llama70b_layer(layer: int, tokens: int = 131072, heads: int = 8) -> np.ndarray:
    """N(0,1) scaled per (K/V, head) by a factor drawn uniformly in [0.5, 2].
    Data seed 300+layer.  Returns [2*heads*tokens, 128]."""
    rng = np.random.default_rng(300 + layer)
    scale = rng.uniform(0.5, 2.0, size=(2, heads, 1, 1)).astype(np.float32)
    x = rng.standard_normal((2, heads, tokens, HEAD_DIM), dtype=np.float32) * scale
    return _f16(x.reshape(-1, HEAD_DIM))


def llama70b_layer_sample(layer: int, frac: float = 0.01, tokens: int = 131072,
                          heads: int = 8) -> np.ndarray:
    """A seeded sample of one 70B-class layer: round(frac * tokens) tokens
    per (K/V, head), N(0,1) times the layer's per-(K/V, head) scales, drawn
    from the stream (300 + layer, 1) -- the layer's distribution, not its
    exact rows.  Returns [2*heads*round(frac*tokens), 128]."""
    n = int(round(frac * tokens))
    scale = llama70b_head_scales(layer, heads)[:, :, None, None]
    rng = np.random.default_rng([300 + layer, 1])
    x = rng.standard_normal((2, heads, n, HEAD_DIM), dtype=np.float32) * scale
    return _f16(x.reshape(-1, HEAD_DIM))


# ---------------------------------------------------------------------------
# decode-attention workload: batch 16, 32 query heads / 8 KV heads,
# 32768 cached tokens per sequence in 16-token pages
# ---------------------------------------------------------------------------

def attn_kv_rows(b: int, g: int, tokens: int, seed: int = 500, outlier_p: float = 0.01,
                 outlier_factor: float = 15.0, head_dim: int = HEAD_DIM) -> np.ndarray:
    """K and V of sequence b, kv head g in token order: [2, tokens, head_dim]
    fp16, N(0,1) with Bernoulli(outlier_p) outlier channels (x outlier_factor)
    fixed for the (sequence, kv head).  Seeded by (seed, b, g) alone, so any
    one stream can be regenerated without the others."""
    rng = np.random.default_rng([seed, b, g])
    mask = rng.random((2, 1, head_dim)) < outlier_p
    kv = rng.standard_normal((2, tokens, head_dim), dtype=np.float32)
    kv = np.where(mask, kv * np.float32(outlier_factor), kv)
    return _f16(kv)


def attn_query(batch: int, num_q_heads: int, seed: int = 500,
               head_dim: int = HEAD_DIM) -> np.ndarray:
    rng = np.random.default_rng([seed, 1 << 30])
    return _f16(rng.standard_normal((batch, num_q_heads, head_dim), dtype=np.float32))


def attn_block_tables(batch: int, max_blocks: int, num_blocks: int,
                      perm_seed: int = 501) -> np.ndarray:
    """A seeded random permutation of the physical blocks, max_blocks per
    sequence: [batch, max_blocks] int32."""
    perm = np.random.default_rng(perm_seed).permutation(num_blocks)[: batch * max_blocks]
    return perm.astype(np.int32).reshape(batch, max_blocks)


def attn_context_lens(batch: int, context: int, ragged: bool, block_size: int = 16,
                      seed: int = 500) -> np.ndarray:
    """All equal to ``context``, or (ragged) drawn in [1, context] with 1, the
    full length, block_size + 1 and context - 3 among them."""
    if not ragged:
        return np.full(batch, context, dtype=np.int32)
    rng = np.random.default_rng([seed, 1 << 31])
    cl = rng.integers(1, context + 1, size=batch).astype(np.int32)
    fixed = [1, context, min(context, block_size + 1), max(1, context - 3)]
    cl[: min(batch, 4)] = fixed[: min(batch, 4)]
    return cl


def scatter_pages(pages: np.ndarray, rows: np.ndarray, block_table_row: np.ndarray, g: int,
                  block_size: int = 16) -> None:
    """Write rows [T, ...] of one (sequence, kv head) into pages
    [num_blocks, block_size, Hkv, ...] following that sequence's block table."""
    T = rows.shape[0]
    t = np.arange(T)
    pages[block_table_row[t // block_size], t % block_size, g] = rows


def attn_workload(batch: int = 16, num_q_heads: int = 32, num_kv_heads: int = 8,
                  context: int = 32768, block_size: int = 16, seed: int = 500,
                  perm_seed: int = 501, ragged: bool = False, outlier_p: float = 0.01,
                  outlier_factor: float = 15.0, extra_blocks: int = 0, head_dim: int = HEAD_DIM):
    """Returns a dict with
      q            [B, Hq, head_dim] fp16, N(0,1)
      k, v         [num_blocks, block_size, Hkv, head_dim] fp16 -- the cache content
                   in physical (paged) order (attn_kv_rows per sequence and kv
                   head; pages no sequence uses hold N(0,1) filler)
      block_tables [B, max_blocks] int32 -- a seeded random permutation of the
                   physical blocks
      context_lens [B] int32 -- see attn_context_lens.
    """
    max_blocks = (context + block_size - 1) // block_size
    nblk = batch * max_blocks + extra_blocks
    q = attn_query(batch, num_q_heads, seed, head_dim)
    bt = attn_block_tables(batch, max_blocks, nblk, perm_seed)
    filler = np.random.default_rng([seed, 1 << 29])
    pages = filler.standard_normal((2, nblk, block_size, num_kv_heads, head_dim),
                                   dtype=np.float32).astype(np.float16)
    for b in range(batch):
        for g in range(num_kv_heads):
            kv = attn_kv_rows(b, g, max_blocks * block_size, seed, outlier_p, outlier_factor,
                              head_dim)
            scatter_pages(pages[0], kv[0], bt[b], g, block_size)
            scatter_pages(pages[1], kv[1], bt[b], g, block_size)
    cl = attn_context_lens(batch, context, ragged, block_size, seed)
    return dict(q=q, k=pages[0], v=pages[1], block_tables=bt, context_lens=cl,
                block_size=block_size, num_kv_heads=num_kv_heads)


def gaussian(n: int, seed: int, head_dim: int = HEAD_DIM) -> np.ndarray:
    """n plain N(0,1) vectors of dimension head_dim (fp16)."""
    rng = np.random.default_rng(seed)
    return _f16(rng.standard_normal((n, head_dim), dtype=np.float32))


def kv_heads_outliers(head_dim: int, tokens: int, heads: int = 8, seed: int = 600,
                      outlier_p: float = 0.01, outlier_factor: float = 15.0) -> np.ndarray:
    """K and V of `heads` KV heads at another head dimension (64 or 256), the
    8B-shaped layer's recipe: N(0,1), every channel of a (K/V, head) an outlier
    (x outlier_factor) with probability outlier_p.  [2*heads*tokens, head_dim]."""
    rng = np.random.default_rng([seed, head_dim])
    mask = rng.random((2, heads, 1, head_dim)) < outlier_p
    x = rng.standard_normal((2, heads, tokens, head_dim), dtype=np.float32)
    x = np.where(mask, x * np.float32(outlier_factor), x)
    return _f16(x.reshape(-1, head_dim))
