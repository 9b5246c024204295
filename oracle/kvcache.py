"""fp64 attention of queries against a (paged) key/value cache — TEST INFRASTRUCTURE ONLY.

Nothing outside ``tests/``, the smoke check and the benchmark's CPU-baseline leg may use this
module (the same rule as the rest of ``oracle/``).

What is computed. The pages name a paged KV cache among FlashAttention's advanced features
("Flash Attention - Fast Memory-Efficient Attention", skill page, section "Advanced features"),
describe KV-cache blocks stored as pages for inference ("FlashAttention V3 principles and
practice", section 4, with a serving configuration of 16-token cache blocks and up to 128
sequences), and list paged attention among the ROCm backends' features ("What FlashAttention is
and how it speeds up attention", section "Versions, hardware and sources"). They give no
interface. The plain reading (RK1): the cache holds fixed-size pages of ``page_size`` tokens,
``k_cache`` / ``v_cache`` ``[num_pages, page_size, Hkv, D]``; sequence b has ``seqlens_k[b]``
keys, and its key j lives in page ``block_table[b, j // page_size]`` at slot ``j % page_size``.
Without a block table the cache is dense, ``[B, max_seqlen_k, Hkv, D]``, and key j of sequence
b is row j of batch b. The result (RK2) is, for every sequence, exactly the attention of its
``Nq`` queries against its own ``seqlens_k[b]`` keys (readings R1-R5 with Nk = seqlens_k[b]; the
causal mask is bottom-right aligned, so with Nq = 1 the query sees every key); a sequence with
no keys gives out = 0 and lse = -inf (R4).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_fp64

__all__ = ["gather_kv", "attention_kvcache_fp64"]


def gather_kv(cache, b: int, n: int, block_table=None, page_size: int = 0):
    """Keys (or values) 0 .. n-1 of sequence b as a dense [n, Hkv, D] array (reading RK1)."""
    cache = np.asarray(cache)
    if block_table is None:
        return cache[b, :n]
    j = np.arange(n)
    pages = np.asarray(block_table)[b, j // page_size]
    return cache[pages, j % page_size]


def attention_kvcache_fp64(q, k_cache, v_cache, seqlens_k, block_table=None, page_size: int = 0,
                           scale: float | None = None, causal: bool = False, window=(-1, -1)):
    """q [B, Nq, Hq, D] against each sequence's cached keys (readings RK1-RK2).

    Returns (out [B, Nq, Hq, D] fp64, lse [B, Hq, Nq] fp64).
    """
    B, Nq, Hq, D = q.shape
    out = np.zeros((B, Nq, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, Nq), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seqlens_k[b])
        if n == 0:
            continue                                  # no keys: 0 / -inf
        kb = gather_kv(k_cache, b, n, block_table, page_size)
        vb = gather_kv(v_cache, b, n, block_table, page_size)
        o, ls = attention_fp64(q[b:b + 1], kb[None], vb[None], scale, causal, window)
        out[b] = o[0]
        lse[b] = ls[0]
    return out, lse
