"""fp64 block-sparse attention — TEST INFRASTRUCTURE ONLY.

Nothing outside ``tests/``, the smoke check and the benchmark's CPU-baseline leg may use this
module (the same rule as the rest of ``oracle/``).

What is computed. The pages report that the authors' block-sparse variant of FlashAttention scales
to 64k tokens and runs 2-4 times faster than the dense one ("What FlashAttention is and how it
speeds up attention", FAQ on the quadratic complexity); they give no interface and no sparsity
pattern. The plain reading (RS1): a block mask ``block_mask[hm, qb, kb]`` over blocks of
``block_q`` query rows and ``block_k`` keys says which (query block, key block) pairs take part;
a (query, key) pair is admitted when its block is set AND the dense mask admits it (readings R1,
R2: causal and window, applied as usual); everything else is the dense definition, so rows whose
admitted keys are all masked out give out = 0 and lse = -inf (R4). ``hm`` is 0 for a mask shared
by all heads, or the query head.
"""
from __future__ import annotations

import numpy as np

from .attention import _check_shapes, _one_head, admitted, kv_head_of

__all__ = ["block_admitted", "attention_blocksparse_fp64"]


def block_admitted(block_mask_2d, Nq: int, Nk: int, block_q: int, block_k: int, rows=None):
    """Boolean [len(rows), Nk]: True where the block of (row i, key j) is set (reading RS1)."""
    i = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    bm = np.asarray(block_mask_2d) != 0
    return bm[(i // block_q)[:, None], (np.arange(Nk) // block_k)[None, :]]


def attention_blocksparse_fp64(q, k, v, block_mask, block_q: int = 128, block_k: int = 64, scale: float | None = None,
                               causal: bool = False, window=(-1, -1), row_chunk: int = 1024):
    """q [B, Nq, Hq, D]; k, v [B, Nk, Hkv, D]; block_mask [1 or Hq, ceil(Nq/block_q), ceil(Nk/block_k)].
    Returns (out [B, Nq, Hq, D] fp64, lse [B, Hq, Nq] fp64)."""
    B, Nq, Nk, Hq, Hkv, D = _check_shapes(q, k, v)
    bm = np.asarray(block_mask)
    nqb, nkb = -(-Nq // block_q), -(-Nk // block_k)
    if bm.ndim != 3 or bm.shape[0] not in (1, Hq) or bm.shape[1:] != (nqb, nkb):
        raise ValueError(f"block_mask must be [1 or {Hq}, {nqb}, {nkb}], got {bm.shape}")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Nq, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kh = np.asarray(k[b, :, g, :], dtype=np.float64)
            vh = np.asarray(v[b, :, g, :], dtype=np.float64)
            bmh = bm[0 if bm.shape[0] == 1 else h]
            for r0 in range(0, Nq, row_chunk):
                rows = np.arange(r0, min(Nq, r0 + row_chunk))
                qh = np.asarray(q[b, r0:r0 + len(rows), h, :], dtype=np.float64)
                mask = admitted(Nq, Nk, causal, window[0], window[1], rows=rows)
                mask &= block_admitted(bmh, Nq, Nk, block_q, block_k, rows=rows)
                o, ls = _one_head(qh, kh, vh, float(scale), mask)
                out[b, r0:r0 + len(rows), h, :] = o
                lse[b, h, r0:r0 + len(rows)] = ls
    return out, lse
