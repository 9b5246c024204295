"""fp64 attention over packed variable-length batches — TEST INFRASTRUCTURE ONLY.

Nothing outside ``tests/``, the smoke check and the benchmark's CPU-baseline leg may use this
module (the same rule as the rest of ``oracle/``).

What is computed. The pages list variable sequence lengths among the features of the ROCm
backends ("What FlashAttention is and how it speeds up attention", section "Versions, hardware
and sources") and describe the V3 kernels as adapting to dynamic sequence lengths without
padding the inputs to a fixed length ("FlashAttention V3 principles and practice", section 1).
They give no interface. The plain reading (RV1): a batch of B sequences is packed along the
token axis, q ``[total_q, Hq, D]`` and k, v ``[total_k, Hkv, D]``, with cumulative offsets
``cu_q`` and ``cu_k`` (B + 1 non-decreasing integers from 0 to the totals): sequence b owns
query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1, and is an attention
problem of its own, exactly as if it were alone in a batch of one. In particular (RV2) the
causal alignment and the window of reading R1/R2 use each sequence's own lengths, and (RV3) a
sequence with queries but no keys gives out = 0 and lse = -inf on its rows (reading R4).
The log-sum-exp is returned as ``[Hq, total_q]``.
"""
from __future__ import annotations

import numpy as np

from .attention import _one_head, admitted, kv_head_of

__all__ = ["attention_varlen_fp64"]


def attention_varlen_fp64(q, k, v, cu_q, cu_k, scale: float | None = None, causal: bool = False, window=(-1, -1)):
    """Exact attention of each packed sequence in fp64.

    q: [total_q, Hq, D]; k, v: [total_k, Hkv, D]; cu_q, cu_k: B + 1 offsets (readings RV1-RV3).
    Returns (out [total_q, Hq, D] fp64, lse [Hq, total_q] fp64).
    """
    if q.ndim != 3 or k.ndim != 3 or k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError(f"q must be [total_q, Hq, D] and k, v [total_k, Hkv, D]: {q.shape} {k.shape} {v.shape}")
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if (cu_q.shape != cu_k.shape or cu_q.ndim != 1 or cu_q[0] != 0 or cu_k[0] != 0 or cu_q[-1] != total_q
            or cu_k[-1] != total_k or np.any(np.diff(cu_q) < 0) or np.any(np.diff(cu_k) < 0)):
        raise ValueError("cu_q / cu_k must be non-decreasing offsets from 0 to the totals, of equal length")
    kv_head_of(0, Hq, Hkv)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    lse = np.full((Hq, total_q), -np.inf, dtype=np.float64)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        nq, nk = qe - qs, ke - ks
        if nq == 0 or nk == 0:
            continue                               # no rows, or rows with no key: 0 / -inf (RV3)
        mask = admitted(nq, nk, causal, window[0], window[1])   # the sequence's own sizes (RV2)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, ls = _one_head(np.asarray(q[qs:qe, h, :], dtype=np.float64), np.asarray(k[ks:ke, g, :], dtype=np.float64),
                              np.asarray(v[ks:ke, g, :], dtype=np.float64), float(scale), mask)
            out[qs:qe, h, :] = o
            lse[h, qs:qe] = ls
    return out, lse
