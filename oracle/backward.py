"""fp64 gradients of exact attention — TEST INFRASTRUCTURE ONLY.

Nothing outside ``tests/``, the smoke check and the benchmark's CPU-baseline leg may use this
module (the same rule as the rest of ``oracle/``).

What is computed. The pages name a backward pass ("Flash Attention - Fast Memory-Efficient
Attention", skill page, Quick start: FlashAttention works by IO-aware tiling and recomputation;
"What FlashAttention is and how it speeds up attention", section "Versions, hardware and
sources": the ROCm backends run the forward and the backward pass) but give no formula for it.
The plain reading: the backward pass returns the gradient of a scalar loss with respect to q, k
and v, given the gradient ``dout`` of that loss with respect to the forward output. For the
forward of ``oracle.attention`` (s = scale * q.k over admitted keys, p = softmax(s) per query row,
out = p @ v) the chain rule gives, per (batch, query head), with dout the rows' output gradient:

    dv  = p^T @ dout                              (out is linear in v)
    dp  = dout @ v^T                              (out is linear in p)
    ds  = p * (dp - rowsum(p * dp))               (Jacobian of the row softmax)
    dq  = scale * ds @ k
    dk  = scale * ds^T @ q

Masked pairs have p = 0 and so take no part; a row with no admitted key contributes nothing.
A K/V head read by several query heads (MQA/GQA, reading R5 of ``oracle.attention``) receives the
sum of their contributions: dk and dv of K/V head g add up the terms of every query head h with
h // (Hq / Hkv) == g.

Readings taken where the pages leave a point open:
  RB1 The gradient is of the exact function (fp64 softmax of the fp64 scores of the given inputs);
      the kernel's own intermediate roundings (its fp16/bf16 out, the P operand of its products)
      are the kernel's error, measured against this.
  RB2 ``rowsum(p * dp)`` equals ``rowsum(dout * out)`` for the exact out; the oracle uses the
      first form (it needs no forward output).
"""
from __future__ import annotations

import numpy as np

from .attention import _check_shapes, admitted, kv_head_of

__all__ = ["attention_bwd_fp64"]


def _one_head_bwd(qh, kh, vh, doh, scale: float, mask):
    """Gradients for one head: qh/doh [n, D], kh/vh [Nk, D], mask [n, Nk]. Returns (dq, dk, dv)."""
    s = np.where(mask, scale * (qh @ kh.T), -np.inf)
    m = s.max(axis=1)
    m_fin = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(s - m_fin[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    nz = l > 0
    p[nz] = e[nz] / l[nz, None]                          # softmax rows; empty rows stay 0
    dv = p.T @ doh
    dp = doh @ vh.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))  # row-softmax Jacobian applied to dp
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv


def attention_bwd_fp64(q, k, v, dout, scale: float | None = None, causal: bool = False, window=(-1, -1),
                       row_chunk: int = 1024):
    """Gradients (dq [B,Nq,Hq,D], dk [B,Nk,Hkv,D], dv [B,Nk,Hkv,D]) in fp64 for upstream ``dout``.

    Layouts and options as in ``attention_fp64``; ``dout`` has the shape of the output
    ``[B, Nq, Hq, D]``. Query rows are processed in chunks of ``row_chunk`` (the gradients of
    different query rows add up independently in dk and dv).
    """
    B, Nq, Nk, Hq, Hkv, D = _check_shapes(q, k, v)
    if tuple(dout.shape) != (B, Nq, Hq, D):
        raise ValueError(f"dout must be {(B, Nq, Hq, D)}, got {tuple(dout.shape)}")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    wl, wr = window
    dq = np.zeros((B, Nq, Hq, D), dtype=np.float64)
    dk = np.zeros((B, Nk, Hkv, D), dtype=np.float64)
    dv = np.zeros((B, Nk, Hkv, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kh = np.asarray(k[b, :, g, :], dtype=np.float64)
            vh = np.asarray(v[b, :, g, :], dtype=np.float64)
            for r0 in range(0, Nq, row_chunk):
                rows = np.arange(r0, min(Nq, r0 + row_chunk))
                qh = np.asarray(q[b, r0:r0 + len(rows), h, :], dtype=np.float64)
                doh = np.asarray(dout[b, r0:r0 + len(rows), h, :], dtype=np.float64)
                mask = admitted(Nq, Nk, causal, wl, wr, rows=rows)
                gq, gk, gv = _one_head_bwd(qh, kh, vh, doh, float(scale), mask)
                dq[b, r0:r0 + len(rows), h, :] = gq
                dk[b, :, g, :] += gk
                dv[b, :, g, :] += gv
    return dq, dk, dv
