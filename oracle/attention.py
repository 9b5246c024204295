"""fp64 attention: the plain definition and the pages' block traversal — TEST INFRASTRUCTURE ONLY.

Nothing outside ``tests/``, the smoke check and the benchmark's CPU-baseline leg may use this
module. It is deliberately slow and plain: numpy fp64, one (batch, query head) at a time, the full
score matrix materialised (chunked over query rows only, to bound memory).

What is computed ("Flash Attention - Fast Memory-Efficient Attention", skill page, Workflow 1
Step 2 and Workflow 2 Steps 2-3):

    out[b, i, h, :] = sum_j softmax_j(scale * <q[b, i, h, :], k[b, j, g(h), :]>) * v[b, j, g(h), :]

with tensors in the ``[batch, seqlen, nheads, headdim]`` layout, softmax over the key axis, the
default scale ``1/sqrt(headdim)``, optional causal masking, an optional ``(left, right)`` sliding
window, and fewer K/V heads than query heads (MQA/GQA). "What FlashAttention is and how it speeds
up attention" (ya.zerocoder.ru), sections 1 and 3, states that the blocked algorithm is exact:
it reaches this same result, so this definition is the oracle.

Readings taken where the pages leave a point open:
  R1  Causal alignment when Nq != Nk is bottom-right: query i may see key j iff
      j <= i + (Nk - Nq). With Nq == Nk this is the usual lower triangle.
  R2  A window (left, right) keeps keys j with i+off-left <= j <= i+off+right (inclusive,
      off = Nk - Nq); -1 means unbounded on that side. With causal it is intersected with the
      causal mask, so the right bound becomes min(right, 0).
  R3  The log-sum-exp output is the natural log of the row's sum of exp(score), with the
      softmax scale included in the score: lse_i = m_i + ln(sum_j exp(s_ij - m_i)).
  R4  A row with no admitted key has output 0 and lse = -inf.
  R5  Query head h reads K/V head h // (Hq / Hkv): consecutive groups of query heads share a KV
      head (K/V "repeat-interleaved" to Hq heads).
"""
from __future__ import annotations

import numpy as np

__all__ = ["kv_head_of", "admitted", "attention_fp64", "attention_rows_fp64", "tiled_online_fp64"]


def kv_head_of(hq: int, Hq: int, Hkv: int) -> int:
    """K/V head read by query head ``hq`` (reading R5; skill page, Workflow 2 Step 3, MQA/GQA)."""
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    return hq // (Hq // Hkv)


def admitted(Nq: int, Nk: int, causal: bool = False, window_left: int = -1, window_right: int = -1,
             rows=None) -> np.ndarray:
    """Boolean [len(rows), Nk] mask: True where query row i may attend to key j.

    Causal masking (skill page, Workflow 2 Step 2) and the ``(left, right)`` sliding window
    (skill page, Workflow 2 Step 3), under readings R1 and R2.
    """
    i = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    i = i[:, None]
    j = np.arange(Nk)[None, :]
    off = Nk - Nq
    ok = np.ones((i.shape[0], Nk), dtype=bool)
    if causal:
        ok &= j <= i + off
    if window_left >= 0:
        ok &= j >= i + off - window_left
    if window_right >= 0:
        ok &= j <= i + off + window_right
    return ok


def _one_head(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, mask: np.ndarray):
    """Definition for one head: qh [n, D], kh/vh [Nk, D] (fp64), mask [n, Nk]. Returns (out, lse)."""
    s = scale * (qh @ kh.T)                     # full score block, fp64
    s = np.where(mask, s, -np.inf)              # masked pairs take no part in the softmax
    m = s.max(axis=1)                           # row max over admitted keys (-inf: empty row)
    m_fin = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(s - m_fin[:, None]), 0.0)
    l = e.sum(axis=1)
    out = np.zeros((qh.shape[0], vh.shape[1]), dtype=np.float64)
    lse = np.full(qh.shape[0], -np.inf, dtype=np.float64)
    nz = l > 0
    out[nz] = (e[nz] @ vh) / l[nz, None]        # softmax weights times V
    lse[nz] = m[nz] + np.log(l[nz])             # reading R3; empty rows keep 0 / -inf (R4)
    return out, lse


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [batch, seqlen, nheads, headdim]")
    B, Nq, Hq, D = q.shape
    Bk, Nk, Hkv, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    kv_head_of(0, Hq, Hkv)
    return B, Nq, Nk, Hq, Hkv, D


def attention_fp64(q, k, v, scale: float | None = None, causal: bool = False, window=(-1, -1),
                   row_chunk: int = 1024):
    """Exact attention in fp64 over the full score matrix.

    q: [B, Nq, Hq, D]; k, v: [B, Nk, Hkv, D] (any real dtype; converted to fp64 per head).
    Returns (out [B, Nq, Hq, D] fp64, lse [B, Hq, Nq] fp64).
    ``scale=None`` means 1/sqrt(D) (skill page, Workflow 2 Step 2, automatic scale).
    """
    B, Nq, Nk, Hq, Hkv, D = _check_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    wl, wr = window
    out = np.zeros((B, Nq, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kh = np.asarray(k[b, :, g, :], dtype=np.float64)
            vh = np.asarray(v[b, :, g, :], dtype=np.float64)
            for r0 in range(0, Nq, row_chunk):
                rows = np.arange(r0, min(Nq, r0 + row_chunk))
                qh = np.asarray(q[b, r0:r0 + len(rows), h, :], dtype=np.float64)
                mask = admitted(Nq, Nk, causal, wl, wr, rows=rows)
                o, ls = _one_head(qh, kh, vh, float(scale), mask)
                out[b, r0:r0 + len(rows), h, :] = o
                lse[b, h, r0:r0 + len(rows)] = ls
    return out, lse


def attention_rows_fp64(q, k, v, b: int, h: int, rows, scale: float | None = None, causal: bool = False,
                        window=(-1, -1)):
    """The same definition for selected query rows of one (batch, query head).

    Used to check full-size runs on a sample of outputs. Returns (out [len(rows), D], lse [len(rows)]).
    """
    B, Nq, Nk, Hq, Hkv, D = _check_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    g = kv_head_of(h, Hq, Hkv)
    qh = np.asarray(q[b, rows, h, :], dtype=np.float64)
    kh = np.asarray(k[b, :, g, :], dtype=np.float64)
    vh = np.asarray(v[b, :, g, :], dtype=np.float64)
    mask = admitted(Nq, Nk, causal, window[0], window[1], rows=rows)
    return _one_head(qh, kh, vh, float(scale), mask)


def tiled_online_fp64(q, k, v, scale: float | None = None, causal: bool = False, window=(-1, -1),
                      block_q: int = 2, block_k: int = 2):
    """The pages' blocked traversal with incremental renormalisation, in fp64.

    "What FlashAttention is and how it speeds up attention" (ya.zerocoder.ru), section 2: the
    score grid is cut into blocks; each block's Q, K, V are brought into fast memory, attention is
    computed inside the block, the output is updated with a correct normalisation, and the walk moves
    on to the next block. Blocks are visited in the order of the grid's labels (row by row: one query
    block against every key block in turn). The running state per query row is the largest score
    seen so far (m), the sum of exp(score - m) (l) and the unnormalised output (acc); when m grows,
    l and acc are multiplied by exp(m_old - m_new) so that every term stays relative to the new max.

    Returns (out, lse, classes) where classes counts the visited blocks as
    ``{"skipped": no pair admitted, "partial": some admitted, "full": all admitted}``.
    """
    B, Nq, Nk, Hq, Hkv, D = _check_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    wl, wr = window
    out = np.zeros((B, Nq, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, Nq), dtype=np.float64)
    classes = {"skipped": 0, "partial": 0, "full": 0}
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for i0 in range(0, Nq, block_q):
                rows = np.arange(i0, min(Nq, i0 + block_q))
                qi = np.asarray(q[b, i0:i0 + len(rows), h, :], dtype=np.float64)
                m = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), D))
                for j0 in range(0, Nk, block_k):
                    cols = slice(j0, min(Nk, j0 + block_k))
                    mask = admitted(Nq, Nk, causal, wl, wr, rows=rows)[:, cols]
                    if not mask.any():
                        classes["skipped"] += 1
                        continue
                    classes["full" if mask.all() else "partial"] += 1
                    kj = np.asarray(k[b, cols, g, :], dtype=np.float64)
                    vj = np.asarray(v[b, cols, g, :], dtype=np.float64)
                    s = np.where(mask, scale * (qi @ kj.T), -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    live = np.isfinite(m_new)                  # rows that have seen an admitted key
                    m_ref = np.where(live, m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
                    p = np.where(mask, np.exp(s - m_ref[:, None]), 0.0)
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ vj
                    m = m_new
                nz = l > 0
                o = np.zeros_like(acc)
                o[nz] = acc[nz] / l[nz, None]
                ls = np.full(len(rows), -np.inf)
                ls[nz] = m[nz] + np.log(l[nz])
                out[b, i0:i0 + len(rows), h, :] = o
                lse[b, h, i0:i0 + len(rows)] = ls
    return out, lse, classes
