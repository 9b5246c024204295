"""Pins of the packed variable-length oracle (``oracle.varlen``) to facts outside its own code.

  * a special case that reduces to the pinned dense oracle: B sequences of equal lengths are the
    dense batch [B, N, H, D] reshaped;
  * an independent library routine: PyTorch's CPU fp64 scaled_dot_product_attention over the
    whole packed token axis as ONE sequence, with a block-diagonal boolean mask built from the
    offsets (same sequence, and the causal / window predicate on the positions inside the
    sequence) — the reading that sequences do not see each other, written a second way;
  * invariants: reversing the order of the sequences permutes the output rows the same way;
    appending an empty sequence changes nothing; a sequence with queries but no keys gives 0 and
    -inf.
Planted mistakes (boundaries off by one, causal alignment on the packed index instead of the
sequence's, keys shared across sequences) must each fail a pin.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.varlen as OV
from oracle import attention_fp64, attention_varlen_fp64


def rand(seed, total_q, total_k, Hq, Hkv, D):
    g = np.random.default_rng(seed)
    return (g.standard_normal((total_q, Hq, D)), g.standard_normal((total_k, Hkv, D)),
            g.standard_normal((total_k, Hkv, D)))


def offsets(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def sdpa_packed(q, k, v, cu_q, cu_k, scale, causal, window):
    """One fp64 SDPA call over all packed tokens with a block-diagonal mask (K/V repeat-interleaved)."""
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[:2]
    seq_q = np.repeat(np.arange(len(cu_q) - 1), np.diff(cu_q))
    seq_k = np.repeat(np.arange(len(cu_k) - 1), np.diff(cu_k))
    pos_q = np.arange(total_q) - cu_q[seq_q]
    pos_k = np.arange(total_k) - cu_k[seq_k]
    nq = np.diff(cu_q)[seq_q]
    nk = np.diff(cu_k)[seq_k]
    same = seq_q[:, None] == seq_k[None, :]
    i = torch.tensor(pos_q)[:, None]
    j = torch.tensor(pos_k)[None, :]
    off = torch.tensor(nk)[None, :] - torch.tensor(nq)[:, None]     # the row's and the key's own sequence (same one)
    m = torch.tensor(same)
    if causal:
        m &= j <= i + off
    if window[0] >= 0:
        m &= j >= i + off - window[0]
    if window[1] >= 0:
        m &= j <= i + off + window[1]
    live = m.any(dim=1)
    msafe = m.clone()
    msafe[~live, 0] = True
    G = Hq // Hkv
    qt = torch.tensor(q).permute(1, 0, 2)[None]
    kt = torch.tensor(k).permute(1, 0, 2)[None].repeat_interleave(G, dim=1)
    vt = torch.tensor(v).permute(1, 0, 2)[None].repeat_interleave(G, dim=1)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=msafe, scale=scale)[0].permute(1, 0, 2).numpy()
    s = scale * torch.einsum("hqd,hkd->hqk", qt[0], kt[0])
    lse = torch.logsumexp(s.masked_fill(~m[None], float("-inf")), dim=-1).numpy()
    out[~live.numpy()] = 0.0
    return out, lse


CASES = [
    # lengths_q, lengths_k, Hq, Hkv, D, causal, window
    ([5, 9, 1, 7], [5, 9, 1, 7], 2, 2, 8, False, (-1, -1)),
    ([5, 9, 1, 7], [5, 9, 1, 7], 4, 2, 8, True, (-1, -1)),
    ([3, 8, 6], [7, 4, 6], 2, 1, 4, True, (-1, -1)),          # Nq != Nk inside sequences
    ([6, 0, 5], [6, 3, 5], 2, 2, 4, False, (2, 1)),           # an empty sequence of queries
    ([4, 3], [0, 3], 2, 2, 4, False, (-1, -1)),               # queries with no keys
    ([10, 12], [10, 12], 3, 1, 8, True, (3, -1)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"q{'-'.join(map(str, c[0]))}_k{'-'.join(map(str, c[1]))}_c{int(c[5])}_w{c[6][0]}_{c[6][1]}")
def test_varlen_matches_block_diagonal_sdpa(case):
    lq, lk, Hq, Hkv, D, causal, window = case
    cu_q, cu_k = offsets(lq), offsets(lk)
    q, k, v = rand(1, cu_q[-1], cu_k[-1], Hq, Hkv, D)
    out, lse = attention_varlen_fp64(q, k, v, cu_q, cu_k, 0.4, causal, window)
    ro, rl = sdpa_packed(q, k, v, cu_q, cu_k, 0.4, causal, window)
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(rl))
    fin = np.isfinite(rl)
    assert np.allclose(lse[fin], rl[fin], rtol=1e-12, atol=1e-12)


def test_varlen_equal_lengths_is_the_dense_batch():
    B, N, Hq, Hkv, D = 3, 11, 4, 2, 8
    q, k, v = rand(2, B * N, B * N, Hq, Hkv, D)
    cu = offsets([N] * B)
    for causal, window in ((False, (-1, -1)), (True, (-1, -1)), (False, (3, 2))):
        out, lse = attention_varlen_fp64(q, k, v, cu, cu, 0.3, causal, window)
        do, dl = attention_fp64(q.reshape(B, N, Hq, D), k.reshape(B, N, Hkv, D), v.reshape(B, N, Hkv, D), 0.3, causal, window)
        assert np.allclose(out.reshape(B, N, Hq, D), do, rtol=1e-13, atol=1e-13)
        assert np.allclose(lse.reshape(Hq, B, N).transpose(1, 0, 2), dl, rtol=1e-13, atol=1e-13)


def test_varlen_sequence_order_and_empty_sequences():
    lq, lk = [4, 7, 2], [6, 7, 3]
    cu_q, cu_k = offsets(lq), offsets(lk)
    q, k, v = rand(3, cu_q[-1], cu_k[-1], 2, 1, 4)
    out, lse = attention_varlen_fp64(q, k, v, cu_q, cu_k, 0.5, True)
    # reversed order
    rq = np.concatenate([q[cu_q[b]:cu_q[b + 1]] for b in (2, 1, 0)])
    rk = np.concatenate([k[cu_k[b]:cu_k[b + 1]] for b in (2, 1, 0)])
    rv = np.concatenate([v[cu_k[b]:cu_k[b + 1]] for b in (2, 1, 0)])
    ro, rl = attention_varlen_fp64(rq, rk, rv, offsets(lq[::-1]), offsets(lk[::-1]), 0.5, True)
    back = np.concatenate([np.arange(cu_q[b], cu_q[b + 1]) for b in (2, 1, 0)])
    assert np.array_equal(ro, out[back]) and np.array_equal(rl, lse[:, back])
    # an empty sequence appended and prepended
    eo, el = attention_varlen_fp64(q, k, v, np.concatenate([[0], cu_q, [cu_q[-1]]]),
                                   np.concatenate([[0], cu_k, [cu_k[-1]]]), 0.5, True)
    assert np.array_equal(eo, out) and np.array_equal(el, lse)
    # queries without keys
    zo, zl = attention_varlen_fp64(q[:4], k[:0], v[:0], [0, 4], [0, 0], 0.5)
    assert np.all(zo == 0) and np.all(zl == -np.inf)


# ---- planted mistakes --------------------------------------------------------------------------
def _mut_boundary(q, k, v, cu_q, cu_k, scale=None, causal=False, window=(-1, -1)):
    cu_k = np.asarray(cu_k).copy()
    cu_k[1:-1] += 1                                  # each sequence takes the next one's first key
    return _REAL(q, k, v, cu_q, cu_k, scale, causal, window)


def _mut_packed_alignment(q, k, v, cu_q, cu_k, scale=None, causal=False, window=(-1, -1)):
    # masks on the packed index with one global offset instead of each sequence's own
    from oracle.attention import _one_head, admitted, kv_head_of
    total_q, Hq, D = q.shape
    mask_all = admitted(total_q, k.shape[0], causal, window[0], window[1])
    out = np.zeros((total_q, Hq, D))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs or ke == ks:
            continue
        m = mask_all[qs:qe, ks:ke]
        for h in range(Hq):
            g = kv_head_of(h, Hq, k.shape[1])
            o, ls = _one_head(q[qs:qe, h], k[ks:ke, g], v[ks:ke, g], scale, m)
            out[qs:qe, h] = o
            lse[h, qs:qe] = ls
    return out, lse


def _mut_shared_keys(q, k, v, cu_q, cu_k, scale=None, causal=False, window=(-1, -1)):
    # every sequence attends to all packed keys
    return _shared(q, k, v, cu_q, scale, causal, window)


def _shared(q, k, v, cu_q, scale, causal, window):
    from oracle.attention import _one_head, admitted, kv_head_of
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        qs, qe = cu_q[b], cu_q[b + 1]
        if qe == qs:
            continue
        m = admitted(qe - qs, k.shape[0], causal, window[0], window[1])
        for h in range(Hq):
            g = kv_head_of(h, Hq, k.shape[1])
            o, ls = _one_head(q[qs:qe, h], k[:, g], v[:, g], scale, m)
            out[qs:qe, h] = o
            lse[h, qs:qe] = ls
    return out, lse


_REAL = OV.attention_varlen_fp64


@pytest.mark.parametrize("mutant", [_mut_boundary, _mut_packed_alignment, _mut_shared_keys])
def test_varlen_pins_catch_mutants(monkeypatch, mutant):
    import tests.test_oracle_varlen_pins as me
    monkeypatch.setattr(me, "attention_varlen_fp64", mutant)
    failures = 0
    for case in CASES:
        try:
            test_varlen_matches_block_diagonal_sdpa(case)
        except AssertionError:
            failures += 1
    assert failures >= 1
