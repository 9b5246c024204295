"""Pins of the KV-cache oracle (``oracle.kvcache``) to facts outside its own code (CPU only).

  * an independent library routine: torch CPU fp64 scaled_dot_product_attention on keys and
    values gathered with torch indexing from the flattened page pool (index = page * page_size +
    slot, built here from the block table), causal masks from torch.tril with the bottom-right
    diagonal;
  * invariants: shuffling the physical pages (and the block table with them) changes nothing;
    a paged cache laid out in order equals the dense cache;
  * closed forms: one query against n identical keys gives the mean of the values and
    lse = s + ln n; a sequence with no keys gives 0 and -inf.
Planted mistakes (slot and page swapped, another sequence's block table, top-left causal
alignment) must each fail a pin.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.kvcache as OK
from oracle import attention_fp64
from oracle.kvcache import attention_kvcache_fp64


def make_cache(seed, B, Nq, Hq, Hkv, D, lens, P):
    g = np.random.default_rng(seed)
    pages_per = [(n + P - 1) // P for n in lens]
    num_pages = sum(pages_per) + 3
    perm = g.permutation(num_pages)
    table = np.full((B, max(max(pages_per), 1)), -1, dtype=np.int64)
    at = 0
    for b, npg in enumerate(pages_per):
        table[b, :npg] = perm[at:at + npg]
        at += npg
    q = g.standard_normal((B, Nq, Hq, D))
    kc = g.standard_normal((num_pages, P, Hkv, D))
    vc = g.standard_normal((num_pages, P, Hkv, D))
    return q, kc, vc, table


def torch_ref(q, kc, vc, lens, table, P, scale, causal):
    B, Nq, Hq, D = q.shape
    Hkv = kc.shape[2]
    G = Hq // Hkv
    flat_k = torch.tensor(kc).reshape(-1, Hkv, D)
    flat_v = torch.tensor(vc).reshape(-1, Hkv, D)
    out = np.zeros_like(q)
    lse = np.full((B, Hq, Nq), -np.inf)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        j = torch.arange(n)
        idx = torch.tensor(table[b])[j // P] * P + j % P
        kb = flat_k.index_select(0, idx).permute(1, 0, 2).repeat_interleave(G, dim=0)
        vb = flat_v.index_select(0, idx).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qb = torch.tensor(q[b]).permute(1, 0, 2)
        mask = torch.ones(Nq, n, dtype=torch.bool)
        if causal:
            mask = mask.tril(diagonal=n - Nq)
        live = mask.any(dim=1)
        msafe = mask.clone()
        msafe[~live, 0] = True
        o = F.scaled_dot_product_attention(qb[None], kb[None], vb[None], attn_mask=msafe, scale=scale)[0]
        o[:, ~live] = 0
        out[b] = o.permute(1, 0, 2).numpy()
        s = scale * qb @ kb.transpose(1, 2)
        lse[b] = torch.logsumexp(s.masked_fill(~mask[None], float("-inf")), dim=-1).numpy()
    return out, lse


CASES = [
    # B, Nq, Hq, Hkv, D, lens, P, causal
    (3, 1, 4, 2, 8, [5, 33, 16], 16, False),
    (2, 4, 4, 1, 8, [20, 7], 16, True),       # Nq > 1: bottom-right causal inside the cache
    (2, 3, 2, 2, 4, [9, 2], 4, True),         # Nq > keys for one sequence: its first row has no key
    (4, 2, 6, 3, 8, [0, 64, 1, 40], 32, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_Nq{c[1]}_H{c[2]}-{c[3]}_P{c[6]}_c{int(c[7])}")
def test_kvcache_matches_torch_gather_sdpa(case):
    B, Nq, Hq, Hkv, D, lens, P, causal = case
    q, kc, vc, table = make_cache(4, B, Nq, Hq, Hkv, D, lens, P)
    out, lse = attention_kvcache_fp64(q, kc, vc, lens, table, P, 0.35, causal)
    ro, rl = torch_ref(q, kc, vc, lens, table, P, 0.35, causal)
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(rl))
    fin = np.isfinite(rl)
    assert np.allclose(lse[fin], rl[fin], rtol=1e-12, atol=1e-12)


def test_kvcache_page_shuffle_and_dense_layout():
    B, Nq, Hq, Hkv, D, lens, P = 3, 2, 4, 2, 8, [17, 40, 3], 8
    q, kc, vc, table = make_cache(5, B, Nq, Hq, Hkv, D, lens, P)
    out, lse = attention_kvcache_fp64(q, kc, vc, lens, table, P, 0.3, True)
    g = np.random.default_rng(9)
    perm = g.permutation(kc.shape[0])          # new physical page p holds old page perm[p]
    inv = np.argsort(perm)
    t2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1)
    o2, l2 = attention_kvcache_fp64(q, kc[perm], vc[perm], lens, t2, P, 0.3, True)
    assert np.array_equal(o2, out) and np.array_equal(l2, lse)
    # the same keys in a dense [B, max_len, Hkv, D] cache, no block table
    maxlen = max(lens)
    dk = np.zeros((B, maxlen, Hkv, D))
    dv = np.zeros((B, maxlen, Hkv, D))
    for b, n in enumerate(lens):
        for j in range(n):
            dk[b, j] = kc[table[b, j // P], j % P]
            dv[b, j] = vc[table[b, j // P], j % P]
    o3, l3 = attention_kvcache_fp64(q, dk, dv, lens, None, 0, 0.3, True)
    assert np.array_equal(o3, out) and np.array_equal(l3, lse)
    for b, n in enumerate(lens):               # and each sequence is the dense definition
        ro, rl = attention_fp64(q[b:b + 1], dk[b:b + 1, :n], dv[b:b + 1, :n], 0.3, True)
        assert np.allclose(o3[b], ro[0], atol=1e-14) and np.allclose(l3[b], rl[0], atol=1e-14)


def test_kvcache_closed_forms():
    B, Nq, Hq, Hkv, D, P = 2, 1, 2, 1, 4, 4
    lens = [10, 0]
    q, kc, vc, table = make_cache(6, B, Nq, Hq, Hkv, D, lens, P)
    kc[:] = kc[0, 0]                           # every key the same
    out, lse = attention_kvcache_fp64(q, kc, vc, lens, table, P, 0.5)
    vals = np.stack([vc[table[0, j // P], j % P, 0] for j in range(10)])
    for h in range(Hq):
        s = 0.5 * q[0, 0, h] @ kc[0, 0, 0]
        assert np.allclose(out[0, 0, h], vals.mean(axis=0), atol=1e-13)
        assert np.isclose(lse[0, h, 0], s + np.log(10), atol=1e-13)
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)


# ---- planted mistakes --------------------------------------------------------------------------
def _mut_slot_page_swapped(cache, b, n, block_table=None, page_size=0):
    cache = np.asarray(cache)
    if block_table is None:
        return cache[b, :n]
    j = np.arange(n)
    return cache[np.asarray(block_table)[b, j % page_size], j // page_size]


def _mut_wrong_sequence(cache, b, n, block_table=None, page_size=0):
    cache = np.asarray(cache)
    if block_table is None:
        return cache[b, :n]
    bt = np.asarray(block_table)
    b2 = (b + 1) % bt.shape[0]
    j = np.arange(n)
    return cache[np.maximum(bt[b2, j // page_size], 0), j % page_size]


@pytest.mark.parametrize("mutant", [_mut_slot_page_swapped, _mut_wrong_sequence])
def test_kvcache_pins_catch_gather_mutants(monkeypatch, mutant):
    monkeypatch.setattr(OK, "gather_kv", mutant)
    failures = 0
    for case in CASES:
        try:
            test_kvcache_matches_torch_gather_sdpa(case)
        except (AssertionError, IndexError):
            failures += 1
    assert failures >= 1


def test_kvcache_pins_catch_top_left_causal(monkeypatch):
    real = OK.attention_fp64

    def top_left(q, k, v, scale=None, causal=False, window=(-1, -1), row_chunk=1024):
        if not causal or q.shape[1] == k.shape[1]:
            return real(q, k, v, scale, causal, window)
        # top-left alignment: query i sees keys 0..i
        Nq, Nk = q.shape[1], k.shape[1]
        out, lse = real(q, k[:, :Nq] if Nk >= Nq else k, v[:, :Nq] if Nk >= Nq else v, scale, True, window)
        return out, lse

    monkeypatch.setattr(OK, "attention_fp64", top_left)
    with pytest.raises(AssertionError):
        test_kvcache_matches_torch_gather_sdpa(CASES[1])
