"""Pins of the block-sparse oracle (``oracle.blocksparse``) to facts outside its own code (CPU).

  * an independent library routine: torch CPU fp64 scaled_dot_product_attention with a boolean
    mask built here from the block mask by torch.repeat_interleave (rows by block_q, keys by
    block_k), intersected with tril / triu masks;
  * special cases that reduce to the pinned dense oracle: an all-ones block mask is dense
    attention; a block mask that sets exactly the blocks a causal mask touches changes nothing
    under that causal mask;
  * closed form: a block mask with only the diagonal blocks of equal-sized blocks is a batch of
    independent block-local attentions (each block equal to the dense oracle on its own slice).
Planted mistakes (transposed block mask, query and key block sizes swapped, the mask ignored for
one head) must each fail a pin.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.blocksparse as OBS
from oracle import attention_blocksparse_fp64, attention_fp64


def rand(seed, B, Nq, Nk, Hq, Hkv, D):
    g = np.random.default_rng(seed)
    return g.standard_normal((B, Nq, Hq, D)), g.standard_normal((B, Nk, Hkv, D)), g.standard_normal((B, Nk, Hkv, D))


def rand_mask(seed, Hm, Nq, Nk, bq, bk, p=0.4):
    g = np.random.default_rng(seed)
    return (g.random((Hm, -(-Nq // bq), -(-Nk // bk))) < p).astype(np.uint8)


def torch_ref(q, k, v, bm, bq, bk, scale, causal, window):
    B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    off = Nk - Nq
    base = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        base &= torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=off)
    if window[0] >= 0:
        base &= torch.ones(Nq, Nk, dtype=torch.bool).triu(diagonal=off - window[0])
    if window[1] >= 0:
        base &= torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=off + window[1])
    out = np.zeros_like(q)
    lse = np.zeros((B, Hq, Nq))
    for h in range(Hq):
        blk = torch.tensor(bm[0 if bm.shape[0] == 1 else h] != 0)
        full = blk.repeat_interleave(bq, dim=0)[:Nq].repeat_interleave(bk, dim=1)[:, :Nk]
        m = base & full
        live = m.any(dim=1)
        msafe = m.clone()
        msafe[~live, 0] = True
        qt = torch.tensor(q[:, :, h, :])[:, None]
        kt = torch.tensor(k[:, :, h // G, :])[:, None]
        vt = torch.tensor(v[:, :, h // G, :])[:, None]
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=msafe, scale=scale)[:, 0]
        o[:, ~live] = 0
        out[:, :, h, :] = o.numpy()
        s = scale * qt[:, 0] @ kt[:, 0].transpose(1, 2)
        lse[:, h, :] = torch.logsumexp(s.masked_fill(~m[None], float("-inf")), dim=-1).numpy()
    return out, lse


CASES = [
    # B, Nq, Nk, Hq, Hkv, D, bq, bk, heads of the mask, causal, window
    (1, 20, 20, 2, 2, 8, 4, 2, 1, False, (-1, -1)),
    (2, 17, 23, 4, 2, 8, 4, 4, 4, False, (-1, -1)),   # ragged blocks, a mask per head
    (1, 24, 24, 3, 1, 4, 8, 4, 3, True, (-1, -1)),
    (1, 30, 30, 2, 1, 8, 4, 2, 1, True, (5, -1)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[1]}x{c[2]}_H{c[3]}-{c[4]}_b{c[6]}x{c[7]}_m{c[8]}_c{int(c[9])}")
def test_blocksparse_matches_torch_mask(case):
    B, Nq, Nk, Hq, Hkv, D, bq, bk, Hm, causal, window = case
    q, k, v = rand(1, B, Nq, Nk, Hq, Hkv, D)
    bm = rand_mask(2, Hm, Nq, Nk, bq, bk)
    out, lse = OBS.attention_blocksparse_fp64(q, k, v, bm, bq, bk, 0.4, causal, window)
    ro, rl = torch_ref(q, k, v, bm, bq, bk, 0.4, causal, window)
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(rl))
    fin = np.isfinite(rl)
    assert np.allclose(lse[fin], rl[fin], rtol=1e-12, atol=1e-12)


def test_blocksparse_all_ones_and_causal_blocks_are_dense():
    B, Nq, Nk, Hq, Hkv, D, bq, bk = 1, 26, 26, 2, 2, 8, 8, 4
    q, k, v = rand(3, B, Nq, Nk, Hq, Hkv, D)
    ones = np.ones((1, -(-Nq // bq), -(-Nk // bk)), dtype=np.uint8)
    for causal in (False, True):
        o, l = attention_blocksparse_fp64(q, k, v, ones, bq, bk, 0.3, causal)
        do, dl = attention_fp64(q, k, v, 0.3, causal)
        assert np.allclose(o, do, atol=1e-14) and np.allclose(l, dl, atol=1e-14)
    # the blocks a causal mask touches: (qb, kb) with kb * bk <= last row of qb
    cb = np.array([[[1 if kb * bk <= min(Nq, (qb + 1) * bq) - 1 else 0 for kb in range(-(-Nk // bk))]
                    for qb in range(-(-Nq // bq))]], dtype=np.uint8)
    o, l = attention_blocksparse_fp64(q, k, v, cb, bq, bk, 0.3, True)
    do, dl = attention_fp64(q, k, v, 0.3, True)
    assert np.allclose(o, do, atol=1e-14) and np.allclose(l, dl, atol=1e-14)


def test_blocksparse_diagonal_blocks_are_local_attention():
    B, N, Hq, Hkv, D, bsz = 1, 24, 2, 2, 8, 8
    q, k, v = rand(4, B, N, N, Hq, Hkv, D)
    diag = np.eye(N // bsz, dtype=np.uint8)[None]
    o, l = attention_blocksparse_fp64(q, k, v, diag, bsz, bsz, 0.5)
    for blk in range(N // bsz):
        sl = slice(blk * bsz, (blk + 1) * bsz)
        do, dl = attention_fp64(q[:, sl], k[:, sl], v[:, sl], 0.5)
        assert np.allclose(o[:, sl], do, atol=1e-14) and np.allclose(l[:, :, sl], dl, atol=1e-14)


# ---- planted mistakes --------------------------------------------------------------------------
def _mut_transposed(block_mask_2d, Nq, Nk, block_q, block_k, rows=None):
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    bm = np.asarray(block_mask_2d) != 0
    kb = np.minimum(np.arange(Nk) // block_k, bm.shape[0] - 1)
    qb = np.minimum(i // block_q, bm.shape[1] - 1)
    return bm[kb[None, :], qb[:, None]]


def _mut_swapped_sizes(block_mask_2d, Nq, Nk, block_q, block_k, rows=None):
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    bm = np.asarray(block_mask_2d) != 0
    qb = np.minimum(i // block_k, bm.shape[0] - 1)
    kb = np.minimum(np.arange(Nk) // block_q, bm.shape[1] - 1)
    return bm[qb[:, None], kb[None, :]]


@pytest.mark.parametrize("mutant", [_mut_transposed, _mut_swapped_sizes])
def test_blocksparse_pins_catch_mask_mutants(monkeypatch, mutant):
    monkeypatch.setattr(OBS, "block_admitted", mutant)
    failures = 0
    for case in CASES:
        try:
            test_blocksparse_matches_torch_mask(case)
        except (AssertionError, IndexError):
            failures += 1
    assert failures >= 1


def test_blocksparse_pins_catch_head_mistake(monkeypatch):
    real = OBS.block_admitted
    calls = {"n": 0}

    def mutant(block_mask_2d, Nq, Nk, block_q, block_k, rows=None):
        calls["n"] += 1
        if calls["n"] % 2 == 0:                     # every second head ignores its mask
            i = np.arange(Nq) if rows is None else np.asarray(rows)
            return np.ones((len(i), Nk), dtype=bool)
        return real(block_mask_2d, Nq, Nk, block_q, block_k, rows)

    monkeypatch.setattr(OBS, "block_admitted", mutant)
    with pytest.raises(AssertionError):
        test_blocksparse_matches_torch_mask(CASES[1])
