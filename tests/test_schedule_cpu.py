"""The order in which forward launches visit their work (fa_block_order, the schedule the kernels
use): every (batch, head, query tile) exactly once, and the XCD placement each launch kind is
built for. Workgroup id goes to XCD id % 8 (the hardware deals blocks round-robin)."""
import itertools

import numpy as np
import pytest

import exact_attention_09_amd as fa


def order(B, H, group, tiles, causal, packed):
    return fa.block_order(B * H * tiles, tiles, H, group, causal, packed)


CASES = [
    # B, H, group, tiles, causal, packed
    (4, 32, 1, 16, True, False),     # causal [4, 4096, 32, 64], 256-row tiles
    (1, 32, 4, 64, True, False),     # causal GQA [1, 16384, 32/8, 128]
    (1, 32, 32, 64, True, False),    # causal MQA
    (4, 32, 1, 16, False, False),
    (2, 3, 1, 5, True, False),       # heads not a multiple of 8
    (3, 5, 5, 7, False, False),
    (8, 32, 1, 16, True, True),      # packed batch, MHA
    (16, 32, 4, 32, True, True),     # packed batch, GQA
    (8, 8, 8, 3, True, True),        # packed batch, one K/V head per sequence
    (3, 16, 2, 9, True, True),       # packed, 8 K/V heads per sequence
    (4, 2, 1, 9, True, True),        # packed, 2 K/V heads per sequence
    (5, 4, 2, 6, True, True),
    (3, 6, 3, 4, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_H{}_g{}_t{}_c{}_p{}".format(*map(int, c)))
def test_every_tile_once(case):
    B, H, group, tiles, causal, packed = case
    b, h, t = order(*case)
    got = sorted(zip(b.tolist(), h.tolist(), t.tolist()))
    assert got == list(itertools.product(range(B), range(H), range(tiles)))


def xcd_of(n):
    return np.arange(n) % 8


@pytest.mark.parametrize("case", [c for c in CASES if c[4] and not c[5] and (c[0] * c[1]) % 8 == 0])
def test_causal_whole_heads_per_xcd_longest_first(case):
    """Dense causal launches: each head runs entirely on one XCD (its K/V in one L2), the heads of
    one K/V head under 4-way GQA on the same XCD, and on each XCD a head's tiles start longest first."""
    B, H, group, tiles, _, _ = case
    b, h, t = order(*case)
    x = xcd_of(len(b))
    bh = b * H + h
    for head in range(B * H):
        assert len(set(x[bh == head])) == 1
        # ids on one XCD are dispatched in id order: tiles of a head in decreasing length
        assert (np.diff(t[bh == head]) < 0).all()
    if group == 4:
        kv = bh // group
        for u in range(B * H // group):
            assert len(set(x[kv == u])) == 1


@pytest.mark.parametrize("case", [c for c in CASES if c[5] and (c[1] // c[2]) % 8 == 0])
def test_packed_kv_heads_dealt_over_xcds(case):
    """Packed batches with K/V heads per sequence a multiple of 8: K/V head u = (batch, K/V head)
    runs on XCD u % 8, so every XCD holds the same
    share of every sequence; on each XCD the query heads are visited a few at a time (the chunk in
    flight), each head's tiles highest first."""
    B, H, group, tiles, _, _ = case
    b, h, t = order(*case)
    n = len(b)
    x = xcd_of(n)
    u = (b * H + h) // group
    assert (u % 8 == x).all()
    for xc in range(8):
        counts = np.bincount(b[x == xc], minlength=B)
        assert (counts == counts[0]).all()          # equal share of every sequence
    hx = B * H // 8
    c = 4 if hx % 4 == 0 else (2 if hx % 2 == 0 else 1)
    for xc in range(8):
        ids = np.nonzero(x == xc)[0]                 # dispatch order on this XCD
        bh = (b * H + h)[ids]
        for k0 in range(0, len(ids), c * tiles):     # one chunk: c heads, all their tiles
            assert len(set(bh[k0:k0 + c * tiles].tolist())) == c
        for head in set(bh.tolist()):
            assert (np.diff(t[ids][bh == head]) < 0).all()


def test_non_causal_contiguous_heads_per_xcd():
    B, H, tiles = 4, 32, 16
    b, h, t = order(B, H, 1, tiles, False, False)
    x = xcd_of(len(b))
    bh = b * H + h
    for xc in range(8):
        heads = sorted(set(bh[x == xc].tolist()))
        assert heads == list(range(heads[0], heads[0] + len(heads)))


@pytest.mark.parametrize("args", [(0, 1, 1, 1), (8, 0, 1, 1), (8, 1, 0, 1), (8, 1, 4, 3), (10, 3, 1, 1),
                                  (1 << 31, 1, 1, 1)])
def test_rejects_bad_shapes(args):
    n, tiles, heads, group = args
    with pytest.raises(fa.FaError):
        fa.block_order(n, tiles, heads, group)


def expected_order(B, H, group, tiles, causal, packed):
    """The launch order written out with plain integer division (the rules the kernels follow)."""
    n = B * H * tiles
    n_bh = B * H
    hx = n_bh // 8
    c = 4 if hx % 4 == 0 else (2 if hx % 2 == 0 else 1)

    def xcd_remap(i):
        x, k = i & 7, i >> 3
        per, rem = n >> 3, n & 7
        return x * per + min(x, rem) + k

    out = []
    for i in range(n):
        if packed and (H // group) % 8 == 0:
            x, k = i & 7, i >> 3
            chunk, r = divmod(k, c * tiles)
            rank, pi = r // c, chunk * c + r % c
            bh = ((pi // group) * 8 + x) * group + pi % group
            t = tiles - 1 - rank
        elif packed or (causal and n_bh % 8):
            rank, bh = divmod(i, n_bh)
            t = tiles - 1 - rank
        elif not causal:
            bh, t = divmod(xcd_remap(i), tiles)
        else:
            chunk, r = divmod(xcd_remap(i), c * tiles)
            rank = r // c
            bh, t = chunk * c + r % c, tiles - 1 - rank
        out.append((bh // H, bh % H, t))
    return out


@pytest.mark.parametrize("case", CASES + [(7, 24, 3, 11, True, False), (9, 16, 2, 13, False, True),
                                          (2, 48, 6, 5, True, True), (1, 8, 1, 1, True, False)],
                         ids=lambda c: "B{}_H{}_g{}_t{}_c{}_p{}".format(*map(int, c)))
def test_matches_plain_division(case):
    """The kernels divide by launch constants with host-computed multipliers; the order must be the
    one plain integer division gives."""
    b, h, t = order(*case)
    assert list(zip(b.tolist(), h.tolist(), t.tolist())) == expected_order(*case)
