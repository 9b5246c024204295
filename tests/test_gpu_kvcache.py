"""GPU parity of fa_fwd_kvcache (queries against a dense or paged KV cache, keys split over
workgroups and merged, through the C ABI) against the fp64 KV-cache oracle (``oracle.kvcache``,
readings RK1-RK2).

Bars as for the forward pass: fp16 max|dout| <= 2e-3, bf16 <= 1.5e-2, lse within 1e-3, no
NaN/Inf; sequences with no keys give exactly 0 / -inf; results bitwise deterministic.
"""
import numpy as np
import pytest
import torch

import exact_attention_09_amd as fa
from exact_attention_09_amd.inputs import KVCACHE_WORKLOADS, make_kvcache_inputs
from oracle import attention_kvcache_fp64
from tests.gpu_util import compare, decode, out_to_f64

pytestmark = pytest.mark.gpu


def run(q, k, v, seqlens, table, max_k, causal=False, window=(-1, -1), scale=None):
    out, lse = fa.fwd_kvcache(q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(),
                              table.cuda() if table is not None else None, max_k, causal, window, scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


CASES = [
    # B, Nq, Hq, Hkv, D, lengths, page_size, causal, window, dtype
    (3, 1, 8, 2, 128, [1, 700, 5000], 16, False, (-1, -1), "bf16"),
    (2, 1, 32, 1, 64, [4096, 33], 16, False, (-1, -1), "f16"),       # MQA: 32 rows in one wave
    (2, 4, 8, 2, 128, [3000, 9], 64, True, (-1, -1), "bf16"),        # 4 new tokens, causal among them
    (2, 5, 8, 1, 64, [1200, 0], 32, True, (-1, -1), "f16"),          # 40 rows: two row blocks; a sequence with no keys
    (1, 2, 4, 4, 128, [2048], 0, True, (100, -1), "bf16"),           # dense cache, window
    (3, 1, 4, 2, 64, [31, 32, 33], 0, False, (-1, -1), "f16"),       # block edges, one split
    (2, 3, 6, 3, 128, [777, 2500], 1, True, (-1, -1), "f16"),        # one-token pages
    # 16 or more splits per (sequence, K/V head) switch the launch order from split-major to
    # consecutive splits of one pair (every case above has fewer)
    (2, 1, 8, 2, 64, [9000, 4100], 16, False, (-1, -1), "bf16"),     # 18 splits of 512 keys
    (1, 3, 8, 4, 128, [12000], 0, True, (-1, -1), "f16"),            # dense cache, 24 splits
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_Nq{c[1]}_H{c[2]}-{c[3]}_D{c[4]}_P{c[6]}_c{int(c[7])}_{c[9]}")
def test_kvcache_matches_oracle(case):
    B, Nq, Hq, Hkv, D, lens, P, causal, window, dtype = case
    q, k, v, seqlens, table = make_kvcache_inputs(B, Nq, Hq, Hkv, D, dtype, lens, P, seed=sum(lens) + Nq)
    max_k = max(lens) + 7
    if P == 0:
        k = torch.cat([k, torch.zeros(B, 7, Hkv, D, dtype=k.dtype)], dim=1)   # a cache longer than any sequence
        v = torch.cat([v, torch.zeros(B, 7, Hkv, D, dtype=v.dtype)], dim=1)
    scale = D ** -0.5
    out, lse = run(q, k, v, seqlens, table, max_k, causal, window, scale)
    ro, rl = attention_kvcache_fp64(decode(q), decode(k), decode(v), lens, table.numpy() if table is not None else None,
                                    P, scale, causal, window)
    compare(dtype, out_to_f64(out), lse.numpy().astype(np.float64), ro, rl, str(case))
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.all(out[b].float() == 0) and torch.all(torch.isneginf(lse[b]))


def test_kvcache_deterministic_and_page_order_free():
    B, Nq, Hq, Hkv, D, lens, P = 4, 2, 8, 2, 128, [5000, 3000, 100, 4096], 16
    q, k, v, seqlens, table = make_kvcache_inputs(B, Nq, Hq, Hkv, D, "bf16", lens, P, seed=1)
    a = run(q, k, v, seqlens, table, 5000, True)
    b = run(q, k, v, seqlens, table, 5000, True)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])
    # the same keys in other physical pages give bitwise the same result
    perm = torch.randperm(k.shape[0], generator=torch.Generator().manual_seed(3))
    inv = torch.argsort(perm)
    c = run(q, k[perm], v[perm], seqlens, inv[table.long()].to(torch.int32), 5000, True)
    assert torch.equal(a[0].view(torch.int16), c[0].view(torch.int16)) and torch.equal(a[1], c[1])


@pytest.mark.parametrize("name", list(KVCACHE_WORKLOADS))
def test_kvcache_benchmark_workload_sampled(name):
    """The benchmark's cache and launch; 6 sequences (the shortest, the longest and 4 more)
    checked in full against the oracle run on those sequences alone."""
    w = KVCACHE_WORKLOADS[name]
    lens = w.lengths(0)
    q, k, v, seqlens, table = make_kvcache_inputs(w.B, w.Nq, w.Hq, w.Hkv, w.D, w.dtype, lens, w.page_size, seed=0)
    out, lse = run(q, k, v, seqlens, table, max(lens), w.causal, (-1, -1), w.softmax_scale())
    assert torch.isfinite(out.float()).all()
    order = np.argsort(lens)
    pick = sorted({int(order[0]), int(order[-1]), 1, w.B // 3, w.B // 2, w.B - 2})
    for b in pick:
        sl = slice(b, b + 1)
        n = lens[b]
        if table is not None:
            # this sequence's pages only, renumbered 0 .. npg-1 (decoding the whole pool would take
            # tens of GB in fp64)
            npg = (n + w.page_size - 1) // w.page_size
            pages = table[b, :npg].long()
            kb, vb = k[pages], v[pages]
            tb = np.arange(npg, dtype=np.int64)[None]
        else:
            kb, vb, tb = k[sl, :n], v[sl, :n], None
        ro, rl = attention_kvcache_fp64(decode(q[sl]), decode(kb), decode(vb), [n], tb, w.page_size,
                                        w.softmax_scale(), w.causal)
        compare(w.dtype, out_to_f64(out[sl]), lse[sl].numpy().astype(np.float64), ro, rl, f"{name} seq {b}")


def test_kvcache_paged_benchmark_every_element_equals_dense_cache():
    """Every element of the paged benchmark workload (128 sequences of 512-8192 keys, 16-key pages):
    the paged launch against the same keys gathered into a dense cache, bit for bit. The split of
    each sequence's keys and every product are the same for both layouts (the page table only
    decides where a key is read from), so only a page gathered wrongly would differ; the dense
    cache is held to the oracle above."""
    w = KVCACHE_WORKLOADS["decode_paged16_b128_len512to8192_hq32_hkv8_d128_bf16"]
    lens = w.lengths(0)
    q, k, v, seqlens, table = make_kvcache_inputs(w.B, w.Nq, w.Hq, w.Hkv, w.D, w.dtype, lens, w.page_size, seed=0)
    max_k = max(lens)
    qd, kd, vd, sd, td = q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(), table.cuda()
    paged = fa.fwd_kvcache(qd, kd, vd, sd, td, max_k, w.causal, (-1, -1), w.softmax_scale())
    npg = (max_k + w.page_size - 1) // w.page_size
    idx = td[:, :npg].long()
    kdense = kd[idx].reshape(w.B, npg * w.page_size, w.Hkv, w.D)
    vdense = vd[idx].reshape(w.B, npg * w.page_size, w.Hkv, w.D)
    dense = fa.fwd_kvcache(qd, kdense, vdense, sd, None, max_k, w.causal, (-1, -1), w.softmax_scale())
    torch.cuda.synchronize()
    assert torch.equal(paged[0].view(torch.int16), dense[0].view(torch.int16))
    assert torch.equal(paged[1], dense[1])
