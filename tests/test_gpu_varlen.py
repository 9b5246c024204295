"""GPU parity of fa_fwd_varlen (packed variable-length batches, through the C ABI) against the fp64
varlen oracle (``oracle.varlen``, readings RV1-RV3).

Bars as for the dense forward: fp16 max|dout| <= 2e-3, bf16 <= 1.5e-2, fp8 RMS(err) <= 6e-2 *
RMS(out), lse within 1e-3, no NaN/Inf; sequences with queries and no keys give exactly 0 / -inf.
Equal-length sequences must give bitwise the dense kernel's result (the same arithmetic).
"""
import numpy as np
import pytest
import torch

import exact_attention_09_amd as fa
from exact_attention_09_amd.inputs import VARLEN_WORKLOADS, make_varlen_inputs
from oracle import attention_rows_fp64, attention_varlen_fp64
from tests.gpu_util import DTYPE_NAME, compare, decode, out_to_f64

pytestmark = pytest.mark.gpu


def run(q, k, v, cu_q, cu_k, max_q, causal, window, scale, descale):
    out, lse = fa.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max_q, causal, window, scale,
                             descale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check(lq, lk, Hq, Hkv, D, dtype, causal, window, seed, max_q=None):
    q, k, v, cu_q, cu_k, d = make_varlen_inputs(lq, lk, Hq, Hkv, D, dtype, seed)
    scale = D ** -0.5
    out, lse = run(q, k, v, cu_q, cu_k, max_q or max(max(lq), 1), causal, window, scale, d)
    dq, dk, dv = d if d is not None else (1.0, 1.0, 1.0)
    ro, rl = attention_varlen_fp64(decode(q, dq), decode(k, dk), decode(v, dv), cu_q.numpy(), cu_k.numpy(), scale,
                                   causal, window)
    compare(DTYPE_NAME[q.dtype], out_to_f64(out), lse.numpy().astype(np.float64), ro, rl,
            f"varlen {lq} {lk} {dtype} c{causal} w{window}")
    return out, lse, cu_q


MIXES = [
    # lengths_q, lengths_k, Hq, Hkv, D, causal, window
    ([1, 77, 300, 129, 256], None, 4, 2, 64, True, (-1, -1)),
    ([513, 64, 1000], None, 2, 1, 128, True, (-1, -1)),
    ([200, 333, 17], [333, 200, 40], 4, 4, 64, False, (-1, -1)),     # Nq != Nk inside sequences
    ([300, 0, 45, 260], [300, 12, 45, 0], 4, 2, 128, True, (37, 11)),  # empty queries, keys-less rows
    ([640, 7, 384], None, 2, 2, 64, False, (100, 100)),
    ([190, 190, 190], None, 6, 3, 128, True, (64, -1)),
    # 8 K/V heads per sequence: the launch deals K/V heads over the XCDs by chunks of query heads
    ([300, 1000, 77, 512], None, 16, 8, 64, True, (-1, -1)),
    ([129, 640], None, 8, 8, 128, False, (-1, -1)),
    # windows with 4-way GQA: four query heads of one K/V head per workgroup
    ([300, 1000, 77, 512], None, 16, 4, 128, True, (100, -1)),
    ([200, 0, 333], [250, 40, 333], 8, 2, 64, False, (60, 30)),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3"])
@pytest.mark.parametrize("mix", MIXES, ids=lambda m: f"q{'-'.join(map(str, m[0]))}_D{m[4]}_c{int(m[5])}_w{m[6][0]}_{m[6][1]}")
def test_varlen_matches_oracle(mix, dtype):
    lq, lk, Hq, Hkv, D, causal, window = mix
    out, lse, cu_q = check(lq, lk or lq, Hq, Hkv, D, dtype, causal, window, seed=sum(lq) + D)
    lk = lk or lq
    for b, (nq, nk) in enumerate(zip(lq, lk)):
        if nq and not nk:     # queries with no keys: exactly 0 and -inf
            rows = slice(int(cu_q[b]), int(cu_q[b + 1]))
            assert torch.all(out[rows].float() == 0) and torch.all(torch.isneginf(lse[:, rows]))


def test_varlen_larger_max_seqlen_is_harmless():
    check([100, 300], [100, 300], 2, 2, 64, "f16", True, (-1, -1), seed=3, max_q=400)   # the limit: total_q


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3"])
def test_varlen_equal_lengths_bitwise_dense(dtype):
    B, N, Hq, Hkv, D = 3, 300, 4, 2, 64
    q, k, v, cu_q, cu_k, d = make_varlen_inputs([N] * B, [N] * B, Hq, Hkv, D, dtype, seed=11)
    out, lse = run(q, k, v, cu_q, cu_k, N, True, (-1, -1), 0.125, d)
    do, dl = fa.fwd(q.reshape(B, N, Hq, D).cuda(), k.reshape(B, N, Hkv, D).cuda(), v.reshape(B, N, Hkv, D).cuda(),
                    True, (-1, -1), 0.125, d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), do.cpu().reshape(B * N, Hq, D).view(torch.int16))
    assert torch.equal(lse, dl.cpu().permute(1, 0, 2).reshape(Hq, B * N))


@pytest.mark.parametrize("name", list(VARLEN_WORKLOADS))
def test_varlen_benchmark_workload_sampled(name):
    """The benchmark's packed batches in the launch it times, written into NaN-filled outputs: every
    element is written, and the first and last 16 rows of every sequence (heads 0 and Hq-1) and
    the first and last 4 rows (every other head) match the oracle of that sequence alone (reading
    RV1: a packed sequence is the dense problem of its own lengths; the dense oracle's row
    sampler)."""
    w = VARLEN_WORKLOADS[name]
    lens = w.lengths(0)
    q, k, v, cu_q, cu_k, d = make_varlen_inputs(lens, lens, w.Hq, w.Hkv, w.D, w.dtype, seed=0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float16 if w.dtype == "f16" else torch.bfloat16,
                     device="cuda")
    lse = torch.full((w.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    st = fa.fwd_varlen_raw(qd, kd, vd, out, lse, cu_q.cuda(), cu_k.cuda(), max(lens), w.causal, w.window,
                           w.softmax_scale(), d)
    torch.cuda.synchronize()
    assert st == 0, fa.status_str(st)
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    G = w.Hq // w.Hkv
    for b, n in enumerate(lens):
        s = int(cu_q[b])
        for h in range(w.Hq):
            rows = np.r_[0:16, n - 16:n] if h in (0, w.Hq - 1) else np.r_[0:4, n - 4:n]
            g = h // G
            qh = decode(q[s:s + n, h])[None, :, None, :]
            kh = decode(k[s:s + n, g])[None, :, None, :]
            vh = decode(v[s:s + n, g])[None, :, None, :]
            ro, rl = attention_rows_fp64(qh, kh, vh, 0, 0, rows, w.softmax_scale(), w.causal, w.window)
            got_o = out_to_f64(out[s:s + n, h])[rows]
            got_l = lse[h, s:s + n].numpy().astype(np.float64)[rows]
            compare(w.dtype, got_o, got_l, ro, rl, f"{name} seq {b} head {h}")


@pytest.mark.parametrize("name", list(VARLEN_WORKLOADS))
def test_varlen_benchmark_workload_every_element_equals_dense(name):
    """Every element of the benchmark's packed batches, in the launch it times, against one dense
    launch per sequence (its rows of the packed tensors as a [1, n, H, D] view), bit for bit: a
    packed sequence is the dense problem of its own lengths with the same tiles and arithmetic
    (reading RV1), so only a tile that the packed launch order skipped or computed twice, or a
    sequence offset gone wrong, would differ. The dense launches are held to the oracle by the
    dense tests; the packed one on sampled rows above."""
    w = VARLEN_WORKLOADS[name]
    lens = w.lengths(0)
    q, k, v, cu_q, cu_k, d = make_varlen_inputs(lens, lens, w.Hq, w.Hkv, w.D, w.dtype, seed=0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    odt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    out = torch.full(q.shape, float("nan"), dtype=odt, device="cuda")
    lse = torch.full((w.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    st = fa.fwd_varlen_raw(qd, kd, vd, out, lse, cu_q.cuda(), cu_k.cuda(), max(lens), w.causal, w.window,
                           w.softmax_scale(), d)
    assert st == 0, fa.status_str(st)
    for b, n in enumerate(lens):
        s = int(cu_q[b])
        do, dl = fa.fwd(qd[s:s + n].unsqueeze(0), kd[s:s + n].unsqueeze(0), vd[s:s + n].unsqueeze(0), w.causal,
                        w.window, w.softmax_scale(), d)
        torch.cuda.synchronize()
        assert torch.equal(out[s:s + n].view(torch.int16), do[0].view(torch.int16)), f"out of sequence {b}"
        assert torch.equal(lse[:, s:s + n], dl[0]), f"lse of sequence {b}"
