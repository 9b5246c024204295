"""The largest tensors a call accepts: every head of q, k, v, out (and for the backward pass dout,
dq, dk, dv) spans as many bytes as the library's span rule allows (include/fa355.h,
FA_ERR_TOO_LARGE; the CPU test of the ABI checks that one 16-byte unit more is refused).

Each tensor is a strided view of a large device buffer: its rows sit the widest accepted stride
apart (a head of 2047 fp16 rows then spans about 1.9 GB), so the kernels' 32-bit in-head offsets
reach their top, and each batch starts more than 2^31 bytes after the one before (batch offsets
are 64-bit). Results must match the fp64 oracle at the usual bars; outputs start NaN-filled, so a
row written nowhere fails. The KV-cache calls, which address each key in 64 bits and have no
span limit, run with used pages past 4 GiB and sequences more than 2 GiB apart. Each case needs
8-35 GB of device memory and none of the host's beyond the small inputs.
"""
import numpy as np
import pytest
import torch

import exact_attention_09_amd as fa
from exact_attention_09_amd.inputs import draw_qkv, make_kvcache_inputs, make_varlen_inputs, to_storage
from oracle import attention_bwd_fp64, attention_kvcache_fp64, attention_varlen_fp64
from tests.gpu_util import DTYPE_NAME, compare, decode, oracle_full, out_to_f64, widest_row_stride
from tests.test_gpu_bwd import check as bwd_check
from tests.test_gpu_bwd import draw as bwd_draw

pytestmark = pytest.mark.gpu

ES = {torch.float16: 2, torch.bfloat16: 2, torch.float8_e4m3fn: 1}


def wide(t, fill=None, dtype=None):
    """A device copy of the CPU tensor t ([B, N, H, D] or [N, H, D]) whose rows sit the widest
    accepted stride apart, as a view of a larger buffer (or, with fill, a view filled with it)."""
    shape = t.shape
    dtype = dtype or t.dtype
    N, H, D = shape[-3], shape[-2], shape[-1]
    B = shape[0] if len(shape) == 4 else 1
    S = widest_row_stride(N, D, ES[dtype])
    assert S >= H * D
    # 300 spare rows per batch: a batch then starts more than 2^31 bytes after the one before
    buf = torch.empty(B, N + 300, S, dtype=dtype, device="cuda")
    assert buf.stride(0) * buf.element_size() > 1 << 31
    v = buf[:, :N, :H * D].view(B, N, H, D)
    if fill is not None:
        v.fill_(fill)
    elif dtype == torch.float8_e4m3fn:
        v.view(torch.uint8).copy_(t.reshape(B, N, H, D).view(torch.uint8).to("cuda"))
    else:
        v.copy_(t.reshape(B, N, H, D).to("cuda"))
    return v if len(shape) == 4 else v[0]


def assert_at_limit(*ts):
    """Each view's head reach under the span rule, ((rows + 256) * row stride + D) bytes, is below
    2^31 by less than one 16-byte unit per row: the widest stride the rule accepts."""
    for t in ts:
        n = t.shape[-3]
        reach = ((n + 256) * t.stride(-3) + t.shape[-1]) * t.element_size()
        assert (1 << 31) - 16 * (n + 256) < reach < 1 << 31, (tuple(t.shape), t.stride(), reach)


FWD = [
    # B, N, Hq, Hkv, D, dtype, causal, window
    (2, 2047, 4, 2, 128, "f16", True, (-1, -1)),     # 8-wave D = 128 shape, batch offsets > 2^31
    (2, 1999, 2, 2, 64, "bf16", False, (-1, -1)),    # two query blocks per wave
    (1, 2047, 4, 1, 128, "bf16", True, (256, 256)),  # few-keys shape, four heads per workgroup
    (2, 2047, 2, 2, 64, "e4m3", True, (-1, -1)),
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: f"b{c[0]}_n{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_{c[5]}_c{int(c[6])}")
def test_forward_widest_spans(case):
    B, N, Hq, Hkv, D, dtype, causal, window = case
    q, k, v = draw_qkv(B, N, N, Hq, Hkv, D, seed=N + D)
    q, k, v, d = to_storage(q, k, v, dtype)
    odt = torch.bfloat16 if dtype in ("bf16", "e4m3") else torch.float16
    qw, kw, vw = wide(q), wide(k), wide(v)
    ow = wide(torch.empty(B, N, Hq, D), fill=float("nan"), dtype=odt)
    assert_at_limit(qw, kw, vw, ow)
    lse = torch.full((B, Hq, N), float("nan"), device="cuda")
    scale = D ** -0.5
    st = fa.fwd_raw(qw, kw, vw, ow, lse, causal, window, scale, d)
    assert st == 0, fa.status_str(st)
    torch.cuda.synchronize()
    out = ow.cpu()
    ro, rl = oracle_full(q, k, v, scale, causal, window, d)
    compare(DTYPE_NAME[q.dtype], out_to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, str(case))


BWD = [
    # B, N, Hq, Hkv, D, dtype, causal
    (2, 1537, 4, 2, 64, torch.float16, True),
    (1, 1023, 2, 1, 128, torch.bfloat16, False),
]


@pytest.mark.parametrize("case", BWD, ids=lambda c: f"b{c[0]}_n{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_{str(c[5])[6:]}")
def test_backward_widest_spans(case):
    B, N, Hq, Hkv, D, dtype, causal = case
    q, k, v, do = bwd_draw(B, N, N, Hq, Hkv, D, dtype, seed=N)
    scale = D ** -0.5
    qw, kw, vw, dow = wide(q), wide(k), wide(v), wide(do)
    ow = wide(q, fill=float("nan"))
    dqw, dkw, dvw = wide(q, fill=float("nan")), wide(k, fill=float("nan")), wide(v, fill=float("nan"))
    assert_at_limit(qw, kw, vw, dow, ow, dqw, dkw, dvw)
    lse = torch.empty(B, Hq, N, device="cuda")
    st = fa.fwd_raw(qw, kw, vw, ow, lse, causal, (-1, -1), scale)
    assert st == 0, fa.status_str(st)
    ws = fa.bwd_workspace(qw, kw)
    st = fa.bwd_raw(qw, kw, vw, ow, dow, lse, dqw, dkw, dvw, ws, causal, (-1, -1), scale)
    assert st == 0, fa.status_str(st)
    torch.cuda.synchronize()
    got = (dqw.cpu(), dkw.cpu(), dvw.cpu())
    ref = attention_bwd_fp64(decode(q), decode(k), decode(v), decode(do), scale, causal, (-1, -1))
    bwd_check(got, ref, dtype, str(case))


def test_varlen_widest_spans():
    lq = [700, 1, 1300]
    q, k, v, cu_q, cu_k, d = make_varlen_inputs(lq, lq, 4, 2, 64, "f16", 11)
    qw, kw, vw = wide(q), wide(k), wide(v)
    ow = wide(q, fill=float("nan"))
    assert_at_limit(qw, kw, vw, ow)
    lse = torch.full((4, q.shape[0]), float("nan"), device="cuda")
    scale = 0.125
    st = fa.fwd_varlen_raw(qw, kw, vw, ow, lse, cu_q.cuda(), cu_k.cuda(), max(lq), True, (-1, -1), scale)
    assert st == 0, fa.status_str(st)
    torch.cuda.synchronize()
    ro, rl = attention_varlen_fp64(decode(q), decode(k), decode(v), cu_q.numpy(), cu_k.numpy(), scale, True,
                                   (-1, -1))
    compare("f16", out_to_f64(ow.cpu()), lse.cpu().numpy().astype(np.float64), ro, rl, "varlen widest spans")


def test_kvcache_pages_past_4_gib():
    # a paged cache of about 4.3 GB per tensor whose used pages sit at its top: page byte offsets
    # above 2^32 (the decode kernel forms each key's address in 64 bits)
    B, Nq, Hq, Hkv, D, lens, P = 3, 2, 8, 2, 128, [1000, 4100, 17], 16
    q, k, v, seqlens, table = make_kvcache_inputs(B, Nq, Hq, Hkv, D, "bf16", lens, P, seed=5)
    base = (1 << 32) // (P * Hkv * D * 2) + 1000
    kc = torch.empty(base + k.shape[0], P, Hkv, D, dtype=k.dtype, device="cuda")
    vc = torch.empty_like(kc)
    kc[base:] = k.cuda()
    vc[base:] = v.cuda()
    scale = D ** -0.5
    out, lse = fa.fwd_kvcache(q.cuda(), kc, vc, seqlens.cuda(), (table + base).to(torch.int32).cuda(), max(lens),
                              True, (-1, -1), scale)
    torch.cuda.synchronize()
    ro, rl = attention_kvcache_fp64(decode(q), decode(k), decode(v), lens, table.numpy(), P, scale, True, (-1, -1))
    compare("bf16", out_to_f64(out.cpu()), lse.cpu().numpy().astype(np.float64), ro, rl, "paged cache past 4 GiB")


def test_kvcache_dense_batches_past_2_gib():
    # a dense cache whose second sequence starts more than 2^31 bytes after the first
    B, Nq, Hq, Hkv, D, lens = 2, 3, 8, 2, 128, [3000, 2500]
    q, k, v, seqlens, _ = make_kvcache_inputs(B, Nq, Hq, Hkv, D, "f16", lens, 0, seed=6)
    rows = (1 << 31) // (Hkv * D * 2) + 64
    kc = torch.empty(B, rows, Hkv, D, dtype=k.dtype, device="cuda")
    vc = torch.empty_like(kc)
    kc[:, :k.shape[1]] = k.cuda()
    vc[:, :v.shape[1]] = v.cuda()
    assert kc.stride(0) * kc.element_size() > 1 << 31
    scale = D ** -0.5
    out, lse = fa.fwd_kvcache(q.cuda(), kc, vc, seqlens.cuda(), None, max(lens), True, (-1, -1), scale)
    torch.cuda.synchronize()
    ro, rl = attention_kvcache_fp64(decode(q), decode(k), decode(v), lens, None, 0, scale, True, (-1, -1))
    compare("f16", out_to_f64(out.cpu()), lse.cpu().numpy().astype(np.float64), ro, rl, "dense cache past 2 GiB")
