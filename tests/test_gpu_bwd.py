"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the fp64 gradient oracle.

Bars (the pages give none for the backward pass; derived from the arithmetic): the
kernels round P and dS to the storage type for their products and round dq, dk, dv once on
output, so each gradient is within a few units of that type's rounding of its own scale. With
u = 2^-11 (fp16) or 2^-8 (bf16), per tensor:
    max |err| <= 4 u * max |ref| + 1e-5        and        RMS(err) <= 2 u * RMS(ref) + 1e-5,
no NaN or Inf, and results bitwise identical between runs (no atomics). The 1e-5 floors cover
gradients that vanish by cancellation (one key: dk = 0; a (0, 0) window: dq = dk = 0), where
the kernel leaves rounding noise of the order of 1e-6. Measured on MI355X the
worst cases use about 1.2 u (max) and 0.7 u (RMS).
The forward pass that feeds the backward (out, lse) is the library's own, as a caller would run.
"""
import numpy as np
import pytest
import torch

import exact_attention_09_amd as fa
from oracle import attention_bwd_fp64
from tests.gpu_util import decode

pytestmark = pytest.mark.gpu

U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def draw(B, Nq, Nk, Hq, Hkv, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Nq, Hq, D, generator=g).to(dtype)
    k = torch.randn(B, Nk, Hkv, D, generator=g).to(dtype)
    v = torch.randn(B, Nk, Hkv, D, generator=g).to(dtype)
    do = torch.randn(B, Nq, Hq, D, generator=g).to(dtype)
    return q, k, v, do


def gpu_grads(q, k, v, do, causal, window, scale):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = fa.fwd(qd, kd, vd, causal=causal, window=window, softmax_scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, out, dod, lse, causal=causal, window=window, softmax_scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(got, ref, dtype, what):
    u = U[dtype]
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        gv = decode(g)
        assert np.isfinite(gv).all(), f"{what} {name}: non-finite"
        err = np.abs(gv - r)
        amax = np.abs(r).max()
        assert err.max() <= 4 * u * amax + 1e-5, f"{what} {name}: max err {err.max():.3g} vs max|ref| {amax:.3g}"
        rms_e, rms_r = np.sqrt((err ** 2).mean()), np.sqrt((r ** 2).mean())
        assert rms_e <= 2 * u * rms_r + 1e-5, f"{what} {name}: RMS err {rms_e:.3g} vs RMS ref {rms_r:.3g}"


CASES = [
    # B, Nq, Nk, Hq, Hkv, D, causal, window
    (1, 128, 128, 2, 2, 64, False, (-1, -1)),
    (1, 128, 128, 2, 2, 64, True, (-1, -1)),
    (2, 200, 333, 4, 2, 128, False, (-1, -1)),
    (1, 333, 200, 4, 1, 64, True, (-1, -1)),        # Nq > Nk: the first 133 rows admit no key
    (1, 300, 300, 4, 2, 128, True, (37, 11)),
    (1, 257, 257, 2, 2, 64, False, (0, 0)),          # out = v: dv = dout, dq = dk = 0
    (2, 129, 65, 4, 4, 64, False, (-1, 5)),
    (1, 1, 513, 2, 1, 128, True, (-1, -1)),
    (1, 513, 1, 2, 2, 64, False, (-1, -1)),
    (3, 190, 190, 6, 3, 128, True, (64, -1)),
    (1, 640, 640, 2, 1, 64, False, (100, 100)),
    (1, 1024, 1024, 8, 2, 64, True, (-1, -1)),
]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(x) for x in c[:6]) + f"-c{int(c[6])}-w{c[7][0]}_{c[7][1]}")
def test_bwd_matches_oracle(case, dtype):
    B, Nq, Nk, Hq, Hkv, D, causal, window = case
    q, k, v, do = draw(B, Nq, Nk, Hq, Hkv, D, dtype, seed=Nq + 7 * Nk + D)
    scale = D ** -0.5
    got = gpu_grads(q, k, v, do, causal, window, scale)
    ref = attention_bwd_fp64(decode(q), decode(k), decode(v), decode(do), scale, causal, window)
    check(got, ref, dtype, f"{case}")


def test_bwd_deterministic():
    q, k, v, do = draw(2, 384, 384, 8, 2, 128, torch.bfloat16, seed=3)
    a = gpu_grads(q, k, v, do, True, (-1, -1), 0.1)
    b = gpu_grads(q, k, v, do, True, (-1, -1), 0.1)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_strided_views():
    """Non-contiguous q / dout views ([B, H, N, D] storage seen as [B, N, H, D]) give the same result."""
    B, N, H, D = 1, 256, 4, 64
    q, k, v, do = draw(B, N, N, H, H, D, torch.float16, seed=5)
    qs = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    dos = do.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert not qs.is_contiguous()
    a = gpu_grads(q, k, v, do, True, (-1, -1), 0.125)
    b = gpu_grads(qs, k, v, dos, True, (-1, -1), 0.125)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_c3_shape_sampled_head():
    """The benchmark's causal [4, 4096, 32, 64] fp16 shape; one (batch, head) checked in full."""
    B, N, H, D = 4, 4096, 32, 64
    q, k, v, do = draw(B, N, N, H, H, D, torch.float16, seed=0)
    got = gpu_grads(q, k, v, do, True, (-1, -1), 0.125)
    b, h = 2, 17
    sl = lambda t: t[b:b + 1, :, h:h + 1, :]
    ref = attention_bwd_fp64(decode(sl(q)), decode(sl(k)), decode(sl(v)), decode(sl(do)), 0.125, True, (-1, -1))
    check(tuple(sl(t) for t in got), ref, torch.float16, "c3 head (2, 17)")


@pytest.mark.parametrize("wl", ["causal_b4_h32_n4096_d64_f16", "gqa_b1_hq32_hkv8_n16384_d128_bf16",
                                "mqa_b1_hq32_hkv1_n16384_d128_bf16"])
def test_bwd_benchmark_shape_tail(wl):
    """The benchmark's shapes and launch (the MQA one splits each K/V head's query heads over 16
    workgroups and adds the partial sums). Under the causal mask the last T keys receive
    gradient only from the last T query rows, so the oracle run on those rows alone (all keys,
    bottom-right alignment keeps every row's mask) gives exact dq for those rows and exact dk, dv
    for those keys."""
    from exact_attention_09_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS[wl]
    assert w.causal and w.window == (-1, -1) and w.Nq == w.Nk
    q, k, v, _ = make_inputs(w, 0)
    g = torch.Generator().manual_seed(1)
    do = torch.randn(w.B, w.Nq, w.Hq, w.D, generator=g).to(q.dtype)
    scale = w.softmax_scale()
    got = gpu_grads(q, k, v, do, True, (-1, -1), scale)
    T = 64
    ref = attention_bwd_fp64(decode(q[:, -T:]), decode(k), decode(v), decode(do[:, -T:]), scale, True, (-1, -1))
    check((got[0][:, -T:], got[1][:, -T:], got[2][:, -T:]), (ref[0], ref[1][:, -T:], ref[2][:, -T:]), q.dtype, wl)


NAN_TAIL = [
    # B, Nq, Nk, Hq, Hkv, D, causal, window: query and key counts off the tile grids
    (1, 200, 333, 4, 2, 64, False, (-1, -1)),
    (2, 150, 290, 4, 1, 128, True, (-1, -1)),
    (1, 333, 200, 2, 2, 64, True, (-1, -1)),
    (1, 100, 100, 8, 1, 64, True, (-1, -1)),      # MQA: the query heads are split over workgroups
]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("case", NAN_TAIL, ids=lambda c: "x".join(str(x) for x in c[:6]) + f"-c{int(c[6])}")
def test_bwd_rows_past_the_end_are_not_read(case, dtype):
    """q, k, v, out and dout are the first N rows of larger tensors whose remaining rows are NaN:
    the last query and key tiles reach past N and must read zeros there (buffer range check)."""
    from tests.gpu_util import nan_tailed
    B, Nq, Nk, Hq, Hkv, D, causal, window = case
    q, k, v, do = draw(B, Nq, Nk, Hq, Hkv, D, dtype, seed=Nq + 5 * Nk)
    scale = D ** -0.5
    qd, kd, vd, dod = nan_tailed(q), nan_tailed(k), nan_tailed(v), nan_tailed(do)
    out, lse = fa.fwd(qd, kd, vd, causal=causal, window=window, softmax_scale=scale)
    outd = nan_tailed(out)
    dq, dk, dv = fa.bwd(qd, kd, vd, outd, dod, lse, causal=causal, window=window, softmax_scale=scale)
    torch.cuda.synchronize()
    ref = attention_bwd_fp64(decode(q), decode(k), decode(v), decode(do), scale, causal, window)
    check((dq.cpu(), dk.cpu(), dv.cpu()), ref, dtype, f"nan tail {case}")


@pytest.mark.parametrize("case", [(1, 333, 200, 4, 1, 64, True), (2, 190, 190, 8, 2, 128, True),
                                  (1, 256, 256, 16, 1, 64, False), (1, 513, 513, 4, 4, 64, False)],
                         ids=lambda c: "x".join(str(x) for x in c[:6]) + f"-c{int(c[6])}")
def test_bwd_workspace_contents_do_not_matter(case):
    """fa_bwd's workspace holds the per-row terms the dq kernel writes and dk/dv reads (and, for
    split query heads, the partial sums): filled with NaN and with zeros beforehand, and with dq,
    dk, dv filled with NaN, the results are the same bit for bit."""
    B, Nq, Nk, Hq, Hkv, D, causal = case
    q, k, v, do = draw(B, Nq, Nk, Hq, Hkv, D, torch.float16, seed=Nq + Nk)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = fa.fwd(qd, kd, vd, causal=causal)
    res = []
    for fill in (float("nan"), 0.0):
        ws = fa.bwd_workspace(qd, kd)
        ws.fill_(fill)
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qd, kd, vd))
        assert fa.bwd_raw(qd, kd, vd, out, dod, lse, dq, dk, dv, ws, causal=causal) == 0
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (dq, dk, dv)])
    for a, b in zip(*res):
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bwd_c3_every_head_equals_single_head_launches():
    """Every element of the causal [4, 4096, 32, 64] fp16 backward: the full launch (its launch
    order, chunked by heads over the XCDs) against 128 launches of one (batch, head) each, which
    take the single-head order. Each workgroup's arithmetic does not depend on where the launch
    order puts it (no atomics, no split at Hq = Hkv), so the two must agree bit for bit; a tile
    that the full order skipped or computed twice would not. Single-head launches are held to the
    oracle by the other tests (one c3 head above in full)."""
    B, N, H, D = 4, 4096, 32, 64
    q, k, v, do = draw(B, N, N, H, H, D, torch.float16, seed=3)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = fa.fwd(qd, kd, vd, causal=True)
    full = [torch.full_like(qd, float("nan")) for _ in range(3)]
    st = fa.bwd_raw(qd, kd, vd, out, dod, lse, *full, fa.bwd_workspace(qd, kd), causal=True)
    assert st == 0, fa.status_str(st)
    ws1 = fa.bwd_workspace(qd[:1, :, :1], kd[:1, :, :1])
    sl = lambda t, b, h: t[b:b + 1, :, h:h + 1, :]
    one = [torch.empty(1, N, 1, D, dtype=torch.float16, device="cuda") for _ in range(3)]
    for b in range(B):
        for h in range(H):
            for t in one:
                t.fill_(float("nan"))
            st = fa.bwd_raw(sl(qd, b, h), sl(kd, b, h), sl(vd, b, h), sl(out, b, h), sl(dod, b, h),
                            lse[b:b + 1, h:h + 1], *one, ws1, causal=True)
            assert st == 0, fa.status_str(st)
            for name, f, o in zip(("dq", "dk", "dv"), full, one):
                assert torch.equal(sl(f, b, h).view(torch.int16), o.view(torch.int16)), f"{name} of ({b}, {h})"
