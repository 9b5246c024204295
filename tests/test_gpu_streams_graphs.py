"""Stream semantics of the C ABI, through the Python binding on the GPU.

The header promises that every entry point is asynchronous on the caller's stream, reentrant and
allocation-free (fa_fwd, fa_fwd_varlen, fa_bwd, fa_fwd_kvcache_noalloc), so that the calls can be
recorded into a HIP graph. These tests hold the library to that:
  * a call on a side stream gives the same bits as on the default stream;
  * two host threads, each driving its own stream with its own tensors, get the bits a serial run
    gets (ctypes drops the GIL during the call, so the calls really overlap);
  * a HIP graph that records fa_fwd (fp16, bf16 GQA with a window, e4m3), fa_bwd and
    fa_fwd_kvcache_noalloc is replayed several times with new inputs copied into its static
    tensors between replays (eager work and a synchronisation between replays), and every replay
    equals an eager call on the same inputs bit for bit. The first replay of each graph is also
    held to the oracle's bars.
"""
import threading

import numpy as np
import pytest
import torch

import exact_attention_09_amd as fa
from exact_attention_09_amd.inputs import draw_qkv, make_kvcache_inputs, to_storage
from oracle import attention_kvcache_fp64
from tests.gpu_util import compare, decode, oracle_full, out_to_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
OUT_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.bfloat16}

# B, N, Hq, Hkv, D, causal, window, dtype
FWD_CASES = [
    (2, 777, 4, 4, 64, True, (-1, -1), "f16"),
    (1, 1500, 8, 2, 128, True, (256, 256), "bf16"),
    (2, 640, 4, 4, 64, True, (-1, -1), "e4m3"),
]


def _inputs(case, seed):
    B, N, Hq, Hkv, D, causal, window, dtype = case
    q, k, v = draw_qkv(B, N, N, Hq, Hkv, D, seed)
    return to_storage(q, k, v, dtype)


def _fwd(qd, kd, vd, case, descale, out=None, lse=None):
    B, N, Hq, Hkv, D, causal, window, dtype = case
    if out is None:
        out = torch.full((B, N, Hq, D), float("nan"), dtype=OUT_DTYPE[dtype], device=DEV)
        lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=DEV)
    st = fa.fwd_raw(qd, kd, vd, out, lse, causal, window, D ** -0.5, descale)
    assert st == 0, fa.status_str(st)
    return out, lse


@pytest.mark.parametrize("case", FWD_CASES[:2], ids=lambda c: f"{c[7]}-d{c[4]}")
def test_side_stream_same_bits(case):
    q, k, v, desc = _inputs(case, 3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o0, l0 = _fwd(qd, kd, vd, case, desc)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o1, l1 = _fwd(qd, kd, vd, case, desc)
    s.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)


def test_two_threads_two_streams():
    cases = [FWD_CASES[0], FWD_CASES[1]]
    data = []
    for i, c in enumerate(cases):
        q, k, v, desc = _inputs(c, 10 + i)
        data.append((c, q.to(DEV), k.to(DEV), v.to(DEV), desc))
    refs = []
    for c, qd, kd, vd, desc in data:
        o, l = _fwd(qd, kd, vd, c, desc)
        refs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    results = [None, None]
    errors = []

    def worker(i):
        try:
            c, qd, kd, vd, desc = data[i]
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                for _ in range(12):
                    outs.append(_fwd(qd, kd, vd, c, desc))
            s.synchronize()
            results[i] = outs
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    for i in range(2):
        for o, l in results[i]:
            assert torch.equal(o, refs[i][0]) and torch.equal(l, refs[i][1])


def _capture(fn):
    """Warm fn up on a side stream, then record it into a CUDA/HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: f"{c[7]}-d{c[4]}-w{c[6][0]}")
def test_graph_replays_fwd(case):
    B, N, Hq, Hkv, D, causal, window, dtype = case
    q, k, v, desc = _inputs(case, 20)
    sq, sk, sv = q.to(DEV), k.to(DEV), v.to(DEV)       # the graph's static inputs
    out = torch.full((B, N, Hq, D), float("nan"), dtype=OUT_DTYPE[dtype], device=DEV)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=DEV)
    g = _capture(lambda: _fwd(sq, sk, sv, case, desc, out, lse))
    for rep, seed in enumerate((21, 22, 23, 24)):
        nq, nk, nv, _ = _inputs(case, seed)               # new inputs; e4m3 keeps the captured descales
        sq.copy_(nq.to(DEV))
        sk.copy_(nk.to(DEV))
        sv.copy_(nv.to(DEV))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo, el = _fwd(sq, sk, sv, case, desc)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eo.view(torch.int16)) and torch.equal(lse, el), f"replay {rep} differs from the eager call"
        if rep == 0:
            ro, rl = oracle_full(nq, nk, nv, D ** -0.5, causal, window, desc)
            compare(dtype, out_to_f64(out.cpu()), lse.cpu().numpy().astype(np.float64), ro, rl, f"graph {dtype}")


def test_graph_replays_bwd():
    B, N, Hq, Hkv, D = 2, 900, 4, 2, 64
    q, k, v = draw_qkv(B, N, N, Hq, Hkv, D, 30)
    q, k, v, _ = to_storage(q, k, v, "f16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = fa.fwd(qd, kd, vd, causal=True)
    dout = torch.empty_like(qd)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = fa.bwd_workspace(qd, kd)

    def call(dq_, dk_, dv_):
        st = fa.bwd_raw(qd, kd, vd, out, dout, lse, dq_, dk_, dv_, ws, causal=True)
        assert st == 0, fa.status_str(st)

    gen = torch.Generator().manual_seed(31)
    dout.copy_(torch.randn(B, N, Hq, D, generator=gen).half().to(DEV))
    g = _capture(lambda: call(dq, dk, dv))
    for rep in range(4):
        dout.copy_(torch.randn(B, N, Hq, D, generator=gen).half().to(DEV))
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eq, ek, ev = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
        call(eq, ek, ev)
        torch.cuda.synchronize()
        assert torch.equal(dq, eq) and torch.equal(dk, ek) and torch.equal(dv, ev), f"replay {rep} differs"


def test_graph_replays_kvcache_noalloc():
    B, Nq, Hq, Hkv, D, lens, P = 3, 2, 8, 2, 128, [4000, 900, 6100], 16
    q, k, v, seqlens, table = make_kvcache_inputs(B, Nq, Hq, Hkv, D, "bf16", lens, P, seed=40)
    max_k = max(lens)
    sq, kd, vd, sd, td = q.to(DEV), k.to(DEV), v.to(DEV), seqlens.to(DEV), table.to(DEV)
    out = torch.full_like(sq, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), device=DEV)

    def call(q_, out_, lse_, noalloc, ws=None):
        st = fa.fwd_kvcache_raw(q_, kd, vd, out_, lse_, sd, td, max_k, causal=True, softmax_scale=D ** -0.5,
                                workspace=ws, noalloc=noalloc)
        assert st == 0, fa.status_str(st)

    g = _capture(lambda: call(sq, out, lse, True))
    ws = fa.kvcache_workspace(sq, Hkv, max_k)
    gen = torch.Generator().manual_seed(41)
    for rep in range(4):
        nq = torch.randn(B, Nq, Hq, D, generator=gen).bfloat16()
        sq.copy_(nq.to(DEV))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo = torch.full_like(sq, float("nan"))
        el = torch.full((B, Hq, Nq), float("nan"), device=DEV)
        call(sq, eo, el, False, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(lse, el), f"replay {rep} differs from the workspace entry point"
        if rep == 0:
            ro, rl = attention_kvcache_fp64(decode(nq), decode(k), decode(v), lens, table.numpy(), P, D ** -0.5,
                                            True, (-1, -1))
            compare("bf16", out_to_f64(out.cpu()), lse.cpu().numpy().astype(np.float64), ro, rl, "graph kvcache")
