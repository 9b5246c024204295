"""fa_fwd_kvcache_noalloc (the KV-cache entry point that allocates nothing: its split partials go
to the library's fixed per-device scratch) against fa_fwd_kvcache with a caller-allocated
workspace, through the C ABI: bitwise equal outputs and lse on two calls in a row, the second
with smaller sizes than the first (so the scratch holds the first call's larger partials when the
second runs), each also held to the KV-cache oracle's bars."""
import numpy as np
import pytest
import torch

import exact_attention_09_amd as fa
from exact_attention_09_amd.inputs import make_kvcache_inputs
from oracle import attention_kvcache_fp64
from tests.gpu_util import compare, decode, out_to_f64

pytestmark = pytest.mark.gpu

CALLS = [
    # B, Nq, Hq, Hkv, D, lengths, page_size, causal, dtype: the second is smaller than the first
    (3, 2, 8, 2, 128, [5000, 700, 9000], 16, True, "bf16"),
    (2, 1, 4, 1, 64, [3000, 100], 0, False, "f16"),
]


def _one(case, noalloc):
    B, Nq, Hq, Hkv, D, lens, P, causal, dtype = case
    q, k, v, seqlens, table = make_kvcache_inputs(B, Nq, Hq, Hkv, D, dtype, lens, P, seed=sum(lens) + Nq)
    max_k = max(lens)
    dev = torch.device("cuda")
    qd, kd, vd, sd = q.to(dev), k.to(dev), v.to(dev), seqlens.to(dev)
    td = table.to(dev) if table is not None else None
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), device=dev)
    ws = None if noalloc else fa.kvcache_workspace(qd, Hkv, max_k)
    st = fa.fwd_kvcache_raw(qd, kd, vd, out, lse, sd, td, max_k, causal=causal, softmax_scale=D ** -0.5,
                            workspace=ws, noalloc=noalloc)
    assert st == 0, fa.status_str(st)
    torch.cuda.synchronize()
    return (q, k, v, table), out.cpu(), lse.cpu()


def test_noalloc_matches_workspace_entry_point_twice():
    for case in CALLS:
        B, Nq, Hq, Hkv, D, lens, P, causal, dtype = case
        # the keys are split, so the partials really go through the scratch
        need = fa.load().fa_fwd_kvcache_workspace_bytes(B, Nq, Hq, Hkv, D, max(lens))
        assert 0 < need <= fa.NOALLOC_SCRATCH_BYTES
        (q, k, v, table), out_ref, lse_ref = _one(case, noalloc=False)
        _, out, lse = _one(case, noalloc=True)
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), f"{case}: out differs"
        assert torch.equal(lse, lse_ref), f"{case}: lse differs"
        ro, rl = attention_kvcache_fp64(decode(q), decode(k), decode(v), lens,
                                        table.numpy() if table is not None else None, P, D ** -0.5, causal, (-1, -1))
        compare(dtype, out_to_f64(out), lse.numpy().astype(np.float64), ro, rl, f"noalloc {case}")
