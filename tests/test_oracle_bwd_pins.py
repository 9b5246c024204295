"""Pins of the fp64 backward oracle (``oracle.backward``) to facts outside its own code (CPU only).

  * an independent library routine: PyTorch's CPU fp64 autograd through
    scaled_dot_product_attention, with K/V heads repeat-interleaved inside the graph (so the
    gradients of shared K/V heads are summed by autograd itself) and masks from torch.tril/triu;
  * central finite differences of the forward oracle (itself pinned in test_oracle_pins.py) along
    random directions: <grad, u> = d/dt sum(dout * out(x + t u)) at t = 0;
  * closed forms: every query row's softmax sums to 1, so the rows of dv add up to the rows of
    dout; the scores of a row shift together when every key moves by the same vector, so the rows
    of dk add up to 0; a (0, 0) window makes out = v, so dv = dout (summed over query heads),
    dq = 0 and dk = 0; a query row with no admitted key has dq = 0.

The mutation tests plant plausible mistakes (a dropped rowsum term in the softmax Jacobian, a
missing scale, the wrong operand order, dk/dv of a shared K/V head overwritten instead of summed,
p not normalised) and check that at least one pin fails for each.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.backward as OB
from oracle import attention_bwd_fp64, attention_fp64


def rand_inputs(seed, B, Nq, Nk, Hq, Hkv, D):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Nq, Hq, D))
    k = g.standard_normal((B, Nk, Hkv, D))
    v = g.standard_normal((B, Nk, Hkv, D))
    do = g.standard_normal((B, Nq, Hq, D))
    return q, k, v, do


def torch_mask(Nq, Nk, causal, wl, wr):
    off = Nk - Nq
    ones = torch.ones(Nq, Nk, dtype=torch.bool)
    m = ones.clone()
    if causal:
        m &= ones.tril(diagonal=off)
    if wl >= 0:
        m &= ones.triu(diagonal=off - wl)
    if wr >= 0:
        m &= ones.tril(diagonal=off + wr)
    return m


def torch_grads(q, k, v, do, scale, causal, window):
    """Gradients by autograd of torch's fp64 SDPA (rows with no admitted key are given zero grads)."""
    B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qt = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kt = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    vt = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    mask = torch_mask(Nq, Nk, causal, window[0], window[1])
    live = mask.any(dim=1)
    # rows with no admitted key: let them see key 0 and zero their upstream gradient instead
    mask_safe = mask.clone()
    mask_safe[~live, 0] = True
    kk = kt.repeat_interleave(G, dim=1)
    vv = vt.repeat_interleave(G, dim=1)
    out = F.scaled_dot_product_attention(qt, kk, vv, attn_mask=mask_safe, scale=scale)
    dot = torch.tensor(do).permute(0, 2, 1, 3).contiguous() * live[None, None, :, None]
    out.backward(dot)
    return (qt.grad.permute(0, 2, 1, 3).numpy(), kt.grad.permute(0, 2, 1, 3).numpy(),
            vt.grad.permute(0, 2, 1, 3).numpy())


CASES = [
    # B, Nq, Nk, Hq, Hkv, D, causal, window
    (1, 9, 9, 2, 2, 8, False, (-1, -1)),
    (2, 12, 12, 4, 2, 16, True, (-1, -1)),
    (1, 10, 16, 3, 1, 8, True, (-1, -1)),       # Nq < Nk, bottom-right causal, MQA
    (1, 16, 10, 2, 1, 8, True, (-1, -1)),       # Nq > Nk: the first 6 rows admit no key
    (1, 20, 20, 4, 2, 8, False, (3, 2)),
    (1, 20, 20, 2, 2, 8, True, (4, -1)),
    (1, 7, 7, 4, 1, 4, False, (0, 0)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}-w{c[7][0]}_{c[7][1]}")
def test_bwd_matches_autograd(case):
    B, Nq, Nk, Hq, Hkv, D, causal, window = case
    q, k, v, do = rand_inputs(3, B, Nq, Nk, Hq, Hkv, D)
    scale = 0.37
    got = attention_bwd_fp64(q, k, v, do, scale, causal, window)
    ref = torch_grads(q, k, v, do, scale, causal, window)
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.allclose(a, r, rtol=1e-10, atol=1e-11), f"{name}: max err {np.abs(a - r).max()}"


def _loss(q, k, v, do, scale, causal, window):
    out, _ = attention_fp64(q, k, v, scale, causal, window)
    return float((out * do).sum())


@pytest.mark.parametrize("case", [(1, 6, 6, 2, 1, 4, True, (-1, -1)), (1, 5, 7, 2, 2, 3, False, (2, 1))])
def test_bwd_finite_differences(case):
    B, Nq, Nk, Hq, Hkv, D, causal, window = case
    q, k, v, do = rand_inputs(11, B, Nq, Nk, Hq, Hkv, D)
    scale = 0.5
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, scale, causal, window)
    g = np.random.default_rng(5)
    eps = 1e-5
    for which in range(3):
        for _ in range(3):
            u = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
            u[which] = g.standard_normal(u[which].shape)
            xp = [x + eps * d for x, d in zip((q, k, v), u)]
            xm = [x - eps * d for x, d in zip((q, k, v), u)]
            fd = (_loss(*xp, do, scale, causal, window) - _loss(*xm, do, scale, causal, window)) / (2 * eps)
            an = float((dq * u[0]).sum() + (dk * u[1]).sum() + (dv * u[2]).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_bwd_row_sums():
    """Softmax rows sum to 1 and shift together: sum_j dv_j = sum_i dout_i, sum_j dk_j = 0."""
    B, Nq, Nk, Hq, Hkv, D = 2, 24, 24, 4, 2, 8
    q, k, v, do = rand_inputs(7, B, Nq, Nk, Hq, Hkv, D)
    for causal, window in ((False, (-1, -1)), (True, (-1, -1)), (False, (5, 3))):
        dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.3, causal, window)
        G = Hq // Hkv
        for b in range(B):
            for g in range(Hkv):
                dsum = do[b, :, g * G:(g + 1) * G, :].sum(axis=(0, 1))
                assert np.allclose(dv[b, :, g, :].sum(axis=0), dsum, atol=1e-11)
                assert np.allclose(dk[b, :, g, :].sum(axis=0), 0.0, atol=1e-11)


def test_bwd_window_zero_is_identity():
    """A (0, 0) window admits only key i for query i: out = v, so dv = dout, dq = dk = 0."""
    B, N, Hq, Hkv, D = 1, 11, 4, 2, 8
    q, k, v, do = rand_inputs(9, B, N, N, Hq, Hkv, D)
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.7, False, (0, 0))
    G = Hq // Hkv
    for g in range(Hkv):
        assert np.allclose(dv[:, :, g, :], do[:, :, g * G:(g + 1) * G, :].sum(axis=2), atol=1e-13)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_bwd_empty_rows_have_no_gradient():
    B, Nq, Nk, Hq, Hkv, D = 1, 12, 5, 2, 1, 4
    q, k, v, do = rand_inputs(2, B, Nq, Nk, Hq, Hkv, D)
    dq, _, _ = attention_bwd_fp64(q, k, v, do, 0.5, True, (-1, -1))
    assert np.abs(dq[:, :Nq - Nk]).max() == 0.0
    assert np.abs(dq[:, Nq - Nk:]).max() > 0.0


# ----------------------------------------------------------------------------------------------
# planted mistakes: each must make at least one pin above fail
# ----------------------------------------------------------------------------------------------
def _mut_no_rowsum(qh, kh, vh, doh, scale, mask):
    s = np.where(mask, scale * (qh @ kh.T), -np.inf)
    m = np.where(np.isfinite(s.max(axis=1)), s.max(axis=1), 0.0)
    e = np.where(mask, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=l[:, None] > 0)
    ds = p * (doh @ vh.T)                                   # rowsum term dropped
    return scale * ds @ kh, scale * ds.T @ qh, p.T @ doh


def _mut_no_scale(qh, kh, vh, doh, scale, mask):
    dq, dk, dv = _REAL(qh, kh, vh, doh, scale, mask)
    return dq, dk / scale, dv


def _mut_operand_order(qh, kh, vh, doh, scale, mask):
    dq, dk, dv = _REAL(qh, kh, vh, doh, scale, mask)
    s = np.where(mask, scale * (qh @ kh.T), -np.inf)
    m = np.where(np.isfinite(s.max(axis=1)), s.max(axis=1), 0.0)
    e = np.where(mask, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=l[:, None] > 0)
    return dq, dk, p.T @ (doh @ vh.T @ vh) / max(1.0, np.abs(vh).max())   # wrong product for dv


def _mut_unnormalised(qh, kh, vh, doh, scale, mask):
    dq, dk, dv = _REAL(qh, kh, vh, doh, scale, mask)
    return dq, dk, dv * 1.5


_REAL = OB._one_head_bwd


@pytest.mark.parametrize("mutant", [_mut_no_rowsum, _mut_no_scale, _mut_operand_order, _mut_unnormalised])
def test_bwd_pins_catch_mutants(monkeypatch, mutant):
    monkeypatch.setattr(OB, "_one_head_bwd", mutant)
    failures = 0
    for fn in (lambda: test_bwd_matches_autograd(CASES[1]), test_bwd_row_sums, test_bwd_window_zero_is_identity):
        try:
            fn()
        except AssertionError:
            failures += 1
    assert failures >= 1


def test_bwd_pins_catch_overwritten_group_sum(monkeypatch):
    """dk/dv of a shared K/V head assigned per query head instead of summed."""
    real = OB.attention_bwd_fp64

    def mutant(q, k, v, dout, scale=None, causal=False, window=(-1, -1), row_chunk=1024):
        B, Nq, Hq, D = q.shape
        Hkv = k.shape[2]
        dq, dk, dv = real(q, k, v, dout, scale, causal, window, row_chunk)
        # keep only the last query head's share of each K/V head
        G = Hq // Hkv
        last = real(q, k, v, dout * (np.arange(Hq) % G == G - 1)[None, None, :, None], scale, causal, window)
        return dq, last[1], last[2]

    monkeypatch.setattr(OB, "attention_bwd_fp64", mutant)
    monkeypatch.setitem(globals(), "attention_bwd_fp64", mutant)
    with pytest.raises(AssertionError):
        test_bwd_matches_autograd(CASES[1])
