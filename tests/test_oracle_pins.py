"""Pins of the CPU fp64 oracle to facts that do not come from the oracle itself (CPU only).

Each pin checks the oracle against something independent of its own code:
  * an independent library routine: PyTorch's CPU fp64 scaled_dot_product_attention and logsumexp,
    with masks built from torch.tril / torch.triu and K/V heads repeat-interleaved;
  * brute force in 40-digit arithmetic (mpmath) on tiny inputs;
  * the pages' worked example: the 8-token grid in 2x2 blocks ("What FlashAttention is and how it
    speeds up attention", section 2), where the blocked traversal with running max / running sum
    must reproduce the full softmax (section 3: the blocked result equals full attention);
  * closed forms and invariants: a constant added to a score row changes nothing but the lse;
    under a causal mask query row 0 sees only key 0; identical keys give the mean of the admitted
    values; a (0, 0) window returns V; windows wider than the sequence change nothing;
  * mask probe: with Q = 0 every admitted key gets the same weight, so exp(lse) counts the keys;
  * format decoders checked against torch's own fp16 / bf16 / float8_e4m3fn conversions.

The mutation tests at the end plant plausible mistakes in the oracle (a wrong GQA mapping, a
causal off-by-one, swapped window sides, a dropped scale, an lse without the max, the wrong tensor
as V, softmax over the wrong axis, a missing rescale, a wrong exponent bias) and check that at
least one pin fails for each.
"""
import math
import sys

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as OA
import oracle.formats as OF
from oracle import admitted, attention_fp64, decode_bf16_bits, decode_e4m3_codes, decode_f16_bits, tiled_online_fp64


def nanmax(*xs):
    """max that keeps a NaN (Python's max drops one that is not its first argument), so a pin
    whose oracle result turns NaN fails instead of passing."""
    return float(np.max(np.array(xs, dtype=np.float64)))


GOLDEN_GRID = __file__.rsplit("/", 1)[0] + "/golden/grid_8x8_2x2.txt"


# ----------------------------------------------------------------------------------------------
# helpers independent of the oracle
# ----------------------------------------------------------------------------------------------
def rand_qkv(seed, B, Nq, Nk, Hq, Hkv, D):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Nq, Hq, D))
    k = g.standard_normal((B, Nk, Hkv, D))
    v = g.standard_normal((B, Nk, Hkv, D))
    return q, k, v


def torch_mask(Nq, Nk, causal, wl, wr):
    """Admission mask from torch.tril/triu (bottom-right alignment, inclusive window bounds)."""
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


def sdpa_reference(q, k, v, scale, causal, window):
    """CPU fp64 torch SDPA + logsumexp on the [B, H, N, D] transpose, K/V repeat-interleaved."""
    B, Nq, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()
    kt = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
    mask = torch_mask(Nq, k.shape[1], causal, *window)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


def read_grid(path=GOLDEN_GRID):
    meta, grid, inside = {}, [], False
    with open(path) as f:
        lines = f.read().splitlines()
    for line in lines:
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line == "grid":
            inside = True
            continue
        if line == "end":
            inside = False
            continue
        if inside:
            grid.append(line)
        else:
            key, val = line.split()
            meta[key] = int(val)
    return meta, grid


# ----------------------------------------------------------------------------------------------
# pins: each returns the worst error found (0 = exact); thresholds are in PIN_TOL
# ----------------------------------------------------------------------------------------------
SDPA_CASES = [
    # B, Nq, Nk, Hq, Hkv, D, causal, window, seed
    (2, 16, 16, 4, 4, 8, False, (-1, -1), 0),
    (2, 16, 16, 4, 2, 8, True, (-1, -1), 1),
    (1, 24, 24, 4, 1, 16, True, (3, 2), 2),
    (1, 20, 20, 2, 2, 8, False, (2, 5), 3),
    (1, 12, 20, 2, 1, 8, True, (-1, -1), 4),
    (1, 20, 20, 6, 2, 8, False, (4, 0), 5),
    (1, 17, 17, 2, 2, 4, True, (5, -1), 6),
]


def pin_sdpa():
    worst = 0.0
    for B, Nq, Nk, Hq, Hkv, D, causal, window, seed in SDPA_CASES:
        q, k, v = rand_qkv(seed, B, Nq, Nk, Hq, Hkv, D)
        scale = 1.0 / math.sqrt(D) * (1.3 if seed % 2 else 1.0)
        o, l = attention_fp64(q, k, v, scale, causal, window)
        ro, rl = sdpa_reference(q, k, v, scale, causal, window)
        worst = nanmax(worst, np.abs(o - ro).max(), np.abs(l - rl).max())
    return worst


def pin_bruteforce():
    """40-digit arithmetic, explicit loops over every (query, key) pair."""
    mpmath.mp.dps = 40
    worst = 0.0
    cases = [(5, 7, 2, 1, 3, False, (-1, -1)), (6, 6, 2, 2, 4, True, (-1, -1)), (7, 7, 3, 1, 2, True, (2, 1)),
             (8, 8, 2, 1, 3, False, (1, 3)), (4, 8, 2, 2, 2, True, (-1, -1))]
    for ci, (Nq, Nk, Hq, Hkv, D, causal, (wl, wr)) in enumerate(cases):
        q, k, v = rand_qkv(100 + ci, 1, Nq, Nk, Hq, Hkv, D)
        scale = 1.0 / math.sqrt(D)
        o, l = attention_fp64(q, k, v, scale, causal, (wl, wr))
        G = Hq // Hkv
        off = Nk - Nq
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                keys = []
                for j in range(Nk):
                    if causal and j > i + off:
                        continue
                    if wl >= 0 and j < i + off - wl:
                        continue
                    if wr >= 0 and j > i + off + wr:
                        continue
                    keys.append(j)
                s = {j: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, i, h, d]) * mpmath.mpf(k[0, j, g, d])
                                                        for d in range(D)) for j in keys}
                z = mpmath.fsum(mpmath.exp(s[j]) for j in keys)
                for d in range(D):
                    ref = mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(v[0, j, g, d]) for j in keys) / z
                    worst = nanmax(worst, abs(float(ref) - o[0, i, h, d]))
                worst = nanmax(worst, abs(float(mpmath.log(z)) - l[0, h, i]))
    return worst


def pin_grid_example():
    """The 8-token / 2x2-block example: blocked online traversal == full softmax, block counts."""
    meta, grid = read_grid()
    n, br, bc = meta["tokens"], meta["block_rows"], meta["block_cols"]
    assert len(grid) == n and all(len(r) == n for r in grid)
    letters = {grid[i][j] for i in range(n) for j in range(n)}
    assert len(letters) == meta["blocks"] == (n // br) * (n // bc)
    worst = 0.0
    for causal in (False, True):
        for seed in range(3):
            q, k, v = rand_qkv(200 + seed, 1, n, n, 1, 1, 4)
            o, l = attention_fp64(q, k, v, 0.5, causal)
            to, tl, classes = tiled_online_fp64(q, k, v, 0.5, causal, block_q=br, block_k=bc)
            worst = nanmax(worst, np.abs(o - to).max(), np.abs(l - tl).max())
            if causal:
                got = (classes["skipped"], classes["partial"], classes["full"])
                want = (meta["causal_skipped"], meta["causal_partial"], meta["causal_full"])
                if got != want:
                    return math.inf
            elif classes != {"skipped": 0, "partial": 0, "full": meta["blocks"]}:
                return math.inf
    # random sizes and block shapes, with masks
    g = np.random.default_rng(7)
    for t in range(6):
        Nq, Nk = int(g.integers(3, 30)), int(g.integers(3, 30))
        causal = bool(t % 2)
        if causal and Nq > Nk:
            Nq = Nk
        win = (int(g.integers(0, 6)), int(g.integers(0, 6))) if t >= 3 else (-1, -1)
        q, k, v = rand_qkv(300 + t, 1, Nq, Nk, 2, 1, 5)
        o, l = attention_fp64(q, k, v, 0.4, causal, win)
        to, tl, _ = tiled_online_fp64(q, k, v, 0.4, causal, win, block_q=int(g.integers(1, 7)),
                                      block_k=int(g.integers(1, 7)))
        fin = np.isfinite(l)
        worst = nanmax(worst, np.abs(o - to).max(), np.abs(l[fin] - tl[fin]).max())
        if not np.array_equal(np.isfinite(l), np.isfinite(tl)):
            return math.inf
    return worst


def pin_row_shift():
    """K -> K + 1 u^T adds c_i = scale * <q_i, u> to row i: out unchanged, lse shifted by c_i."""
    worst = 0.0
    for causal, win in ((False, (-1, -1)), (True, (-1, -1)), (True, (4, 0))):
        q, k, v = rand_qkv(11, 2, 12, 12, 4, 2, 8)
        u = np.random.default_rng(12).standard_normal(8) * 3.0
        scale = 0.35
        o, l = attention_fp64(q, k, v, scale, causal, win)
        o2, l2 = attention_fp64(q, k + u, v, scale, causal, win)
        G = 2
        c = scale * np.einsum("bihd,d->bhi", q, u)
        worst = nanmax(worst, np.abs(o - o2).max(), np.abs((l2 - l) - c).max())
    return worst


def pin_causal_row0():
    q, k, v = rand_qkv(21, 2, 9, 9, 4, 2, 8)
    o, l = attention_fp64(q, k, v, 0.3, True)
    worst = 0.0
    for h in range(4):
        worst = nanmax(worst, np.abs(o[:, 0, h, :] - v[:, 0, h // 2, :]).max())
        worst = nanmax(worst, np.abs(l[:, h, 0] - 0.3 * np.sum(q[:, 0, h, :] * k[:, 0, h // 2, :], -1)).max())
    return worst


def pin_identical_keys():
    worst = 0.0
    N, D = 10, 6
    for causal, win in ((False, (-1, -1)), (True, (-1, -1)), (False, (2, 3)), (True, (3, 0))):
        q, k, v = rand_qkv(31, 1, N, N, 2, 1, D)
        k[:] = k[:, :1]                      # every key equal to key 0
        o, l = attention_fp64(q, k, v, 0.7, causal, win)
        for i in range(N):
            lo = 0 if win[0] < 0 else max(0, i - win[0])
            hi = i if causal else (N - 1 if win[1] < 0 else min(N - 1, i + win[1]))
            mean = v[0, lo:hi + 1, 0, :].mean(0)
            cnt = hi - lo + 1
            for h in range(2):
                worst = nanmax(worst, np.abs(o[0, i, h] - mean).max())
                worst = nanmax(worst, abs(l[0, h, i] - (0.7 * q[0, i, h] @ k[0, 0, 0] + math.log(cnt))))
    return worst


def pin_window_zero():
    q, k, v = rand_qkv(41, 2, 11, 11, 3, 3, 5)
    o, l = attention_fp64(q, k, v, 0.9, False, (0, 0))
    s_diag = 0.9 * np.einsum("bihd,bihd->bhi", q, k)
    return max(np.abs(o - v).max(), np.abs(l - s_diag).max())


def pin_big_window():
    q, k, v = rand_qkv(51, 1, 13, 13, 2, 1, 4)
    worst = 0.0
    for causal in (False, True):
        o, l = attention_fp64(q, k, v, 0.5, causal)
        for win in ((13, 13), (40, 99), (12, 12)):
            o2, l2 = attention_fp64(q, k, v, 0.5, causal, win)
            worst = nanmax(worst, np.abs(o - o2).max(), np.abs(l - l2).max())
    return worst


def pin_gqa():
    q, k, v = rand_qkv(61, 2, 7, 9, 6, 2, 4)
    o, l = attention_fp64(q, k, v, 0.5, False)
    o2, l2 = attention_fp64(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 0.5, False)
    return max(np.abs(o - o2).max(), np.abs(l - l2).max())


def pin_mask_probe():
    """Q = 0: weights uniform over admitted keys; exp(lse) and one-hot V recover integer counts."""
    worst = 0.0
    for Nq, Nk, causal, win in ((16, 16, True, (-1, -1)), (16, 16, True, (3, 3)), (16, 16, False, (2, 5)),
                                (10, 16, True, (4, -1)), (16, 16, False, (0, 7))):
        D = 4
        q = np.zeros((1, Nq, 1, D))
        k = np.random.default_rng(71).standard_normal((1, Nk, 1, D))
        v = np.zeros((1, Nk, 1, D))
        v[0, np.arange(Nk), 0, np.arange(Nk) % D] = 1.0
        o, l = attention_fp64(q, k, v, 1.0, causal, win)
        m = torch_mask(Nq, Nk, causal, *win).numpy()
        cnt = m.sum(1)
        got = np.where(np.isfinite(l[0, 0]), np.rint(np.exp(l[0, 0])), 0)
        if not np.array_equal(got, cnt):
            return math.inf
        for i in range(Nq):
            want = np.array([m[i, d::D].sum() for d in range(D)])
            have = np.rint(o[0, i, 0] * cnt[i]) if cnt[i] else np.zeros(D)
            if not np.array_equal(have, want):
                return math.inf
            worst = nanmax(worst, np.abs(o[0, i, 0] * cnt[i] - want).max())
    return worst


def pin_formats():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = decode_e4m3_codes(codes.numpy())
    if not np.array_equal(np.isnan(ref), np.isnan(ours)):
        return math.inf
    fin = ~np.isnan(ref)
    worst = np.abs(ref[fin] - ours[fin]).max()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    tb = torch.from_numpy(bits.view(np.int16))
    for dec, tdt in ((decode_f16_bits, torch.float16), (decode_bf16_bits, torch.bfloat16)):
        r = tb.view(tdt).to(torch.float64).numpy()
        o = dec(bits)
        if not np.array_equal(np.isnan(r), np.isnan(o)):
            return math.inf
        f = ~np.isnan(r)
        if not np.array_equal(r[f], o[f]):
            return math.inf
    return worst


PINS = {
    "sdpa": (pin_sdpa, 1e-12),
    "bruteforce": (pin_bruteforce, 1e-13),
    "grid_example": (pin_grid_example, 1e-13),
    "row_shift": (pin_row_shift, 1e-12),
    "causal_row0": (pin_causal_row0, 1e-14),
    "identical_keys": (pin_identical_keys, 1e-13),
    "window_zero": (pin_window_zero, 1e-14),
    "big_window": (pin_big_window, 0.0),
    "gqa": (pin_gqa, 0.0),
    "mask_probe": (pin_mask_probe, 1e-12),
    "formats": (pin_formats, 0.0),
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    err = fn()
    assert err <= tol, f"pin {name}: worst error {err} > {tol}"


def test_fp8_special_values():
    t = OF.e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite magnitude
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x38] == 1.0 and t[0x08] == 2.0 ** -6          # 1.0, smallest normal
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2                           # no infinities, two NaN codes


def test_empty_rows_zero_and_neg_inf():
    # Nq > Nk with bottom-right causal alignment: the first Nq - Nk rows admit no key (reading R4).
    q, k, v = rand_qkv(81, 1, 8, 5, 2, 1, 4)
    o, l = attention_fp64(q, k, v, 0.5, True)
    assert np.all(o[0, :3] == 0) and np.all(np.isneginf(l[0, :, :3]))
    assert np.all(np.isfinite(l[0, :, 3:]))


def test_rows_variant_equals_full():
    q, k, v = rand_qkv(91, 2, 33, 40, 4, 2, 8)
    o, l = attention_fp64(q, k, v, 0.3, True, (7, -1), row_chunk=5)
    rows = [0, 5, 17, 32]
    for b in range(2):
        for h in range(4):
            ro, rl = OA.attention_rows_fp64(q, k, v, b, h, rows, 0.3, True, (7, -1))
            assert np.array_equal(ro, o[b, rows, h]) and np.array_equal(rl, l[b, h, rows])


# ----------------------------------------------------------------------------------------------
# mutation tests: a plausible mistake planted in the oracle must make some pin fail
# ----------------------------------------------------------------------------------------------
def _failing_pins(names):
    bad = []
    for n in names:
        fn, tol = PINS[n]
        try:
            err = fn()
        except Exception:
            err = math.inf
        if not (err <= tol):
            bad.append(n)
    return bad


def _mut_one_head(change):
    def one_head(qh, kh, vh, scale, mask):
        if change == "no_scale":
            scale = 1.0
        if change == "k_as_v":
            vh = kh
        s = scale * (qh @ kh.T)
        s = np.where(mask, s, -np.inf)
        axis = 0 if change == "wrong_axis" else 1
        m = s.max(axis=axis, keepdims=True)
        m_fin = np.where(np.isfinite(m), m, 0.0)
        e = np.where(mask, np.exp(s - m_fin), 0.0)
        l = e.sum(axis=axis, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            w = np.nan_to_num(e / l)
        out = w @ vh
        lr = l.reshape(-1)[: qh.shape[0]] if axis == 1 else e.sum(axis=1)
        mr = m.reshape(-1)[: qh.shape[0]] if axis == 1 else s.max(axis=1)
        with np.errstate(divide="ignore"):
            lse = np.log(lr) if change == "lse_no_max" else mr + np.log(lr)
        return out, lse
    return one_head


def _mut_admitted(change):
    orig = OA.admitted

    def adm(Nq, Nk, causal=False, window_left=-1, window_right=-1, rows=None):
        if change == "swap_window":
            window_left, window_right = window_right, window_left
        if change == "causal_strict":
            base = orig(Nq, Nk, False, window_left, window_right, rows)
            i = (np.arange(Nq) if rows is None else np.asarray(rows))[:, None]
            j = np.arange(Nk)[None, :]
            return base & (j < i + (Nk - Nq)) if causal else base
        return orig(Nq, Nk, causal, window_left, window_right, rows)
    return adm


MUTANTS = {
    "gqa_modulo": ("kv_head_of", lambda hq, Hq, Hkv: hq % Hkv),
    "causal_strict": ("admitted", _mut_admitted("causal_strict")),
    "swap_window": ("admitted", _mut_admitted("swap_window")),
    "no_scale": ("_one_head", _mut_one_head("no_scale")),
    "lse_no_max": ("_one_head", _mut_one_head("lse_no_max")),
    "k_as_v": ("_one_head", _mut_one_head("k_as_v")),
    "wrong_axis": ("_one_head", _mut_one_head("wrong_axis")),
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    attr, repl = MUTANTS[mutant]
    monkeypatch.setattr(OA, attr, repl)
    bad = _failing_pins(["sdpa", "causal_row0", "row_shift", "gqa", "mask_probe", "identical_keys"])
    assert bad, f"no pin caught mutant {mutant}"


def test_pins_catch_missing_rescale(monkeypatch):
    # A blocked traversal that forgets to rescale acc when the max grows must fail the grid pin.
    orig_exp = np.exp

    def tiled_no_rescale(q, k, v, scale=None, causal=False, window=(-1, -1), block_q=2, block_k=2):
        B, Nq, Hq, D = q.shape
        out = np.zeros_like(q)
        lse = np.zeros((B, Hq, Nq))
        for b in range(B):
            for h in range(Hq):
                for i0 in range(0, Nq, block_q):
                    qi = q[b, i0:i0 + block_q, h]
                    m = np.full(qi.shape[0], -np.inf); l = np.zeros(qi.shape[0]); acc = np.zeros((qi.shape[0], D))
                    for j0 in range(0, k.shape[1], block_k):
                        mask = OA.admitted(Nq, k.shape[1], causal, *window, rows=np.arange(i0, i0 + qi.shape[0]))[:, j0:j0 + block_k]
                        if not mask.any():
                            continue
                        s = np.where(mask, scale * qi @ k[b, j0:j0 + block_k, h].T, -np.inf)
                        mn = np.maximum(m, s.max(1))
                        p = np.where(mask, orig_exp(s - mn[:, None]), 0.0)
                        l = orig_exp(np.where(np.isfinite(m), m - mn, -np.inf)) * l + p.sum(1)
                        acc = acc + p @ v[b, j0:j0 + block_k, h]     # planted mistake: acc not rescaled
                        m = mn
                    out[b, i0:i0 + block_q, h] = acc / l[:, None]
                    lse[b, h, i0:i0 + block_q] = m + np.log(l)
        return out, lse, {"skipped": 6, "partial": 4, "full": 6}

    me = sys.modules[__name__]
    monkeypatch.setattr(me, "tiled_online_fp64", tiled_no_rescale)
    assert "grid_example" in _failing_pins(["grid_example"])


def test_pins_catch_wrong_fp8_bias(monkeypatch):
    bad_table = OF.e4m3_table() * 0.5     # as if the exponent bias were 8
    monkeypatch.setattr(OF, "_E4M3", bad_table)
    assert "formats" in _failing_pins(["formats"])
