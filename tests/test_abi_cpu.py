"""C ABI checks that need no GPU: the library loads, exports what include/fa355.h declares,
rejects every invalid argument before touching a device, and plans K/V tiles exactly as the
admission rule says (checked against brute-force masks built independently with numpy)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import exact_attention_09_amd as fa
from exact_attention_09_amd.fa355 import FaStrides
from tests.gpu_util import widest_row_stride

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa355.so is not built; run `python -m exact_attention_09_amd.build`")
    return fa.load()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(fa.EXPORTED), declared
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True, check=True).stdout
    dyn = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared:
        assert name in dyn, f"{name} not exported"
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.fa_version() >= 100
    seen = set()
    for code in range(13):
        s = fa.status_str(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 13
    assert fa.status_str(99) == "unknown status"


# --- validation: every invalid argument is rejected before any device call -------------------
P = 0x10000  # a 16-byte aligned fake address; never dereferenced because validation fails first


def call(lib, q=P, k=P, v=P, o=P, lse=None, B=1, Nq=128, Nk=128, Hq=2, Hkv=2, D=64, strides="c", scale=0.125,
         causal=0, wl=-1, wr=-1, dtype=0, descale=None):
    if strides == "c":
        s = FaStrides(Nq * Hq * D, Hq * D, D, Nk * Hkv * D, Hkv * D, D, Nk * Hkv * D, Hkv * D, D, Nq * Hq * D, Hq * D, D)
    else:
        s = strides
    d = (ctypes.c_float * 3)(*descale) if descale is not None else None
    return lib.fa_fwd(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, D, ctypes.byref(s) if s is not None else None, scale,
                      causal, wl, wr, dtype, None, d)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(strides=None), 1),
    (dict(B=0), 2), (dict(Nq=0), 2), (dict(Nk=-3), 2), (dict(Hq=3, Hkv=2), 2), (dict(Hkv=0), 2),
    (dict(Nq=(1 << 30) + 1), 2),
    (dict(D=96), 3), (dict(D=256), 3), (dict(D=0), 3),
    (dict(wl=-2), 4), (dict(wr=-5), 4),
    (dict(scale=0.0), 5), (dict(scale=-1.0), 5), (dict(scale=float("inf")), 5), (dict(scale=float("nan")), 5),
    (dict(q=P + 8), 6), (dict(o=P + 4), 6),
    (dict(dtype=3), 7), (dict(dtype=-1), 7),
    (dict(dtype=2), 8),
    (dict(dtype=2, descale=(1.0, 0.0, 1.0)), 5), (dict(dtype=2, descale=(1.0, 1.0, float("nan"))), 5),
])
def test_rejects_invalid(lib, kw, code):
    assert call(lib, **kw) == code


def test_rejects_bad_strides(lib):
    base = dict(B=1, Nq=128, Nk=128, Hq=2, Hkv=2, D=64)
    ok = [128 * 2 * 64, 2 * 64, 64] * 4
    for i in range(12):
        bad = list(ok)
        bad[i] = -64
        assert call(lib, strides=FaStrides(*bad), **base) == 6
    for i in range(12):          # not a multiple of 16 bytes
        bad = list(ok)
        bad[i] = ok[i] + 1
        assert call(lib, strides=FaStrides(*bad), **base) == 6
    overlap = list(ok)
    overlap[10] = 32             # output rows closer than D elements
    assert call(lib, strides=FaStrides(*overlap), **base) == 6
    fp8 = [128 * 2 * 64, 2 * 64, 64] * 3 + [128 * 2 * 64, 2 * 64, 64]
    fp8[1] = 2 * 64 + 8          # 8 bytes of e4m3 rows: misaligned for 128-bit loads
    assert call(lib, strides=FaStrides(*fp8), dtype=2, descale=(1, 1, 1), **base) == 6


def test_rejects_too_large(lib):
    # one head of k spans more than 2^31 bytes
    s = FaStrides(0, 64, 64, 0, 1 << 20, 64, 0, 64, 64, 0, 64, 64)
    assert call(lib, B=1, Nq=1, Nk=2048, Hq=1, Hkv=1, strides=s) == 10


@pytest.mark.parametrize("dtype,D,rows", [(0, 64, 2047), (1, 128, 1999), (2, 64, 2047), (2, 128, 1)])
@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_rejects_one_unit_past_the_widest_span(lib, dtype, D, rows, which):
    # the widest stride of widest_row_stride is the one the GPU max-span tests run; one 16-byte
    # unit more in any one tensor's row stride must be refused before any launch
    es = 1 if dtype == 2 else 2
    es_of = {"q": es, "k": es, "v": es, "o": 2}
    st = {}
    for t in "qkvo":
        st[t] = widest_row_stride(rows, D, es_of[t])
    st[which] += 16 // es_of[which]
    s = FaStrides(0, st["q"], D, 0, st["k"], D, 0, st["v"], D, 0, st["o"], D)
    desc = (1.0, 1.0, 1.0) if dtype == 2 else None
    assert call(lib, B=1, Nq=rows, Nk=rows, Hq=1, Hkv=1, D=D, strides=s, dtype=dtype, descale=desc) == 10


# --- K/V tile planning vs brute-force admission --------------------------------------------
def brute_mask(Nq, Nk, causal, wl, wr):
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    off = Nk - Nq
    m = np.ones((Nq, Nk), bool)
    if causal:
        m &= j - i <= off
    if wl >= 0:
        m &= i + off - j <= wl
    if wr >= 0:
        m &= j - i - off <= wr
    return m


def check_tiles(Nq, Nk, causal, win, bn, r0, r1):
    tb, te, nf, npart, ns = fa.kv_tile_range(Nq, Nk, causal, win, bn, r0, r1)
    m = brute_mask(Nq, Nk, causal, *win)[r0:r1]
    ntiles = (Nk + bn - 1) // bn
    for t in range(ntiles):
        blk = m[:, t * bn:(t + 1) * bn]
        inside = tb <= t < te
        if blk.any():
            assert inside, (Nq, Nk, causal, win, bn, r0, r1, t)
    full = part = skip = 0
    for t in range(tb, te):
        blk = m[:, t * bn:(t + 1) * bn]
        pad = (t + 1) * bn > Nk           # keys past Nk are never admitted
        if blk.all() and not pad:
            full += 1
        elif blk.any():
            part += 1
        else:
            skip += 1
    # the planner may call a tile partial when it is in fact empty, never the reverse, and
    # "full" must be exact
    assert nf == full, (Nq, Nk, causal, win, bn, r0, r1)
    assert npart + ns == part + skip and ns <= skip, (Nq, Nk, causal, win, bn, r0, r1)
    return tb, te, nf, npart, ns


def test_grid_example_block_classes():
    # 8 tokens in 2x2 blocks under a causal mask: per block row, the counts add to 6 skipped
    # (not visited), 4 diagonal (partial), 6 full.
    full = part = visited = 0
    for r0 in range(0, 8, 2):
        tb, te, nf, npart, ns = check_tiles(8, 8, True, (-1, -1), 2, r0, r0 + 2)
        full += nf
        part += npart
        visited += te - tb
    assert (16 - visited, part, full) == (6, 4, 6)


def test_tile_range_random():
    g = np.random.default_rng(3)
    for _ in range(400):
        Nq, Nk = int(g.integers(1, 300)), int(g.integers(1, 300))
        causal = bool(g.integers(0, 2))
        win = tuple(int(x) for x in g.integers(-1, 40, size=2))
        bn = int(g.choice([2, 16, 32, 64]))
        r0 = int(g.integers(0, Nq))
        r1 = int(g.integers(r0 + 1, Nq + 1))
        check_tiles(Nq, Nk, causal, win, bn, r0, r1)


def test_causal_4096_tile_counts():
    # 128-row query tiles against 64-key tiles, causal, Nq = Nk = 4096: tile t visits 2(t+1)
    # key tiles, the last two partial (the diagonal), all others full.
    for t in range(32):
        tb, te, nf, npart, ns = fa.kv_tile_range(4096, 4096, True, (-1, -1), 64, 128 * t, 128 * (t + 1))
        assert (tb, te, nf, npart, ns) == (0, 2 * (t + 1), 2 * t, 2, 0)


def test_plan(lib):
    # D = 64, fp16/bf16: 4 waves of two 32-row query blocks per workgroup: 16 query tiles of 256
    # rows, and query tile qt visits 8 (qt + 1) key tiles of 32 under a causal mask
    p = fa.plan(4, 4096, 4096, 32, 32, 64, causal=True)
    assert p["block_m"] == 256 and p["block_n"] == 32 and p["waves"] == 4 and p["num_q_tiles"] == 16
    assert p["grid"] == 4 * 32 * 16
    assert p["kv_tiles"] == 4 * 32 * sum(8 * (t + 1) for t in range(16))
    assert p["lds_bytes"] == 6 * 32 * 64 * 2
    # D = 128 runs 8 waves: 256 rows of one head, or with 4-way GQA 64 rows of 4 heads
    p = fa.plan(1, 16384, 16384, 32, 32, 128, causal=True, dtype=fa.FA_BF16)
    assert p["block_m"] == 256 and p["waves"] == 8 and p["num_q_tiles"] == 64 and p["heads_per_wg"] == 1
    p = fa.plan(1, 16384, 16384, 32, 8, 128, causal=True, dtype=fa.FA_BF16)
    assert p["block_m"] == 64 and p["waves"] == 8 and p["num_q_tiles"] == 256 and p["heads_per_wg"] == 4
    assert p["grid"] == 8 * 256
    # fp8: 4-wave kernel
    p = fa.plan(2, 4096, 4096, 32, 32, 64, causal=True, dtype=fa.FA_FP8_E4M3)
    assert p["block_m"] == 128 and p["grid"] == 2 * 32 * 32


def _window_key_tiles(Nq, Nk, causal, window, block_m, block_n):
    """Key tiles of block_n keys holding an admitted key of some row of each query tile of block_m
    rows, by brute force over the admission rule (0 <= j < Nk, j <= i + off under the causal
    mask, i + off - wl <= j <= i + off + wr for a window, off = Nk - Nq)."""
    off = Nk - Nq
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    m = np.ones((Nq, Nk), bool)
    if causal:
        m &= j <= i + off
    if window[0] >= 0:
        m &= j >= i + off - window[0]
    if window[1] >= 0:
        m &= j <= i + off + window[1]
    total = 0
    for r0 in range(0, Nq, block_m):
        cols = m[r0:r0 + block_m].any(0)
        total += len(np.unique(np.nonzero(cols)[0] // block_n))
    return total


@pytest.mark.parametrize("Hq,Hkv,hp", [(32, 8, 4), (32, 1, 4), (8, 2, 4), (12, 3, 4), (24, 2, 4), (6, 3, 1), (4, 2, 1), (4, 4, 1)])
@pytest.mark.parametrize("D", [64, 128])
def test_plan_few_keys_packs_gqa_heads(lib, Hq, Hkv, hp, D):
    # few-keys calls whose query heads share a K/V head 4 (or more, a multiple of 4) ways put 4
    # such heads in a workgroup, one wave each over the same 32 rows; other groups keep one head
    Nq, Nk, window = 1000, 1100, (256, 256)
    p = fa.plan(2, Nq, Nk, Hq, Hkv, D, causal=True, window=window, dtype=fa.FA_BF16)
    bm = 128 // hp
    assert (p["block_m"], p["block_n"], p["waves"], p["heads_per_wg"]) == (bm, 32, 4, hp)
    assert p["num_q_tiles"] == -(-Nq // bm) and p["grid"] == 2 * (Hq // hp) * p["num_q_tiles"]
    assert p["kv_tiles"] == 2 * (Hq // hp) * _window_key_tiles(Nq, Nk, True, window, bm, 32)
    # full causal rows: at D = 128 the 8-wave shape packs the same way (64 rows of 4 heads), at
    # D = 64 the two-block shape keeps one head
    q = fa.plan(2, Nq, Nk, Hq, Hkv, D, causal=True, dtype=fa.FA_BF16)
    assert q["heads_per_wg"] == (hp if D == 128 else 1)
    assert q["block_m"] == (256 // q["heads_per_wg"] if D == 128 else 256)


@pytest.mark.parametrize("causal,window,few", [(False, (100, 30), True), (True, (256, 256), True),
                                               (True, (4095, -1), True), (True, (4096, -1), False),
                                               (False, (1000, 100), True), (False, (4000, 100), False),
                                               (False, (100, -1), False)])
def test_plan_few_keys_launch_shape(lib, causal, window, few):
    # fp16/bf16 calls whose rows admit at most 4096 keys take 4-wave workgroups with 32-key tiles;
    # other calls at D = 128 keep 8 waves and 64-key tiles. fp8 never changes.
    Nq, Nk = 1000, 1100
    p = fa.plan(2, Nq, Nk, 4, 2, 128, causal=causal, window=window, dtype=fa.FA_BF16)
    bm, bn = (128, 32) if few else (256, 64)
    assert (p["block_m"], p["block_n"], p["waves"]) == (bm, bn, bm // 32)
    assert p["lds_bytes"] == 6 * bn * 128 * 2
    assert p["num_q_tiles"] == -(-Nq // bm) and p["grid"] == 2 * 4 * p["num_q_tiles"]
    assert p["kv_tiles"] == 2 * 4 * _window_key_tiles(Nq, Nk, causal, window, bm, bn)
    # D = 64: the few-keys shape, else 4 waves of two 32-row blocks (256 rows) against 32-key tiles
    q = fa.plan(2, Nq, Nk, 4, 2, 64, causal=causal, window=window, dtype=fa.FA_F16)
    assert (q["block_m"], q["block_n"], q["waves"]) == (128 if few else 256, 32, 4)
    assert q["kv_tiles"] == 2 * 4 * _window_key_tiles(Nq, Nk, causal, window, q["block_m"], q["block_n"])
    for D in (64, 128):
        q = fa.plan(2, Nq, Nk, 4, 2, D, causal=causal, window=window, dtype=fa.FA_FP8_E4M3)
        assert (q["block_m"], q["block_n"], q["waves"]) == (128, 64, 4)
    with pytest.raises(fa.FaError):
        fa.plan(1, 128, 128, 3, 2, 64)


# --- the binding rejects tensors the kernels would index out of bounds -----------------------
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.float16)


@pytest.mark.parametrize("what", ["v_shape", "k_dtype", "out_shape", "out_dtype", "lse_shape", "lse_dtype",
                                  "lse_strided", "k_rank"])
def test_binding_rejects_mismatched_tensors(lib, what):
    import torch
    q, k, v = _t(1, 64, 4, 64), _t(1, 80, 2, 64), _t(1, 80, 2, 64)
    out, lse = _t(1, 64, 4, 64), torch.zeros(1, 4, 64)
    if what == "v_shape":
        v = _t(1, 79, 2, 64)
    elif what == "k_dtype":
        k = _t(1, 80, 2, 64, dtype=torch.bfloat16)
    elif what == "out_shape":
        out = _t(1, 64, 4, 32)
    elif what == "out_dtype":
        out = _t(1, 64, 4, 64, dtype=torch.bfloat16)
    elif what == "lse_shape":
        lse = torch.zeros(1, 64, 4)
    elif what == "lse_dtype":
        lse = torch.zeros(1, 4, 64, dtype=torch.float64)
    elif what == "lse_strided":
        lse = torch.zeros(1, 64, 4).transpose(1, 2)
    elif what == "k_rank":
        k = _t(80, 2, 64)
    with pytest.raises((ValueError, TypeError)):
        fa.fwd_raw(q, k, v, out, lse, stream=0)


def test_binding_rejects_mismatched_bwd_tensors(lib):
    import torch
    q, k, v = _t(1, 64, 4, 64), _t(1, 80, 2, 64), _t(1, 80, 2, 64)
    out, do, lse = _t(1, 64, 4, 64), _t(1, 64, 4, 64), torch.zeros(1, 4, 64)
    dq, dk, dv = _t(1, 64, 4, 64), _t(1, 80, 2, 64), _t(1, 79, 2, 64)   # dv one row short
    ws = torch.zeros(1 << 12)
    with pytest.raises(ValueError):
        fa.bwd_raw(q, k, v, out, do, lse, dq, dk, dv, ws, stream=0)
