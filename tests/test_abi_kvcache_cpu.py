"""fa_fwd_kvcache argument validation on the CPU: every invalid argument is rejected with its code
before any device call (fake, never-dereferenced addresses)."""
import ctypes
import os

import pytest

import exact_attention_09_amd as fa
from exact_attention_09_amd.fa355 import FaStrides

P = 0x10000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa355.so is not built; run `python -m exact_attention_09_amd.build`")
    return fa.load()


def strides(B=2, Nq=1, Hq=8, Hkv=2, D=64, L=1024):
    q = [Nq * Hq * D, Hq * D, D]
    k = [L * Hkv * D, Hkv * D, D]
    return q + k + k + q


def call(lib, ptrs=None, B=2, Nq=1, Hq=8, Hkv=2, D=64, max_k=1024, page=0, max_pages=0, num_pages=0, st=None,
         scale=0.125, causal=0, wl=-1, wr=-1, dtype=1, ws=P, ws_bytes=1 << 40, null_strides=False):
    p = [P] * 6 + [None] if ptrs is None else ptrs      # default: dense cache (no block table)
    s = FaStrides(*(st or strides(B, Nq, Hq, Hkv, D, max_k)))
    return lib.fa_fwd_kvcache(*p, B, Nq, Hq, Hkv, D, max_k, page, max_pages, num_pages,
                              None if null_strides else ctypes.byref(s), scale, causal, wl, wr, dtype, ws, ws_bytes,
                              None)


@pytest.mark.parametrize("i", [0, 1, 2, 3, 5])
def test_kvcache_null_pointer(lib, i):
    p = [P] * 6 + [None]
    p[i] = None
    assert call(lib, ptrs=p) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(null_strides=True), 1),
    (dict(B=0), 2), (dict(Nq=0), 2), (dict(max_k=0), 2), (dict(Hq=6, Hkv=4), 2),
    (dict(page=0, max_pages=4, num_pages=8), 2),          # paged (block table given) needs page_size
    (dict(D=80), 3),
    (dict(wl=-3), 4),
    (dict(scale=-1.0), 5),
    (dict(dtype=2), 7), (dict(dtype=9), 7),
    (dict(ws_bytes=0), 11),
])
def test_kvcache_rejects_invalid(lib, kw, code):
    ptrs = None
    if kw.get("max_pages"):
        ptrs = [P] * 7                                     # block_table non-NULL
    assert call(lib, ptrs=ptrs, **kw) == code


def test_kvcache_workspace_bytes(lib):
    # long keys and few (batch, K/V head) pairs: the keys are split, the workspace holds
    # n_split fp32 rows of D + 1 values per query row
    n = lib.fa_fwd_kvcache_workspace_bytes(2, 1, 8, 2, 64, 1 << 16)
    rows = 2 * 8 * 1
    assert n > 0 and n % (rows * 65 * 4) == 0 and n // (rows * 65 * 4) > 1
    # many pairs and short keys: no split, no workspace (then NULL is accepted)
    assert lib.fa_fwd_kvcache_workspace_bytes(512, 1, 32, 8, 128, 256) == 0
    assert lib.fa_fwd_kvcache_workspace_bytes(0, 1, 8, 2, 64, 1024) == 0
    assert call(lib, B=2, Nq=1, Hq=8, Hkv=2, D=64, max_k=1 << 16, ws_bytes=n - 1,
                st=strides(L=1 << 16)) == 11


def test_kvcache_rejects_bad_strides_and_alignment(lib):
    ok = strides()
    for i in range(12):
        bad = list(ok)
        bad[i] = -64
        assert call(lib, st=bad) == 6
        bad[i] = ok[i] + 4
        assert call(lib, st=bad) == 6
    bad = list(ok)
    bad[11] = 32                                          # output heads overlap
    assert call(lib, st=bad) == 6
    for i in (0, 1, 2, 3):
        p = [P] * 6 + [None]
        p[i] = P + 8
        assert call(lib, ptrs=p) == 6
    for i in (4, 5, 6):                                   # lse, seqlens, block table: 4 bytes
        p = [P] * 7
        p[i] = P + 2
        assert call(lib, ptrs=p, page=16, max_pages=4, num_pages=8) == 6
    assert call(lib, ws=P + 8) == 6                       # the workspace: 16 bytes


# --- fa_fwd_kvcache_noalloc: the same checks, and FA_ERR_SCRATCH before any device call --------
def call_noalloc(lib, ptrs=None, B=2, Nq=1, Hq=8, Hkv=2, D=64, max_k=1024, page=0, max_pages=0, num_pages=0,
                 st=None, scale=0.125, causal=0, wl=-1, wr=-1, dtype=1):
    p = [P] * 6 + [None] if ptrs is None else ptrs
    s = FaStrides(*(st or strides(B, Nq, Hq, Hkv, D, max_k)))
    return lib.fa_fwd_kvcache_noalloc(*p, B, Nq, Hq, Hkv, D, max_k, page, max_pages, num_pages, ctypes.byref(s),
                                      scale, causal, wl, wr, dtype, None)


def test_noalloc_scratch_limit_matches_header(lib):
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa355.h")).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_what_fa_fwd_kvcache_rejects(lib):
    for kw, code in [(dict(B=0), 2), (dict(D=80), 3), (dict(wl=-3), 4), (dict(scale=-1.0), 5), (dict(dtype=2), 7)]:
        assert call_noalloc(lib, **kw) == code == call(lib, **kw)
    p = [P] * 6 + [None]
    p[0] = None
    assert call_noalloc(lib, ptrs=p) == 1
    p[0] = P + 8
    assert call_noalloc(lib, ptrs=p) == 6


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    # 64 sequences x 64 query heads x 16 queries against 16 K/V heads and 2^20 keys: split
    # partials of far more than the fixed scratch. Rejected before any device call.
    B, Nq, Hq, Hkv, D, L = 64, 16, 64, 16, 128, 1 << 20
    need = lib.fa_fwd_kvcache_workspace_bytes(B, Nq, Hq, Hkv, D, L)
    assert need > fa.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(lib, B=B, Nq=Nq, Hq=Hq, Hkv=Hkv, D=D, max_k=L, st=strides(B, Nq, Hq, Hkv, D, L)) == 12
    assert "FA_NOALLOC_SCRATCH_BYTES" in fa.status_str(12)
