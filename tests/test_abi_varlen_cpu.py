"""fa_fwd_varlen argument validation on the CPU: every invalid argument is rejected with its code
before any device call (fake, never-dereferenced addresses)."""
import ctypes
import os

import pytest

import exact_attention_09_amd as fa
from exact_attention_09_amd.fa355 import FaVarlenStrides

P = 0x10000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa355.so is not built; run `python -m exact_attention_09_amd.build`")
    return fa.load()


def call(lib, ptrs=None, B=2, total_q=300, total_k=300, max_q=200, Hq=4, Hkv=2, D=64, strides=None, scale=0.125,
         causal=0, wl=-1, wr=-1, dtype=0, null_strides=False, descale=None):
    p = [P] * 7 if ptrs is None else ptrs
    st = FaVarlenStrides(*(strides or [Hq * D, D, Hkv * D, D, Hkv * D, D, Hq * D, D]))
    return lib.fa_fwd_varlen(*p, B, total_q, total_k, max_q, Hq, Hkv, D, None if null_strides else ctypes.byref(st),
                             scale, causal, wl, wr, dtype, None, descale)


@pytest.mark.parametrize("i", [0, 1, 2, 3, 5, 6])
def test_varlen_null_pointer(lib, i):
    p = [P] * 7
    p[i] = None
    assert call(lib, ptrs=p) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(null_strides=True), 1),
    (dict(B=0), 2), (dict(total_q=0), 2), (dict(total_k=0), 2), (dict(max_q=0), 2), (dict(max_q=301), 2),
    (dict(Hq=3, Hkv=2), 2),
    (dict(D=96), 3),
    (dict(wl=-2), 4),
    (dict(scale=0.0), 5), (dict(scale=float("inf")), 5),
    (dict(dtype=2), 8),                       # e4m3 without descale
    (dict(dtype=7), 7),
])
def test_varlen_rejects_invalid(lib, kw, code):
    assert call(lib, **kw) == code


def test_varlen_rejects_bad_strides_and_alignment(lib):
    ok = [4 * 64, 64, 2 * 64, 64, 2 * 64, 64, 4 * 64, 64]
    for i in range(8):
        bad = list(ok)
        bad[i] = -64
        assert call(lib, strides=bad) == 6
        bad[i] = ok[i] + 1
        assert call(lib, strides=bad) == 6
    bad = list(ok)
    bad[6] = 32                                # output rows overlap
    assert call(lib, strides=bad) == 6
    for i in (0, 1, 2, 3):
        p = [P] * 7
        p[i] = P + 8
        assert call(lib, ptrs=p) == 6
    for i in (5, 6):                           # offsets need 4-byte alignment
        p = [P] * 7
        p[i] = P + 2
        assert call(lib, ptrs=p) == 6


def test_varlen_too_large(lib):
    # one packed tensor spanning 2^31 bytes
    assert call(lib, total_q=1 << 24, total_k=300, max_q=200, Hq=64, Hkv=2, D=64,
                strides=[64 * 64, 64, 2 * 64, 64, 2 * 64, 64, 64 * 64, 64]) == 10
