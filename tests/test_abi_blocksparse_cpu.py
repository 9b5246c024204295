"""fa_fwd_blocksparse argument validation on the CPU: invalid arguments are rejected with their
code before any device call (fake, never-dereferenced addresses)."""
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


def call(lib, ptrs=None, B=1, Nq=256, Nk=256, Hq=4, Hkv=2, D=64, scale=0.125, causal=1, wl=-1, wr=-1, dtype=0,
         mask=P, mask_heads=1, strides=None):
    p = [P] * 5 if ptrs is None else ptrs
    qs = [Nq * Hq * D, Hq * D, D]
    ks = [Nk * Hkv * D, Hkv * D, D]
    st = FaStrides(*(strides or (qs + ks + ks + qs)))
    return lib.fa_fwd_blocksparse(*p, B, Nq, Nk, Hq, Hkv, D, ctypes.byref(st), scale, causal, wl, wr, dtype, None,
                                  mask, mask_heads)


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), 1),
    (dict(ptrs=[P, None, P, P, P]), 1),
    (dict(dtype=2), 7),                            # e4m3 has no block-sparse path
    (dict(mask_heads=2), 2), (dict(mask_heads=0), 2),
    (dict(Nk=4096 * 64 + 1), 2),                   # the LDS tile list holds 4096 key blocks
    (dict(B=0), 2), (dict(D=96), 3), (dict(wl=-5), 4), (dict(scale=0.0), 5),
])
def test_blocksparse_rejects_invalid(lib, kw, code):
    assert call(lib, **kw) == code


def test_blocksparse_rejects_bad_alignment(lib):
    for i in range(4):
        p = [P] * 5
        p[i] = P + 8
        assert call(lib, ptrs=p) == 6
