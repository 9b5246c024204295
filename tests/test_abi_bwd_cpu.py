"""fa_bwd argument validation on the CPU: every invalid argument is rejected with its code
before any device call (fake, never-dereferenced addresses)."""
import ctypes
import os

import pytest

import exact_attention_09_amd as fa
from exact_attention_09_amd.fa355 import FaBwdStrides

P = 0x10000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa355.so is not built; run `python -m exact_attention_09_amd.build`")
    return fa.load()


def contiguous_strides(B, Nq, Nk, Hq, Hkv, D):
    qs = [Nq * Hq * D, Hq * D, D]
    ks = [Nk * Hkv * D, Hkv * D, D]
    return qs + ks + ks + qs + qs + qs + ks + ks      # q k v o do dq dk dv


def call(lib, ptrs=None, B=1, Nq=128, Nk=128, Hq=2, Hkv=2, D=64, strides=None, scale=0.125, causal=0, wl=-1, wr=-1,
         dtype=0, null_strides=False, ws_bytes=1 << 40):
    p = [P] * 10 if ptrs is None else ptrs
    st = FaBwdStrides(*(strides or contiguous_strides(B, Nq, Nk, Hq, Hkv, D)))
    return lib.fa_bwd(*p, ws_bytes, B, Nq, Nk, Hq, Hkv, D, None if null_strides else ctypes.byref(st), scale, causal,
                      wl, wr, dtype, None)


@pytest.mark.parametrize("i", range(10))
def test_bwd_null_pointer(lib, i):
    p = [P] * 10
    p[i] = None
    assert call(lib, ptrs=p) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(null_strides=True), 1),
    (dict(B=0), 2), (dict(Nq=0), 2), (dict(Hq=3, Hkv=2), 2),
    (dict(D=96), 3),
    (dict(wl=-2), 4),
    (dict(scale=0.0), 5), (dict(scale=float("nan")), 5), (dict(scale=2.0 ** -121), 5),
    (dict(dtype=2), 7), (dict(dtype=5), 7),
])
def test_bwd_rejects_invalid(lib, kw, code):
    assert call(lib, **kw) == code


def test_bwd_rejects_bad_strides_and_alignment(lib):
    ok = contiguous_strides(1, 128, 128, 2, 2, 64)
    for i in range(24):
        bad = list(ok)
        bad[i] = -64
        assert call(lib, strides=bad) == 6
        bad[i] = ok[i] + 1                      # not a multiple of 16 bytes
        assert call(lib, strides=bad) == 6
    for i in (16, 19, 22):                      # gradient rows closer than D elements
        bad = list(ok)
        bad[i] = 32
        assert call(lib, strides=bad) == 6
    for i in range(10):
        if i == 5:
            continue                            # lse needs only 4-byte alignment
        p = [P] * 10
        p[i] = P + 8                            # the 16-bit tensors and the workspace need 16 bytes
        assert call(lib, ptrs=p) == 6


def test_bwd_misaligned_fp32_buffers(lib):
    p = [P] * 10
    p[5] = P + 2
    assert call(lib, ptrs=p) == 6
    p[5] = P + 4                                # 4-byte aligned lse is accepted (up to the launch)
    p[9] = P + 4
    assert call(lib, ptrs=p) == 6


@pytest.mark.parametrize("sizes", [(1, 128, 128, 2, 2, 64), (2, 200, 333, 4, 2, 128), (1, 16384, 16384, 32, 1, 128),
                                   (4, 4096, 4096, 32, 32, 64), (1, 7, 5, 6, 3, 64)])
def test_bwd_workspace_size(lib, sizes):
    B, Nq, Nk, Hq, Hkv, D = sizes
    n = lib.fa_bwd_workspace_bytes(*sizes)
    rows = 2 * B * Hq * Nq * 4                  # two fp32 values per query row
    assert n % 16 == 0 or n == (rows + 15) // 16 * 16
    assert n >= rows
    # partial sums, when present, are whole fp32 [split, B, Hkv, Nk, D] slabs for dk and dv
    extra = n - (rows + 15) // 16 * 16
    assert extra % (2 * B * Hkv * Nk * D * 4) == 0
    splits = extra // (2 * B * Hkv * Nk * D * 4)
    assert splits == 0 or (splits > 1 and (Hq // Hkv) % splits == 0)
    # one byte short is refused before anything else is looked at
    assert call(lib, B=B, Nq=Nq, Nk=Nk, Hq=Hq, Hkv=Hkv, D=D, ws_bytes=n - 1) == 11
    assert call(lib, B=B, Nq=Nq, Nk=Nk, Hq=Hq, Hkv=Hkv, D=D, ws_bytes=n, strides=[-64] * 24) == 6


def test_bwd_workspace_size_invalid(lib):
    assert lib.fa_bwd_workspace_bytes(0, 128, 128, 2, 2, 64) == 0
    assert lib.fa_bwd_workspace_bytes(1, 128, 128, 3, 2, 64) == 0
    assert lib.fa_bwd_workspace_bytes(1, 128, 128, 2, 2, 96) == 0
    # MQA with long keys: the query heads are split, so partial sums are part of the workspace
    assert lib.fa_bwd_workspace_bytes(1, 16384, 16384, 32, 1, 128) > 2 * 32 * 16384 * 4
