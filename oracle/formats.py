"""Exact decoders of the kernel's storage formats to fp64 — TEST INFRASTRUCTURE ONLY.

The oracle runs on the exact values the GPU sees: inputs rounded to fp16, bf16 or fp8 e4m3 are
decoded bit-exactly here, from each format's published field layout, never through the HIP path.

* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is subnormal.
* bfloat16: the top half of an IEEE binary32: 1 sign, 8 exponent (bias 127), 7 fraction bits.
* OCP FP8 E4M3 ("float8_e4m3fn", the fp8 format named for the pages' fp8 path, skill page,
  Workflow 3 Step 3): 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent 0 is subnormal
  (fraction/8 * 2^-6); there are no infinities, and only S.1111.111 (0x7F, 0xFF) is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np

__all__ = ["e4m3_table", "decode_e4m3_codes", "decode_f16_bits", "decode_bf16_bits"]


def e4m3_table() -> np.ndarray:
    """256-entry fp64 table: value of every E4M3 (fn) code."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        f = code & 0x7
        if e == 0xF and f == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * (f / 8.0) * 2.0 ** (1 - 7)
        else:
            t[code] = sign * (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3_table()


def decode_e4m3_codes(codes, descale: float = 1.0) -> np.ndarray:
    """fp64 value of E4M3 codes (uint8 array) times a per-tensor dequantisation scale."""
    c = np.asarray(codes, dtype=np.uint8)
    return _E4M3[c] * np.float64(descale)


def decode_f16_bits(bits) -> np.ndarray:
    """fp64 value of IEEE binary16 bit patterns (uint16 array)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        val = np.where(e == 0, f * 2.0 ** -24, (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0))
        val = np.where(e == 0x1F, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def decode_bf16_bits(bits) -> np.ndarray:
    """fp64 value of bfloat16 bit patterns (uint16 array)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        val = np.where(e == 0, f * 2.0 ** -133, (1.0 + f / 128.0) * np.exp2(e.astype(np.float64) - 127.0))
        val = np.where(e == 0xFF, np.where(f == 0, np.inf, np.nan), val)
    return sign * val
