"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the attention arithmetic: it only draws q, k, v and rounds them to the
storage format the kernel reads. Both the HIP path and the CPU oracle are fed from here.

Recipe (the workloads the pages describe; no dataset is involved):
  * q [B, Nq, Hq, D], then k [B, Nk, Hkv, D], then v [B, Nk, Hkv, D], drawn in that order as iid
    N(0, 1) fp32 from ``torch.Generator("cpu").manual_seed(seed)``;
  * fp16 / bf16: round-to-nearest-even cast of the fp32 draw;
  * fp8 e4m3 (OCP "fn" variant): per-tensor scale s = amax|x| / 448, codes = cast(clamp(x / s, +-448))
    with round-to-nearest-even; the dequantisation scale handed to the kernel is s. The clamp is
    needed because the cast maps values past the largest finite code to NaN instead of saturating.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

E4M3_MAX = 448.0


def draw_qkv(B, Nq, Nk, Hq, Hkv, D, seed):
    """fp32 CPU tensors q, k, v drawn iid N(0, 1) in the order q, k, v."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn(B, Nq, Hq, D, generator=g)
    k = torch.randn(B, Nk, Hkv, D, generator=g)
    v = torch.randn(B, Nk, Hkv, D, generator=g)
    return q, k, v


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor e4m3 quantisation: returns (codes as torch.float8_e4m3fn, dequant scale float)."""
    amax = float(x.abs().max())
    s = amax / E4M3_MAX if amax > 0 else 1.0
    s = float(torch.tensor(s, dtype=torch.float32))          # the scale is an fp32 number
    x8 = (x / s).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return x8, s


def to_storage(q, k, v, dtype: str):
    """Round fp32 q, k, v to the kernel's storage type. Returns (q, k, v, descale) with
    descale = (sq, sk, sv) for e4m3 and None otherwise."""
    if dtype == "f16":
        return q.half(), k.half(), v.half(), None
    if dtype == "bf16":
        return q.bfloat16(), k.bfloat16(), v.bfloat16(), None
    if dtype == "e4m3":
        (q8, sq), (k8, sk), (v8, sv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
        return q8, k8, v8, (sq, sk, sv)
    raise ValueError(f"unknown dtype {dtype}")


@dataclass(frozen=True)
class Workload:
    """One attention forward problem: sizes, storage type, mask and scale (None = 1/sqrt(D))."""
    name: str
    B: int
    Nq: int
    Nk: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    causal: bool = False
    window: tuple = (-1, -1)
    scale: float | None = None
    seeds: tuple = field(default=(0,))

    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else self.D ** -0.5


# The workloads the pages use, in the [batch, seqlen, nheads, headdim] layout.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("mha_b1_h2_n128_d64_f16", 1, 128, 128, 2, 2, 64, "f16", seeds=(0, 1, 2)),
        Workload("mha_b2_h8_n512_d64_f16", 2, 512, 512, 8, 8, 64, "f16", scale=0.125, seeds=(0, 1, 2)),
        Workload("causal_b4_h32_n4096_d64_f16", 4, 4096, 4096, 32, 32, 64, "f16", causal=True, scale=0.125),
        Workload("causal_b4_h32_n4096_d64_bf16", 4, 4096, 4096, 32, 32, 64, "bf16", causal=True, scale=0.125),
        Workload("gqa_b1_hq32_hkv8_n16384_d128_bf16", 1, 16384, 16384, 32, 8, 128, "bf16", causal=True),
        Workload("mqa_b1_hq32_hkv1_n16384_d128_bf16", 1, 16384, 16384, 32, 1, 128, "bf16", causal=True),
        Workload("gqa_win256_b1_hq32_hkv8_n16384_d128_bf16", 1, 16384, 16384, 32, 8, 128, "bf16", causal=True,
                 window=(256, 256)),
        Workload("mqa_win256_b1_hq32_hkv1_n16384_d128_bf16", 1, 16384, 16384, 32, 1, 128, "bf16", causal=True,
                 window=(256, 256)),
        Workload("causal_fp8_b2_h32_n4096_d64_e4m3", 2, 4096, 4096, 32, 32, 64, "e4m3", causal=True, scale=0.125),
    ]
}


def make_inputs(w: Workload, seed: int):
    """(q, k, v, descale) for workload ``w`` on the CPU, in storage format."""
    q, k, v = draw_qkv(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.D, seed)
    return to_storage(q, k, v, w.dtype)


# ---- packed variable-length batches
@dataclass(frozen=True)
class VarlenWorkload:
    """B sequences with seeded lengths, uniform on [len_lo, len_hi] (queries and keys of a
    sequence have the same length), packed along the token axis."""
    name: str
    B: int
    len_lo: int
    len_hi: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    causal: bool = False
    window: tuple = (-1, -1)
    scale: float | None = None

    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else self.D ** -0.5

    def lengths(self, seed: int = 0):
        g = torch.Generator().manual_seed(10_000 + seed)
        return torch.randint(self.len_lo, self.len_hi + 1, (self.B,), generator=g).tolist()


def offsets(lengths):
    """int32 [B + 1] cumulative offsets of the sequence lengths."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def make_varlen_inputs(lengths_q, lengths_k, Hq, Hkv, D, dtype: str, seed: int):
    """Packed (q [total_q, Hq, D], k, v [total_k, Hkv, D], cu_q, cu_k, descale) on the CPU, in storage
    format; the values are one draw_qkv draw of a batch of one packed sequence."""
    cu_q, cu_k = offsets(lengths_q), offsets(lengths_k)
    q, k, v = draw_qkv(1, int(cu_q[-1]), int(cu_k[-1]), Hq, Hkv, D, seed)
    q, k, v, d = to_storage(q[0], k[0], v[0], dtype)
    return q, k, v, cu_q, cu_k, d


# The pages' variable-length use (no padding): a mix of sequence lengths with about as many
# tokens as the [4, 4096, 32, 64] causal workload.
VARLEN_WORKLOADS = {
    w.name: w
    for w in [
        VarlenWorkload("varlen_b8_len512to4096_h32_d64_f16", 8, 512, 4096, 32, 32, 64, "f16", causal=True, scale=0.125),
        VarlenWorkload("varlen_b16_len128to8192_hq32_hkv8_d128_bf16", 16, 128, 8192, 32, 8, 128, "bf16", causal=True),
    ]
}


# ---- decode-shaped attention against a (paged) key/value cache
@dataclass(frozen=True)
class KVCacheWorkload:
    """B sequences, Nq new queries each, against cached keys of seeded lengths uniform on
    [len_lo, len_hi]; page_size 0 means a dense cache [B, len_hi, Hkv, D]."""
    name: str
    B: int
    Nq: int
    len_lo: int
    len_hi: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    page_size: int = 0
    causal: bool = False
    scale: float | None = None

    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else self.D ** -0.5

    def lengths(self, seed: int = 0):
        g = torch.Generator().manual_seed(20_000 + seed)
        return torch.randint(self.len_lo, self.len_hi + 1, (self.B,), generator=g).tolist()


def _randn_storage(shape, g, dtype: str, chunk_rows: int = 4096):
    """N(0, 1) fp32 draws rounded to the storage type, generated along the first axis in chunks
    (so that a multi-GB cache never exists in fp32)."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    out = torch.empty(shape, dtype=tdt)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g).to(tdt)
    return out


def make_kvcache_inputs(B, Nq, Hq, Hkv, D, dtype: str, lengths, page_size: int, seed: int, max_len: int | None = None):
    """(q [B, Nq, Hq, D], k_cache, v_cache, seqlens_k int32 [B], block_table int32 [B, pages] or None) on the
    CPU. Paged: each sequence's pages are a seeded random choice among all pages of the pool
    (pool = the pages the sequences need plus 3 spare); unused table entries are 0. Dense: the
    cache is [B, max_len, Hkv, D] (max_len defaults to the longest sequence)."""
    g = torch.Generator().manual_seed(seed)
    q = _randn_storage((B, Nq, Hq, D), g, dtype)
    seqlens = torch.tensor(lengths, dtype=torch.int32)
    if page_size == 0:
        L = max_len or max(max(lengths), 1)
        k = _randn_storage((B, L, Hkv, D), g, dtype)
        v = _randn_storage((B, L, Hkv, D), g, dtype)
        return q, k, v, seqlens, None
    need = [(n + page_size - 1) // page_size for n in lengths]
    num_pages = sum(need) + 3
    perm = torch.randperm(num_pages, generator=g)
    table = torch.zeros(B, max(max(need), 1), dtype=torch.int32)
    at = 0
    for b, npg in enumerate(need):
        table[b, :npg] = perm[at:at + npg].to(torch.int32)
        at += npg
    k = _randn_storage((num_pages, page_size, Hkv, D), g, dtype)
    v = _randn_storage((num_pages, page_size, Hkv, D), g, dtype)
    return q, k, v, seqlens, table


# The pages' serving configuration: 16-token cache pages and up to 128 sequences
# ("FlashAttention V3 principles and practice", section 4), a Llama-3-8B-shaped attention layer
# (32 query heads, 8 K/V heads, D = 128, bf16), one new token per sequence; and a dense cache with
# 4 new tokens per sequence (causal among them).
KVCACHE_WORKLOADS = {
    w.name: w
    for w in [
        KVCacheWorkload("decode_paged16_b128_len512to8192_hq32_hkv8_d128_bf16", 128, 1, 512, 8192, 32, 8, 128, "bf16",
                        page_size=16),
        KVCacheWorkload("decode_dense_b16_nq4_len4096to16384_hq32_hkv8_d128_bf16", 16, 4, 4096, 16384, 32, 8, 128,
                        "bf16", causal=True),
    ]
}


# ---- block-sparse attention
def sparse_block_mask(Nq: int, Nk: int, heads: int, band: int, sinks: int, p_random: float, seed: int,
                      causal: bool = True):
    """uint8 [heads, ceil(Nq / 128), ceil(Nk / 64)] block mask of a local + sink + random pattern:
    for query block r (rows 128 r .. 128 r + 127) the key blocks of the band reaching `band` blocks
    of 64 keys before its diagonal blocks (2 r, 2 r + 1; keys and queries aligned at the end), the
    first `sinks` key blocks, and each other key block with probability `p_random` (seeded). With
    `causal`, blocks entirely after the diagonal are left out."""
    nqb, nkb = -(-Nq // 128), -(-Nk // 64)
    off = Nk - Nq
    g = torch.Generator().manual_seed(30_000 + seed)
    m = (torch.rand(heads, nqb, nkb, generator=g) < p_random)
    r = torch.arange(nqb)[:, None]
    kb = torch.arange(nkb)[None, :]
    diag_lo = (128 * r + off) // 64            # key block of the block's first row's diagonal
    diag_hi = (128 * r + 127 + off) // 64
    m |= ((kb >= diag_lo - band) & (kb <= diag_hi))[None]
    m |= (kb < sinks)[None]
    if causal:
        m &= (kb <= diag_hi)[None]
    return m.to(torch.uint8)


@dataclass(frozen=True)
class SparseWorkload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    band: int
    sinks: int
    p_random: float
    mask_heads: int = 1
    causal: bool = True
    scale: float | None = None

    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else self.D ** -0.5

    def mask(self, seed: int = 0):
        return sparse_block_mask(self.N, self.N, self.mask_heads, self.band, self.sinks, self.p_random, seed,
                                 self.causal)


# The pages' block-sparse claim is for long sequences (64k tokens): a 65 536-token causal
# sequence with a local band of 512 keys, 2 sink blocks and 5 % random blocks, shared by all 16
# heads (D = 64, fp16); and a per-head pattern at 16k tokens, D = 128, bf16.
SPARSE_WORKLOADS = {
    w.name: w
    for w in [
        SparseWorkload("blocksparse_b1_h16_n65536_d64_f16", 1, 65536, 16, 16, 64, "f16", band=8, sinks=2,
                       p_random=0.05, scale=0.125),
        SparseWorkload("blocksparse_b1_h32_n16384_d128_bf16_perhead", 1, 16384, 32, 8, 128, "bf16", band=4, sinks=1,
                       p_random=0.1, mask_heads=32),
    ]
}
