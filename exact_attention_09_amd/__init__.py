"""libfa355: the FlashAttention forward pass (and its backward pass) on AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of ``include/fa355.h``
(``libfa355.so``, built in-tree by ``python -m exact_attention_09_amd.build``). This package is
the thin Python binding used by the tests and the benchmark; importing it does not load the
library — the first call does, and raises if the library is missing.
"""
from .fa355 import (EXPORTED, FA_BF16, FA_F16, FA_FP8_E4M3, LIB_PATH, NOALLOC_SCRATCH_BYTES, FaError, block_order,
                    bwd, bwd_raw, bwd_workspace, fwd,
                    fwd_blocksparse, fwd_blocksparse_raw,
                    fwd_kvcache, fwd_kvcache_raw, fwd_raw, fwd_varlen, fwd_varlen_raw,
                    kv_tile_range, kvcache_workspace, load, plan, status_str)

__all__ = ["EXPORTED", "FA_BF16", "FA_F16", "FA_FP8_E4M3", "LIB_PATH", "NOALLOC_SCRATCH_BYTES", "FaError", "block_order", "bwd", "bwd_raw", "bwd_workspace", "fwd",
           "fwd_blocksparse", "fwd_blocksparse_raw",
           "fwd_kvcache", "fwd_kvcache_raw", "fwd_raw", "fwd_varlen",
           "fwd_varlen_raw", "kv_tile_range", "kvcache_workspace", "load", "plan", "status_str"]
