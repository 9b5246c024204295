"""CPU fp64 oracle for the FlashAttention forward pass — TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The HIP library and its Python binding never
import, call or link anything here, and nothing here imports them: the two sides share no code.

Sources (the web pages this method is taken from):
  * "Flash Attention - Fast Memory-Efficient Attention" (skill page, skillsmd.top): the quick-start and
    Workflow 1-3 sections give the computed result (standard softmax attention), the
    ``[batch, seqlen, nheads, headdim]`` layout, causal masking, MQA/GQA, the ``(left, right)``
    sliding window, the default ``1/sqrt(d)`` scale and the fp8 e4m3 inputs.
  * "What FlashAttention is and how it speeds up attention" (ya.zerocoder.ru), sections 1-3: the
    method is exact; it visits blocks of Q, K, V held in fast memory and updates the output with a
    correct renormalisation; the 8-token grid in 2x2 blocks is the worked example.

Contents:
  * :mod:`oracle.attention` — ``attention_fp64`` (the plain definition, full score matrix),
    ``tiled_online_fp64`` (the pages' block traversal with running max / running sum),
    ``admitted`` (which (query, key) pairs a causal / window mask keeps), ``kv_head_of``.
  * :mod:`oracle.formats` — exact decoders of fp16, bf16 and OCP e4m3 bit patterns to fp64.
  * :mod:`oracle.backward` — ``attention_bwd_fp64``: the gradients of the same function with
    respect to q, k and v for an upstream gradient of the output (the backward pass).
  * :mod:`oracle.varlen` — ``attention_varlen_fp64``: the same definition applied to each
    sequence of a packed variable-length batch.
  * :mod:`oracle.kvcache` — ``attention_kvcache_fp64``: queries against each sequence's keys in
    a dense or paged key/value cache (the decode-shaped workload).
  * :mod:`oracle.blocksparse` — ``attention_blocksparse_fp64``: the definition restricted to the
    (query block, key block) pairs a block mask sets.

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed forms, invariants,
the worked example, brute force and an independent library routine.
"""
from .attention import admitted, attention_fp64, attention_rows_fp64, kv_head_of, tiled_online_fp64
from .backward import attention_bwd_fp64
from .blocksparse import attention_blocksparse_fp64, block_admitted
from .formats import decode_bf16_bits, decode_e4m3_codes, decode_f16_bits, e4m3_table
from .kvcache import attention_kvcache_fp64, gather_kv
from .varlen import attention_varlen_fp64

__all__ = [
    "admitted",
    "attention_blocksparse_fp64",
    "attention_bwd_fp64",
    "block_admitted",
    "attention_fp64",
    "attention_kvcache_fp64",
    "gather_kv",
    "attention_rows_fp64",
    "attention_varlen_fp64",
    "kv_head_of",
    "tiled_online_fp64",
    "decode_bf16_bits",
    "decode_e4m3_codes",
    "decode_f16_bits",
    "e4m3_table",
]
