"""Python binding of libfa355 (ctypes): argument marshalling only.

Every step of the attention forward pass runs in the HIP kernels behind ``fa_fwd``; this module
only allocates the outputs with PyTorch, reads tensor strides and the current HIP stream, and
calls the C ABI declared in ``include/fa355.h``. There is no fallback: if the library is missing
or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa355.so")

FA_F16, FA_BF16, FA_FP8_E4M3 = 0, 1, 2
_DTYPE_CODE = {torch.float16: FA_F16, torch.bfloat16: FA_BF16, torch.float8_e4m3fn: FA_FP8_E4M3}
_OUT_DTYPE = {FA_F16: torch.float16, FA_BF16: torch.bfloat16, FA_FP8_E4M3: torch.bfloat16}

# Every symbol include/fa355.h declares.
EXPORTED = ("fa_fwd", "fa_fwd_blocksparse", "fa_fwd_varlen", "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_bytes",
            "fa_fwd_kvcache_noalloc", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_str", "fa_fwd_plan",
            "fa_kv_tile_range", "fa_block_order", "fa_version")
# FA_NOALLOC_SCRATCH_BYTES of include/fa355.h: the fixed per-device scratch of fa_fwd_kvcache_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20


class FaStrides(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("q_b", "q_n", "q_h", "k_b", "k_n", "k_h", "v_b", "v_n", "v_h", "o_b", "o_n", "o_h")]


class FaBwdStrides(ctypes.Structure):
    _fields_ = [(f"{t}_{a}", ctypes.c_int64) for t in ("q", "k", "v", "o", "do", "dq", "dk", "dv") for a in "bnh"]


class FaVarlenStrides(ctypes.Structure):
    _fields_ = [(f"{t}_{a}", ctypes.c_int64) for t in ("q", "k", "v", "o") for a in "nh"]


class FaPlanInfo(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("waves", ctypes.c_int),
                ("num_q_tiles", ctypes.c_int), ("grid", ctypes.c_int64), ("lds_bytes", ctypes.c_int),
                ("kv_tiles", ctypes.c_int64), ("heads_per_wg", ctypes.c_int)]


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfa355 call failed: status {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libfa355.so from the package directory (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_09_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_float, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.fa_fwd.restype = c_int
    lib.fa_fwd.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                           c_int, c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(FaStrides),
                           c_float, c_int, c_int, c_int, c_int, c_void_p, ctypes.POINTER(c_float)]
    lib.fa_fwd_blocksparse.restype = c_int
    lib.fa_fwd_blocksparse.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_int, c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(FaStrides),
                                       c_float, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_int]
    lib.fa_fwd_varlen.restype = c_int
    lib.fa_fwd_varlen.argtypes = [c_void_p] * 7 + [c_int] * 7 + [ctypes.POINTER(FaVarlenStrides), c_float, c_int, c_int,
                                                                  c_int, c_int, c_void_p, ctypes.POINTER(c_float)]
    lib.fa_fwd_kvcache.restype = c_int
    lib.fa_fwd_kvcache.argtypes = ([c_void_p] * 7 + [c_int] * 9 + [ctypes.POINTER(FaStrides), c_float, c_int, c_int,
                                   c_int, c_int, c_void_p, ctypes.c_size_t, c_void_p])
    lib.fa_fwd_kvcache_noalloc.restype = c_int
    lib.fa_fwd_kvcache_noalloc.argtypes = ([c_void_p] * 7 + [c_int] * 9 + [ctypes.POINTER(FaStrides), c_float, c_int,
                                           c_int, c_int, c_int, c_void_p])
    lib.fa_fwd_kvcache_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_kvcache_workspace_bytes.argtypes = [c_int] * 6
    lib.fa_bwd.restype = c_int
    lib.fa_bwd.argtypes = [c_void_p] * 10 + [ctypes.c_size_t] + [c_int] * 6 + [ctypes.POINTER(FaBwdStrides), c_float,
                                                                   c_int, c_int, c_int, c_int, c_void_p]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [c_int] * 6
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [c_int]
    lib.fa_fwd_plan.restype = c_int
    lib.fa_fwd_plan.argtypes = [c_int] * 10 + [ctypes.POINTER(FaPlanInfo)]
    lib.fa_kv_tile_range.restype = c_int
    lib.fa_kv_tile_range.argtypes = [c_int] * 8 + [ctypes.POINTER(c_int)] * 5
    lib.fa_block_order.restype = c_int
    lib.fa_block_order.argtypes = [ctypes.c_int64] + [c_int] * 5 + [ctypes.c_void_p] * 3
    lib.fa_version.restype = c_int
    lib.fa_version.argtypes = []
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().fa_status_str(int(status)).decode()


def _strides(q, k, v, o) -> FaStrides:
    s = FaStrides()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous (stride 1), got {t.stride()}")
        setattr(s, name + "_b", t.stride(0))
        setattr(s, name + "_n", t.stride(1))
        setattr(s, name + "_h", t.stride(2))
    return s


def _expect(t, name, shape, dtype, device, contiguous=False):
    """Raise unless tensor t has the given shape, dtype and device (and is contiguous if asked)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _check_fwd(q, k, v, out, lse, code):
    """Shapes, dtypes and devices of a dense forward call: q [B, Nq, Hq, D]; k, v [B, Nk, Hkv, D] of
    q's dtype; out [B, Nq, Hq, D] of the output dtype; lse a contiguous fp32 [B, Hq, Nq] or None."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"q and k must be [batch, seqlen, heads, headdim], got {tuple(q.shape)}, {tuple(k.shape)}")
    B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    _expect(k, "k", (B, Nk, Hkv, D), q.dtype, q.device)
    _expect(v, "v", (B, Nk, Hkv, D), q.dtype, q.device)
    _expect(out, "out", (B, Nq, Hq, D), _OUT_DTYPE[code], q.device)
    if lse is not None:
        _expect(lse, "lse", (B, Hq, Nq), torch.float32, q.device, contiguous=True)


def fwd_raw(q, k, v, out, lse, causal=False, window=(-1, -1), softmax_scale=None, descale=None,
            stream=None) -> int:
    """Call fa_fwd on caller-provided tensors; returns the status code (0 = ok) without raising."""
    lib = load()
    code = _DTYPE_CODE.get(q.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _check_fwd(q, k, v, out, lse, code)
    B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = float(D) ** -0.5 if softmax_scale is None else float(softmax_scale)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    desc = None
    if descale is not None:
        desc = (ctypes.c_float * 3)(*[float(x) for x in descale])
    st = _strides(q, k, v, out)
    return lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      lse.data_ptr() if lse is not None else None,
                      B, Nq, Nk, Hq, Hkv, D, ctypes.byref(st), scale, int(bool(causal)),
                      int(window[0]), int(window[1]), code, stream, desc)


def fwd(q, k, v, causal=False, window=(-1, -1), softmax_scale=None, descale=None, return_lse=True,
        out=None, lse=None):
    """FlashAttention forward on the GPU.

    q: [B, Nq, Hq, D]; k, v: [B, Nk, Hkv, D], all fp16, all bf16, or all float8_e4m3fn (then
    ``descale=(dq, dk, dv)`` is required). ``softmax_scale=None`` means 1/sqrt(D).
    Returns (out [B, Nq, Hq, D], lse [B, Hq, Nq] fp32 or None).
    """
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    code = _DTYPE_CODE.get(q.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, Nq, Hq, D = q.shape
    if out is None:
        out = torch.empty(B, Nq, Hq, D, dtype=_OUT_DTYPE[code], device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device)
    status = fwd_raw(q, k, v, out, lse, causal, window, softmax_scale, descale)
    if status != 0:
        raise FaError(status, status_str(status))
    return out, lse


def fwd_blocksparse_raw(q, k, v, out, lse, block_mask, causal=False, window=(-1, -1), softmax_scale=None,
                        stream=None) -> int:
    """Call fa_fwd_blocksparse on caller-provided tensors; returns the status code without raising.
    ``block_mask``: device uint8 [1 or Hq, ceil(Nq / 128), ceil(Nk / 64)]."""
    lib = load()
    code = _DTYPE_CODE.get(q.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _check_fwd(q, k, v, out, lse, code)
    B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if block_mask.device != q.device:
        raise ValueError("block_mask must be on q's device")
    if block_mask.dtype != torch.uint8 or block_mask.dim() != 3 or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 [mask_heads, nqb, nkb] tensor")
    nqb, nkb = -(-Nq // 128), -(-Nk // 64)
    if tuple(block_mask.shape[1:]) != (nqb, nkb):
        raise ValueError(f"block_mask must be [1 or {Hq}, {nqb}, {nkb}], got {tuple(block_mask.shape)}")
    scale = float(D) ** -0.5 if softmax_scale is None else float(softmax_scale)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _strides(q, k, v, out)
    return lib.fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, B, Nq, Nk, Hq, Hkv, D,
                                  ctypes.byref(st), scale, int(bool(causal)), int(window[0]), int(window[1]), code,
                                  stream, block_mask.data_ptr(), block_mask.shape[0])


def fwd_blocksparse(q, k, v, block_mask, causal=False, window=(-1, -1), softmax_scale=None):
    """Block-sparse FlashAttention forward: fwd restricted to the (128-row, 64-key) blocks that
    ``block_mask`` (device uint8 [1 or Hq, ceil(Nq/128), ceil(Nk/64)]) sets. Returns (out, lse)."""
    if not all(t.is_cuda for t in (q, k, v, block_mask)):
        raise ValueError("all tensors must be device tensors")
    B, Nq, Hq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device)
    status = fwd_blocksparse_raw(q, k, v, out, lse, block_mask, causal, window, softmax_scale)
    if status != 0:
        raise FaError(status, status_str(status))
    return out, lse


def fwd_varlen_raw(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False, window=(-1, -1),
                   softmax_scale=None, descale=None, stream=None) -> int:
    """Call fa_fwd_varlen on caller-provided tensors; returns the status code without raising."""
    lib = load()
    code = _DTYPE_CODE.get(q.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError(f"q and k must be [tokens, heads, headdim], got {tuple(q.shape)}, {tuple(k.shape)}")
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    _expect(k, "k", (total_k, Hkv, D), q.dtype, q.device)
    _expect(v, "v", (total_k, Hkv, D), q.dtype, q.device)
    _expect(out, "out", (total_q, Hq, D), _OUT_DTYPE[code], q.device)
    if lse is not None:
        _expect(lse, "lse", (Hq, total_q), torch.float32, q.device, contiguous=True)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on q's device")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1 or cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be int32 tensors of B + 1 offsets")
    scale = float(D) ** -0.5 if softmax_scale is None else float(softmax_scale)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    desc = None
    if descale is not None:
        desc = (ctypes.c_float * 3)(*[float(x) for x in descale])
    st = FaVarlenStrides()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", out)):
        if t.stride(2) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous (stride 1), got {t.stride()}")
        setattr(st, name + "_n", t.stride(0))
        setattr(st, name + "_h", t.stride(1))
    return lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None, cu_seqlens_q.data_ptr(),
                             cu_seqlens_k.data_ptr(), B, total_q, total_k, int(max_seqlen_q), Hq, Hkv, D,
                             ctypes.byref(st), scale, int(bool(causal)), int(window[0]), int(window[1]), code, stream,
                             desc)


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False, window=(-1, -1),
               softmax_scale=None, descale=None, return_lse=True):
    """FlashAttention forward over a packed batch of variable-length sequences.

    q: [total_q, Hq, D]; k, v: [total_k, Hkv, D]; cu_seqlens_q / cu_seqlens_k: device int32
    [B + 1] offsets; max_seqlen_q: the longest query sequence (a host int).
    Returns (out [total_q, Hq, D], lse [Hq, total_q] fp32 or None).
    """
    if not all(t.is_cuda for t in (q, k, v, cu_seqlens_q, cu_seqlens_k)):
        raise ValueError("all tensors must be device tensors")
    code = _DTYPE_CODE.get(q.dtype)
    if code is None or not (q.dtype == k.dtype == v.dtype):
        raise TypeError(f"unsupported or mixed dtypes {q.dtype} {k.dtype} {v.dtype}")
    total_q, Hq, D = q.shape
    out = torch.empty(total_q, Hq, D, dtype=_OUT_DTYPE[code], device=q.device)
    lse = torch.empty(Hq, total_q, dtype=torch.float32, device=q.device) if return_lse else None
    status = fwd_varlen_raw(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal, window,
                            softmax_scale, descale)
    if status != 0:
        raise FaError(status, status_str(status))
    return out, lse


def kvcache_workspace(q, Hkv, max_seqlen_k):
    """The device workspace fa_fwd_kvcache needs for queries q [B, Nq, Hq, D] (None when none)."""
    B, Nq, Hq, D = q.shape
    nbytes = load().fa_fwd_kvcache_workspace_bytes(B, Nq, Hq, Hkv, D, int(max_seqlen_k))
    return torch.empty(nbytes // 4, dtype=torch.float32, device=q.device) if nbytes else None


def fwd_kvcache_raw(q, k_cache, v_cache, out, lse, seqlens_k, block_table, max_seqlen_k, num_pages=0,
                    causal=False, window=(-1, -1), softmax_scale=None, workspace=None, stream=None,
                    noalloc=False) -> int:
    """Call fa_fwd_kvcache on caller-provided tensors; returns the status code without raising.
    Dense cache: block_table None, k_cache/v_cache [B, max_seqlen_k, Hkv, D]. Paged: k_cache/v_cache
    [num_pages, page_size, Hkv, D] and block_table int32 [B, max_pages_per_seq]. ``noalloc=True``
    calls fa_fwd_kvcache_noalloc instead (no workspace: the library's fixed per-device scratch)."""
    lib = load()
    code = _DTYPE_CODE.get(q.dtype)
    if code is None or code == FA_FP8_E4M3:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError(f"q and k_cache must be 4-d, got {tuple(q.shape)}, {tuple(k_cache.shape)}")
    B, Nq, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if k_cache.shape[3] != D:
        raise ValueError(f"k_cache head dimension {k_cache.shape[3]} != {D}")
    if block_table is None and (k_cache.shape[0] != B or k_cache.shape[1] < max_seqlen_k):
        raise ValueError(f"dense cache must be [{B}, >= max_seqlen_k = {max_seqlen_k}, Hkv, {D}], got "
                         f"{tuple(k_cache.shape)}")
    _expect(v_cache, "v_cache", tuple(k_cache.shape), q.dtype, q.device)
    _expect(k_cache, "k_cache", tuple(k_cache.shape), q.dtype, q.device)
    _expect(out, "out", (B, Nq, Hq, D), q.dtype, q.device)
    if lse is not None:
        _expect(lse, "lse", (B, Hq, Nq), torch.float32, q.device, contiguous=True)
    _expect(seqlens_k, "seqlens_k", (B,), torch.int32, q.device, contiguous=True)
    if block_table is not None:
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError(f"block_table must be [{B}, max_pages], got {tuple(block_table.shape)}")
        _expect(block_table, "block_table", tuple(block_table.shape), torch.int32, q.device, contiguous=True)
    if workspace is not None and workspace.device != q.device:
        raise ValueError("workspace must be on q's device")
    scale = float(D) ** -0.5 if softmax_scale is None else float(softmax_scale)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    page_size = k_cache.shape[1] if block_table is not None else 0
    max_pages = block_table.shape[1] if block_table is not None else 0
    npages = (num_pages or k_cache.shape[0]) if block_table is not None else 0
    st = _strides(q, k_cache, v_cache, out)
    if noalloc:
        if workspace is not None:
            raise ValueError("fa_fwd_kvcache_noalloc takes no workspace")
        return lib.fa_fwd_kvcache_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                          lse.data_ptr() if lse is not None else None, seqlens_k.data_ptr(),
                                          block_table.data_ptr() if block_table is not None else None, B, Nq, Hq,
                                          Hkv, D, int(max_seqlen_k), page_size, max_pages, npages, ctypes.byref(st),
                                          scale, int(bool(causal)), int(window[0]), int(window[1]), code, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return lib.fa_fwd_kvcache(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                              lse.data_ptr() if lse is not None else None, seqlens_k.data_ptr(),
                              block_table.data_ptr() if block_table is not None else None, B, Nq, Hq, Hkv, D,
                              int(max_seqlen_k), page_size, max_pages, npages, ctypes.byref(st), scale,
                              int(bool(causal)), int(window[0]), int(window[1]), code,
                              workspace.data_ptr() if workspace is not None else None, ws_bytes, stream)


def fwd_kvcache(q, k_cache, v_cache, seqlens_k, block_table=None, max_seqlen_k=None, causal=False,
                window=(-1, -1), softmax_scale=None):
    """Attention of q [B, Nq, Hq, D] against each sequence's keys in a dense or paged cache.
    ``seqlens_k``: device int32 [B]; ``max_seqlen_k``: host bound on them (default: the cache's
    capacity). Returns (out [B, Nq, Hq, D], lse [B, Hq, Nq] fp32)."""
    if not all(t.is_cuda for t in (q, k_cache, v_cache, seqlens_k)):
        raise ValueError("all tensors must be device tensors")
    if block_table is not None and (not block_table.is_cuda or block_table.dtype != torch.int32):
        raise ValueError("block_table must be a device int32 tensor")
    if seqlens_k.dtype != torch.int32:
        raise ValueError("seqlens_k must be int32")
    B, Nq, Hq, D = q.shape
    if max_seqlen_k is None:
        max_seqlen_k = block_table.shape[1] * k_cache.shape[1] if block_table is not None else k_cache.shape[1]
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device)
    ws = kvcache_workspace(q, k_cache.shape[2], max_seqlen_k)
    status = fwd_kvcache_raw(q, k_cache, v_cache, out, lse, seqlens_k, block_table, max_seqlen_k, causal=causal,
                             window=window, softmax_scale=softmax_scale, workspace=ws)
    if status != 0:
        raise FaError(status, status_str(status))
    return out, lse


def plan(B, Nq, Nk, Hq, Hkv, D, causal=False, window=(-1, -1), dtype=FA_F16) -> dict:
    info = FaPlanInfo()
    st = load().fa_fwd_plan(B, Nq, Nk, Hq, Hkv, D, int(bool(causal)), int(window[0]), int(window[1]), int(dtype),
                            ctypes.byref(info))
    if st != 0:
        raise FaError(st, status_str(st))
    return {f: getattr(info, f) for f, _ in FaPlanInfo._fields_}


def kv_tile_range(Nq, Nk, causal, window, block_n, row_begin, row_end):
    """(tile_begin, tile_end, full, partial, skipped) for query rows [row_begin, row_end)."""
    vals = [ctypes.c_int() for _ in range(5)]
    st = load().fa_kv_tile_range(Nq, Nk, int(bool(causal)), int(window[0]), int(window[1]), block_n, row_begin,
                                 row_end, *[ctypes.byref(x) for x in vals])
    if st != 0:
        raise FaError(st, status_str(st))
    return tuple(x.value for x in vals)


def block_order(n, num_tiles, heads, group=1, causal=False, packed=False):
    """(b, h, t) int32 numpy arrays: the (batch, head, query tile) of workgroups 0 .. n-1 of a launch."""
    import numpy as np
    b, h, t = (np.empty(n, dtype=np.int32) for _ in range(3))
    st = load().fa_block_order(n, num_tiles, heads, group, int(bool(causal)), int(bool(packed)), b.ctypes.data,
                               h.ctypes.data, t.ctypes.data)
    if st != 0:
        raise FaError(st, status_str(st))
    return b, h, t


def bwd_raw(q, k, v, out, dout, lse, dq, dk, dv, workspace, causal=False, window=(-1, -1), softmax_scale=None,
            stream=None) -> int:
    """Call fa_bwd on caller-provided tensors; returns the status code (0 = ok) without raising.
    ``workspace``: device tensor of at least fa_bwd_workspace_bytes bytes (see ``bwd_workspace``)."""
    lib = load()
    code = _DTYPE_CODE.get(q.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"q and k must be [batch, seqlen, heads, headdim], got {tuple(q.shape)}, {tuple(k.shape)}")
    B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    for name, t, shape in (("k", k, (B, Nk, Hkv, D)), ("v", v, (B, Nk, Hkv, D)), ("out", out, (B, Nq, Hq, D)),
                           ("dout", dout, (B, Nq, Hq, D)), ("dq", dq, (B, Nq, Hq, D)), ("dk", dk, (B, Nk, Hkv, D)),
                           ("dv", dv, (B, Nk, Hkv, D))):
        _expect(t, name, shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, Nq), torch.float32, q.device, contiguous=True)
    if workspace.device != q.device:
        raise ValueError("workspace must be on q's device")
    scale = float(D) ** -0.5 if softmax_scale is None else float(softmax_scale)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = FaBwdStrides()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", out), ("do", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous (stride 1), got {t.stride()}")
        setattr(st, name + "_b", t.stride(0))
        setattr(st, name + "_n", t.stride(1))
        setattr(st, name + "_h", t.stride(2))
    return lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), B, Nq, Nk, Hq, Hkv, D,
                      ctypes.byref(st), scale, int(bool(causal)), int(window[0]), int(window[1]), code, stream)


def bwd_workspace(q, k):
    """The device workspace fa_bwd needs for queries q [B, Nq, Hq, D] and keys k [B, Nk, Hkv, D]
    (fa_bwd_workspace_bytes of the sizes, as an fp32 tensor)."""
    B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    nbytes = load().fa_bwd_workspace_bytes(B, Nq, Nk, Hq, Hkv, D)
    if nbytes == 0:
        raise ValueError(f"invalid sizes for the backward pass: q {tuple(q.shape)}, k {tuple(k.shape)}")
    return torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)


def bwd(q, k, v, out, dout, lse, causal=False, window=(-1, -1), softmax_scale=None):
    """FlashAttention backward on the GPU: (dq, dk, dv) for the forward pass that produced
    ``out`` and ``lse`` from q, k, v with the same options, given dout = dLoss/dout."""
    if not all(t.is_cuda for t in (q, k, v, out, dout, lse)):
        raise ValueError("all tensors must be device tensors")
    B, Nq, Hq, D = q.shape
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    status = bwd_raw(q, k, v, out, dout, lse, dq, dk, dv, bwd_workspace(q, k), causal, window, softmax_scale)
    if status != 0:
        raise FaError(status, status_str(status))
    return dq, dk, dv
