"""Helpers for the GPU parity tests: decode storage tensors with the oracle's own decoders and
compare kernel outputs with the fp64 oracle under the stated tolerances."""
import numpy as np
import torch

from oracle import attention_fp64, attention_rows_fp64, decode_bf16_bits, decode_e4m3_codes, decode_f16_bits

# Tolerances against the fp64 oracle on the same (already rounded) inputs.
OUT_TOL = {"f16": 2e-3, "bf16": 1.5e-2}   # max |out - ref|
FP8_RMS_TOL = 6e-2                           # RMS(out - ref) <= 6e-2 * RMS(ref)
LSE_TOL = 1e-3                               # max |lse - ref|, natural log

DTYPE_NAME = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3"}


def decode(x: torch.Tensor, descale: float = 1.0) -> np.ndarray:
    """Exact fp64 values of a CPU storage tensor (fp16 / bf16 / e4m3 codes times descale)."""
    x = x.contiguous()
    if x.dtype == torch.float16:
        return decode_f16_bits(x.view(torch.int16).numpy().view(np.uint16))
    if x.dtype == torch.bfloat16:
        return decode_bf16_bits(x.view(torch.int16).numpy().view(np.uint16))
    if x.dtype == torch.float8_e4m3fn:
        return decode_e4m3_codes(x.view(torch.uint8).numpy(), descale)
    raise TypeError(x.dtype)


def out_to_f64(o: torch.Tensor) -> np.ndarray:
    return decode(o.cpu())


def oracle_full(q, k, v, scale, causal, window, descale=None):
    dq, dk, dv = descale if descale is not None else (1.0, 1.0, 1.0)
    return attention_fp64(decode(q, dq), decode(k, dk), decode(v, dv), scale, causal, window)


def oracle_rows(q, k, v, b, h, rows, scale, causal, window, descale=None):
    """Oracle for selected rows of one (batch, head); decodes only that head's slices."""
    dq, dk, dv = descale if descale is not None else (1.0, 1.0, 1.0)
    Hq, Hkv = q.shape[2], k.shape[2]
    g = h // (Hq // Hkv)
    qh = decode(q[b, :, h, :], dq)[None, :, None, :]
    kh = decode(k[b, :, g, :], dk)[None, :, None, :]
    vh = decode(v[b, :, g, :], dv)[None, :, None, :]
    return attention_rows_fp64(qh, kh, vh, 0, 0, rows, scale, causal, window)


def compare(dtype_name, out, lse, ref_o, ref_l, what=""):
    """Assert the kernel result matches the oracle. out/ref_o fp64 arrays of equal shape."""
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs from the oracle"
    assert np.all(np.isneginf(lse[~fin])), f"{what}: empty rows must have lse = -inf"
    lse_err = float(np.abs(lse[fin] - ref_l[fin]).max()) if fin.any() else 0.0
    err = np.abs(out - ref_o)
    if dtype_name == "e4m3":
        rms_ref = float(np.sqrt(np.mean(ref_o ** 2)))
        rms_err = float(np.sqrt(np.mean(err ** 2)))
        assert rms_err <= FP8_RMS_TOL * rms_ref, f"{what}: RMS err {rms_err} > {FP8_RMS_TOL} * {rms_ref}"
        stats = {"rms_err": rms_err, "rms_ref": rms_ref, "max_err": float(err.max())}
    else:
        assert err.max() <= OUT_TOL[dtype_name], f"{what}: max |out err| {err.max()} > {OUT_TOL[dtype_name]}"
        stats = {"max_err": float(err.max())}
    assert lse_err <= LSE_TOL, f"{what}: max |lse err| {lse_err} > {LSE_TOL}"
    stats["lse_err"] = lse_err
    return stats


def oracle_heads(q, k, v, heads, rows, scale, causal, window, descale=None, workers=None):
    """oracle_rows for each (b, h) of ``heads`` (same ``rows`` for every head), run on a pool of
    host threads with single-threaded BLAS (numpy releases the GIL in its products and ufuncs).
    Returns a list of (out [len(rows), D], lse [len(rows)]) in the order of ``heads``."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    n = workers or max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=n) as ex:
        futs = [ex.submit(oracle_rows, q, k, v, b, h, rows, scale, causal, window, descale) for b, h in heads]
        return [f.result() for f in futs]


def nan_outputs(B, Nq, Hq, D, out_dtype, device="cuda"):
    """out [B, Nq, Hq, D] and lse [B, Hq, Nq] filled with NaN, so that an element the kernel never
    writes fails the comparison."""
    out = torch.full((B, Nq, Hq, D), float("nan"), dtype=out_dtype, device=device)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=device)
    return out, lse


def nan_tailed(x, extra=128, device="cuda"):
    """x [B, N, H, D] on the device as the first N rows of a [B, N + extra, H, D] tensor whose other
    rows are NaN (e4m3: code 0x7F). A kernel that reads rows past N of a head reads NaN inside the
    same allocation, which shows in its output without leaving the allocation."""
    B, N, H, D = x.shape
    if x.dtype == torch.float8_e4m3fn:
        big = torch.full((B, N + extra, H, D), 0x7F, dtype=torch.uint8, device=device)
        big[:, :N] = x.view(torch.uint8).to(device)
        return big.view(torch.float8_e4m3fn)[:, :N]
    big = torch.full((B, N + extra, H, D), float("nan"), dtype=x.dtype, device=device)
    big[:, :N] = x.to(device)
    return big[:, :N]


def widest_row_stride(rows: int, D: int, elem_bytes: int) -> int:
    """The largest row stride (in elements, a whole number of 16-byte units) for which a head of
    ``rows`` rows passes the library's span rule, ((rows + 256) * stride + D) * elem_bytes < 2^31
    (include/fa355.h, FA_ERR_TOO_LARGE); one 16-byte unit more is rejected."""
    s = ((1 << 31) - 1 - D * elem_bytes) // ((rows + 256) * elem_bytes)
    return s - s % (16 // elem_bytes)
