"""Python binding of the three groupwise FP8 GEMM entry points (argument marshalling only).

The ``fp8_*`` functions mirror the C ABI (include/fp8g.h) one to one and write into a caller-given
``out``. The ``gemm_fp8_nt_groupwise`` / ``group_deepgemm_fp8_nt_groupwise`` /
``batch_deepgemm_fp8_nt_groupwise`` wrappers follow the parameter lists of the MATE FlashInfer-API
page (section "GEMM"): they allocate ``out`` when it is omitted and return it. PyTorch supplies
device memory and the current stream; every step of the computation runs in libfp8g.so.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)
_OUT_DTYPES = (torch.bfloat16, torch.float16)  # out_dtype 0 and 1 of the C ABI
_GRAN = (1, 128, 128)


def _out_code(out: torch.Tensor) -> int:
    return _OUT_DTYPES.index(out.dtype)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(t: torch.Tensor, name: str, dtypes, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _major(scale_major) -> int:
    if scale_major in (None, "K", _lib.SCALE_K_MAJOR):
        return _lib.SCALE_K_MAJOR
    if scale_major in ("MN", _lib.SCALE_MN_MAJOR):
        return _lib.SCALE_MN_MAJOR
    raise ValueError(f"scale_major must be 'K' or 'MN', got {scale_major!r}")


def _require_cuda(a: torch.Tensor) -> torch.device:
    if not isinstance(a, torch.Tensor) or a.device.type != "cuda":
        raise ValueError("operands must be HIP device tensors (device 'cuda')")
    return a.device


def fp8_gemm_nt_groupwise(a, b, a_scale, b_scale, out, scale_major="K", granularity=_GRAN) -> torch.Tensor:
    """out (m,n) bf16 or fp16 = a (m,k) @ b (n,k).T with 1x128 / 128x128 FP32 scales (any n: b_scale
    has ceil(n/128) blocks)."""
    dev = _require_cuda(a)
    m, k = a.shape
    n = b.shape[0]
    kb, nb = k // 128, (n + 127) // 128
    major = _major(scale_major)
    _check(a, "a", _FP8_DTYPES, (m, k), dev)
    _check(b, "b", _FP8_DTYPES, (n, k), dev)
    _check(a_scale, "a_scale", (torch.float32,), (m, kb) if major == 0 else (kb, m), dev)
    _check(b_scale, "b_scale", (torch.float32,), (nb, kb) if major == 0 else (kb, nb), dev)
    _check(out, "out", _OUT_DTYPES, (m, n), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_gemm_nt_groupwise(_ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale), _ptr(out),
                                               _out_code(out), m, n, k, major, *granularity, _stream(dev))
    _lib.check(st, "fp8_gemm_nt_groupwise")
    return out


def fp8_gemm_nt_groupwise_fp8_out(a, b, a_scale, b_scale, output_scale, out, scale_major="K",
                                  granularity=_GRAN) -> torch.Tensor:
    """out (m,n) E4M3 codes = E4M3(saturate(a @ b.T / output_scale[0])), output_scale a 1-element FP32
    device tensor (the per-tensor dequantisation scale of the output)."""
    dev = _require_cuda(a)
    m, k = a.shape
    n = b.shape[0]
    kb, nb = k // 128, (n + 127) // 128
    major = _major(scale_major)
    _check(a, "a", _FP8_DTYPES, (m, k), dev)
    _check(b, "b", _FP8_DTYPES, (n, k), dev)
    _check(a_scale, "a_scale", (torch.float32,), (m, kb) if major == 0 else (kb, m), dev)
    _check(b_scale, "b_scale", (torch.float32,), (nb, kb) if major == 0 else (kb, nb), dev)
    _check(output_scale, "output_scale", (torch.float32,), tuple(output_scale.shape), dev)
    if output_scale.numel() != 1:
        raise ValueError(f"output_scale must hold one element (per-tensor scale), got shape {tuple(output_scale.shape)}")
    _check(out, "out", _FP8_DTYPES, (m, n), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_gemm_nt_groupwise_fp8_out(_ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale), _ptr(out),
                                                       _ptr(output_scale), m, n, k, major, *granularity, _stream(dev))
    _lib.check(st, "fp8_gemm_nt_groupwise_fp8_out")
    return out


def fp8_group_gemm_contiguous(a, b, a_scale, b_scale, m_indices, out, scale_major="K",
                              granularity=_GRAN) -> torch.Tensor:
    """out[i] = a[i] @ b[m_indices[i]].T for rows with m_indices[i] >= 0 (others untouched)."""
    dev = _require_cuda(a)
    m, k = a.shape
    groups, n, _ = b.shape
    kb, nb = k // 128, n // 128
    major = _major(scale_major)
    _check(a, "a", _FP8_DTYPES, (m, k), dev)
    _check(b, "b", _FP8_DTYPES, (groups, n, k), dev)
    _check(a_scale, "a_scale", (torch.float32,), (m, kb) if major == 0 else (kb, m), dev)
    _check(b_scale, "b_scale", (torch.float32,), (groups, nb, kb) if major == 0 else (groups, kb, nb), dev)
    _check(m_indices, "m_indices", (torch.int32,), (m,), dev)
    _check(out, "out", _OUT_DTYPES, (m, n), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_group_gemm_contiguous(_ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale), _ptr(m_indices),
                                                   _ptr(out), _out_code(out), m, n, k, groups, major, *granularity,
                                                   _stream(dev))
    _lib.check(st, "fp8_group_gemm_contiguous")
    return out


def fp8_group_gemm_contiguous_gather(a, a_scale, a_rows, b, b_scale, m_indices, out, scale_major="K",
                                     granularity=_GRAN) -> torch.Tensor:
    """out[i] = a[a_rows[i]] @ b[m_indices[i]].T for rows with m_indices[i] >= 0 (others untouched)."""
    dev = _require_cuda(a)
    rows_total, k = a.shape
    m = m_indices.shape[0]
    groups, n, _ = b.shape
    kb, nb = k // 128, n // 128
    major = _major(scale_major)
    _check(a, "a", _FP8_DTYPES, (rows_total, k), dev)
    _check(a_scale, "a_scale", (torch.float32,), (rows_total, kb) if major == 0 else (kb, rows_total), dev)
    _check(a_rows, "a_rows", (torch.int32,), (m,), dev)
    _check(b, "b", _FP8_DTYPES, (groups, n, k), dev)
    _check(b_scale, "b_scale", (torch.float32,), (groups, nb, kb) if major == 0 else (groups, kb, nb), dev)
    _check(m_indices, "m_indices", (torch.int32,), (m,), dev)
    _check(out, "out", _OUT_DTYPES, (m, n), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_group_gemm_contiguous_gather(_ptr(a), _ptr(a_scale), rows_total, _ptr(a_rows), _ptr(b),
                                                          _ptr(b_scale), _ptr(m_indices), _ptr(out), _out_code(out),
                                                          m, n, k, groups, major, *granularity, _stream(dev))
    _lib.check(st, "fp8_group_gemm_contiguous_gather")
    return out


def fp8_batch_gemm_masked(a, b, a_scale, b_scale, masked_m, expected_m, out, scale_major="K",
                          granularity=_GRAN) -> torch.Tensor:
    """out[g, :masked_m[g]] = a[g, :masked_m[g]] @ b[g].T (other rows untouched)."""
    dev = _require_cuda(a)
    groups, max_m, k = a.shape
    n = b.shape[1]
    kb, nb = k // 128, n // 128
    major = _major(scale_major)
    _check(a, "a", _FP8_DTYPES, (groups, max_m, k), dev)
    _check(b, "b", _FP8_DTYPES, (groups, n, k), dev)
    _check(a_scale, "a_scale", (torch.float32,), (groups, max_m, kb) if major == 0 else (groups, kb, max_m), dev)
    _check(b_scale, "b_scale", (torch.float32,), (groups, nb, kb) if major == 0 else (groups, kb, nb), dev)
    _check(masked_m, "masked_m", (torch.int32,), (groups,), dev)
    _check(out, "out", _OUT_DTYPES, (groups, max_m, n), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_batch_gemm_masked(_ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale), _ptr(masked_m),
                                               int(expected_m), _ptr(out), _out_code(out), groups, max_m, n, k,
                                               major, *granularity, _stream(dev))
    _lib.check(st, "fp8_batch_gemm_masked")
    return out


def _out_dtype(out, out_dtype):
    """dtype of the result: out's when given, else out_dtype (BF16 by default; BF16 or FP16)."""
    if out is not None:
        return out.dtype
    if out_dtype is None:
        return torch.bfloat16
    if out_dtype not in _OUT_DTYPES:
        raise NotImplementedError(f"out_dtype {out_dtype} is not implemented (BF16 or FP16)")
    return out_dtype


def gemm_fp8_nt_groupwise(a: torch.Tensor, b: torch.Tensor, a_scale: torch.Tensor, b_scale: torch.Tensor,
                          scale_major_mode: Optional[str] = None, mma_sm: int = 1,
                          scale_granularity_mnk: Tuple[int, int, int] = _GRAN, out: Optional[torch.Tensor] = None,
                          out_dtype: Optional[torch.dtype] = None, backend: str = "auto",
                          output_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Groupwise FP8 NT GEMM with the MATE page's parameters; ``mma_sm`` has no meaning here and is
    ignored, ``backend`` must be 'auto'. With ``output_scale`` (a one-element FP32 tensor) the output
    is E4M3 (``out_dtype`` torch.float8_e4m3fn, the default then, or torch.uint8). A 0-d ``b_scale``
    is one scale for every 128x128 block of b."""
    if backend != "auto":
        raise NotImplementedError("backend must be 'auto'")
    m, k = a.shape
    n = b.shape[0]
    major = _major(scale_major_mode)
    if b_scale.dim() == 0:
        nb = (n + 127) // 128
        shape = (nb, k // 128) if major == 0 else (k // 128, nb)
        b_scale = b_scale.to(torch.float32).expand(shape).contiguous()
    if output_scale is not None:
        if out is None:
            dtype = torch.float8_e4m3fn if out_dtype is None else out_dtype
            if dtype not in _FP8_DTYPES:
                raise NotImplementedError("with output_scale the output is E4M3 (torch.float8_e4m3fn or uint8)")
            out = torch.empty((m, n), dtype=dtype, device=a.device)
        return fp8_gemm_nt_groupwise_fp8_out(a, b, a_scale, b_scale, output_scale, out, major,
                                             tuple(scale_granularity_mnk))
    dtype = _out_dtype(out, out_dtype)
    if out is None:
        out = torch.empty((m, n), dtype=dtype, device=a.device)
    return fp8_gemm_nt_groupwise(a, b, a_scale, b_scale, out, major, tuple(scale_granularity_mnk))


def group_deepgemm_fp8_nt_groupwise(a: torch.Tensor, b: torch.Tensor, a_scale: torch.Tensor,
                                    b_scale: torch.Tensor, m_indices: torch.Tensor,
                                    scale_granularity_mnk: Tuple[int, int, int] = _GRAN,
                                    out: Optional[torch.Tensor] = None,
                                    out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Contiguous grouped FP8 NT GEMM (K-major scales); padding rows of ``out`` are unspecified."""
    if out is None:
        out = torch.empty((a.shape[0], b.shape[1]), dtype=_out_dtype(None, out_dtype), device=a.device)
    return fp8_group_gemm_contiguous(a, b, a_scale, b_scale, m_indices, out, "K", tuple(scale_granularity_mnk))


def batch_deepgemm_fp8_nt_groupwise(a: torch.Tensor, b: torch.Tensor, a_scale: torch.Tensor,
                                    b_scale: torch.Tensor, masked_m: torch.Tensor, expected_m: int,
                                    scale_granularity_mnk: Tuple[int, int, int] = _GRAN,
                                    out: Optional[torch.Tensor] = None,
                                    out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Masked batched FP8 NT GEMM (K-major scales); rows at or beyond masked_m[g] are unspecified."""
    if out is None:
        out = torch.empty((a.shape[0], a.shape[1], b.shape[1]), dtype=_out_dtype(None, out_dtype), device=a.device)
    return fp8_batch_gemm_masked(a, b, a_scale, b_scale, masked_m, expected_m, out, "K",
                                 tuple(scale_granularity_mnk))


def fp8_bmm(a, b, a_scale, b_scale, out, a_scale_per_row: bool, b_scale_per_col: bool) -> torch.Tensor:
    """out (batch,m,n) = sa * sb * (a (batch,m,k) @ b (batch,k,n)); a_scale is one value or (batch, m),
    b_scale one value or (batch, n). b is read in place."""
    dev = _require_cuda(a)
    batch, m, k = a.shape
    n = b.shape[2]
    _check(a, "a", _FP8_DTYPES, (batch, m, k), dev)
    _check(b, "b", _FP8_DTYPES, (batch, k, n), dev)
    _check(a_scale, "a_scale", (torch.float32,), (batch, m) if a_scale_per_row else tuple(a_scale.shape), dev)
    _check(b_scale, "b_scale", (torch.float32,), (batch, n) if b_scale_per_col else tuple(b_scale.shape), dev)
    if not a_scale_per_row and a_scale.numel() != 1:
        raise ValueError("a per-tensor a_scale holds one value")
    if not b_scale_per_col and b_scale.numel() != 1:
        raise ValueError("a per-tensor b_scale holds one value")
    _check(out, "out", _OUT_DTYPES, (batch, m, n), dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        st = lib.fp8_bmm(_ptr(a), _ptr(b), _ptr(a_scale), int(bool(a_scale_per_row)), _ptr(b_scale),
                         int(bool(b_scale_per_col)), _ptr(out), _out_code(out), batch, m, n, k, _stream(dev))
    _lib.check(st, "fp8_bmm")
    return out


def _bmm_scale(scale: torch.Tensor, batch: int, size: int, channel_shape, name: str):
    """(tensor, per_channel) from a tensorwise scalar or a rank-3 channelwise scale."""
    if scale.numel() == 1:
        return scale.reshape(1).to(torch.float32).contiguous(), False
    if scale.dim() == 3 and tuple(scale.shape) == channel_shape:
        return scale.reshape(batch, size).to(torch.float32).contiguous(), True
    raise ValueError(f"{name} must be a scalar or have shape {channel_shape}, got {tuple(scale.shape)}")


def bmm_fp8(A: torch.Tensor, B: torch.Tensor, A_scale: torch.Tensor, B_scale: torch.Tensor, dtype: torch.dtype,
            out: Optional[torch.Tensor] = None, backend: str = "auto") -> torch.Tensor:
    """Batched FP8 GEMM with the MATE page's parameters: A (batch,m,k), B (batch,k,n) E4M3; A_scale a
    scalar or (batch, m, 1), B_scale a scalar or (batch, 1, n); BF16 or FP16 output. With ``out``
    given, nothing is allocated (scales already FP32 and contiguous are used as they are)."""
    if backend != "auto":
        raise NotImplementedError("backend must be 'auto'")
    if A.dtype == torch.float8_e5m2 or B.dtype == torch.float8_e5m2:
        raise NotImplementedError("E5M2 inputs are not implemented (E4M3 only)")
    batch, m, k = A.shape
    n = B.shape[2]
    sa, sa_rows = _bmm_scale(A_scale, batch, m, (batch, m, 1), "A_scale")
    sb, sb_cols = _bmm_scale(B_scale, batch, n, (batch, 1, n), "B_scale")
    if out is None:
        if dtype not in _OUT_DTYPES:
            raise NotImplementedError(f"dtype {dtype} is not implemented (BF16 or FP16)")
        out = torch.empty((batch, m, n), dtype=dtype, device=A.device)
    return fp8_bmm(A, B, sa, sb, out, sa_rows, sb_cols)
