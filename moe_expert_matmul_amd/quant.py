"""Producers of the GEMM's a operand (argument marshalling only).

``fp8_quantize_1x128`` quantises BF16 rows into 1x128 E4M3 blocks with FP32 scales, and
``fused_add_rmsnorm_fp8_block_quant`` follows the MATE FlashInfer-API page (section "norm"): the
residual add and RMSNorm of a row, its BF16 result in ``normed_out``, and the row's 1x128 FP8
quantisation in ``out``/``block_scale``, which are the ``a``/``a_scale`` operands of the section
"GEMM" calls. Both write into caller-given tensors; every step runs in libfp8g.so.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from .gemm import _FP8_DTYPES, _check, _major, _ptr, _require_cuda, _stream


def _scale_shape(rows: int, cols: int, major: int):
    return (rows, cols // 128) if major == _lib.SCALE_K_MAJOR else (cols // 128, rows)


def fp8_quantize_1x128(x: torch.Tensor, out: torch.Tensor, scale_out: torch.Tensor, scale_major="K") -> None:
    """out (rows, cols) E4M3, scale_out 1x128 FP32 scales (K- or MN-major) of x (rows, cols) BF16."""
    dev = _require_cuda(x)
    rows, cols = x.shape
    major = _major(scale_major)
    _check(x, "x", (torch.bfloat16,), (rows, cols), dev)
    _check(out, "out", _FP8_DTYPES, (rows, cols), dev)
    _check(scale_out, "scale_out", (torch.float32,), _scale_shape(rows, cols, major), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_quantize_1x128(_ptr(x), rows, cols, _ptr(out), _ptr(scale_out), major, _stream(dev))
    _lib.check(st, "fp8_quantize_1x128")


def fused_add_rmsnorm_fp8_block_quant(out: torch.Tensor, block_scale: torch.Tensor, normed_out: torch.Tensor,
                                      input: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor,
                                      eps: float = 1e-6, enable_pdl: Optional[bool] = None,
                                      scale_major="K") -> None:
    """residual += input (BF16, in place); normed_out = RMSNorm(residual) * weight (BF16);
    out/block_scale = its 1x128 E4M3 quantisation (row-major scales by default, ``scale_major='MN'``
    for the transposed layout). ``enable_pdl`` has no meaning here and is ignored."""
    dev = _require_cuda(input)
    rows, hidden = input.shape
    major = _major(scale_major)
    _check(input, "input", (torch.bfloat16,), (rows, hidden), dev)
    _check(residual, "residual", (torch.bfloat16,), (rows, hidden), dev)
    _check(weight, "weight", (torch.bfloat16,), (hidden,), dev)
    _check(normed_out, "normed_out", (torch.bfloat16,), (rows, hidden), dev)
    _check(out, "out", _FP8_DTYPES, (rows, hidden), dev)
    _check(block_scale, "block_scale", (torch.float32,), _scale_shape(rows, hidden, major), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_fused_add_rmsnorm_quant(_ptr(out), _ptr(block_scale), _ptr(normed_out), _ptr(input),
                                                     _ptr(residual), _ptr(weight), float(eps), rows, hidden, major,
                                                     _stream(dev))
    _lib.check(st, "fp8_fused_add_rmsnorm_quant")
