"""Fused add-RMSNorm with 1x128 FP8 quantisation (oracle; test infrastructure).

Follows ``fused_add_rmsnorm_fp8_block_quant`` of the MATE FlashInfer-API page (section "norm"):
the residual add, RMSNorm of the result with a per-column weight, and the row-major 1x128 FP8
quantisation whose codes and scales are the ``a`` / ``a_scale`` operands of the section "GEMM"
calls. The page fixes the tensors, not the rounding points; this oracle takes these readings:

  * the updated residual is the BF16 tensor residual + input (exact sum, one RNE rounding);
  * RMSNorm acts on that stored BF16 residual: inv = 1 / sqrt(mean_j r_j^2 + eps), the mean over the
    row's ``hidden`` columns, and normed_out = bf16(r * inv * weight) (weight as is, no 1 + weight);
  * ``out`` / ``block_scale`` are the 1x128 quantisation of the BF16 normed_out values, so that they
    can be reproduced from normed_out alone.

Everything between the rounding points is float64 here.
"""

from __future__ import annotations

import numpy as np

from . import bf16
from .moe import quantize_1x128


def add_residual(input_bits, residual_bits) -> np.ndarray:
    """uint16 BF16 bits of bf16(input + residual); the sum of two BF16 values is exact in float64
    unless their exponents are more than 44 apart, where the single rounding still decides alike."""
    s = bf16.from_bf16_bits(input_bits) + bf16.from_bf16_bits(residual_bits)
    return bf16.to_bf16_bits(s)


def rmsnorm_values(residual_bits, weight_bits, eps: float) -> np.ndarray:
    """float64 RMSNorm of each row before the final BF16 rounding: r * inv * w."""
    r = bf16.from_bf16_bits(residual_bits)
    w = bf16.from_bf16_bits(weight_bits)
    hidden = r.shape[-1]
    mean_sq = np.sum(r * r, axis=-1, keepdims=True) / hidden
    inv = 1.0 / np.sqrt(mean_sq + float(np.float32(eps)))
    return r * inv * w[None, :]


def fused_add_rmsnorm_fp8_block_quant(input_bits, residual_bits, weight_bits, eps: float = 1e-6):
    """Returns (residual_out bits, normed_out bits, codes uint8, scales float32 (rows, hidden/128))."""
    res = add_residual(input_bits, residual_bits)
    normed = bf16.to_bf16_bits(rmsnorm_values(res, weight_bits, eps))
    codes, scales = quantize_1x128(bf16.from_bf16_bits(normed))
    return res, normed, codes, scales
