"""Round-to-nearest-even float -> bfloat16, from the format definition (oracle; test infrastructure).

The groupwise GEMMs of the MATE FlashInfer-API page (section "GEMM") return BF16 by default.
bfloat16 keeps float32's 8 exponent bits and 7 explicit mantissa bits, so a finite normal value
a in [2^E, 2^(E+1)) is rounded to a multiple of 2^(E-7), ties to the even multiple.
"""

from __future__ import annotations

import numpy as np


def round_to_bf16(x) -> np.ndarray:
    """float64 values of the bf16 numbers nearest to ``x`` (RNE). Overflow gives +-inf."""
    a = np.asarray(x, dtype=np.float64)
    out = np.empty_like(a)
    finite = np.isfinite(a)
    mag = np.abs(np.where(finite, a, 0.0))
    # exponent of the leading bit; below the smallest normal (2^-126) the quantum stays 2^-133
    _, e2 = np.frexp(np.where(mag > 0, mag, 1.0))
    e_unb = np.maximum(e2.astype(np.int64) - 1, -126)
    quantum = np.ldexp(1.0, e_unb - 7)
    r = np.rint(mag / quantum) * quantum                  # rint rounds half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)              # beyond the largest finite bf16
    out[:] = np.where(finite, np.copysign(r, a), a)
    return out


def to_bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of round_to_bf16(x)."""
    r = round_to_bf16(x).astype(np.float32)               # exact: bf16 values are float32 values
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
