"""E4M3FN codec written from the format's bit definition (oracle; test infrastructure only).

The MATE FlashInfer-API page names ``torch.float8_e4m3fn`` as the FP8 dtype (section "Attention",
``mla_rope_quantize_fp8``) and asks for "FP8 E4M3" inputs to every groupwise GEMM (section "GEMM").
E4M3FN (the OCP 8-bit floating-point format, "FN" = finite + NaN, no infinities):

  bit 7 = sign s, bits 6..3 = exponent e (bias 7), bits 2..0 = mantissa f
  e == 0            : (-1)^s * f * 2^-9              (subnormal; f = 0 gives +-0)
  e == 15 and f == 7: NaN                            (codes 0x7F and 0xFF)
  otherwise         : (-1)^s * (1 + f/8) * 2^(e-7)   (largest finite: 0x7E = 448)
"""

from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0


def _decode_one(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    f = code & 0x7
    if e == 0xF and f == 0x7:
        return math.nan
    if e == 0:
        mag = f * 2.0 ** -9
    else:
        mag = (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def decode_table() -> np.ndarray:
    """All 256 codes decoded to float64 (NaN at 0x7F and 0xFF; 0x80 is -0.0)."""
    return np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


_LUT = decode_table()


def decode(codes: np.ndarray) -> np.ndarray:
    """Exact float64 values of an array of E4M3 codes (uint8)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return _LUT[codes]


def _encode_one(x: float) -> int:
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    # Saturating mode: magnitudes that round beyond 448 clamp to 448. The midpoint between 448 and
    # the (absent) next step 480 is 464; RNE sends 464 itself to 448 (even mantissa).
    if a >= 464.0:
        return sign | 0x7E
    if a < 2.0 ** -6:
        # Subnormal range: quantum 2^-9. q may reach 8, which is exactly the code of 2^-6.
        q = _rne(a / 2.0 ** -9)
        return sign | q
    mant, exp2 = math.frexp(a)          # a = mant * 2^exp2, mant in [0.5, 1)
    e_unb = exp2 - 1                    # a in [2^e_unb, 2^(e_unb+1))
    quantum = 2.0 ** (e_unb - 3)        # 3 mantissa bits
    q = _rne(a / quantum)               # in [8, 16]
    if q == 16:
        e_unb += 1
        q = 8
    code = ((e_unb + 7) << 3) | (q - 8)
    return sign | code


def _rne(v: float) -> int:
    """Round a non-negative float64 to the nearest integer, ties to even (exact for our ranges)."""
    fl = math.floor(v)
    frac = v - fl
    if frac > 0.5:
        return int(fl) + 1
    if frac < 0.5:
        return int(fl)
    return int(fl) if int(fl) % 2 == 0 else int(fl) + 1


def encode_rne(x) -> np.ndarray:
    """Round float values to E4M3FN codes, round-to-nearest-even, saturating at +-448.

    ``x`` is taken at its own precision (pass float32 to round a float32 value). Each element is
    converted to float64 exactly and rounded once.
    """
    arr = np.asarray(x)
    flat = arr.astype(np.float64).ravel()
    out = np.empty(flat.shape, dtype=np.uint8)
    # Vectorised path for the common case, checked element-wise against _encode_one by the tests.
    out[:] = _encode_vec(flat)
    return out.reshape(arr.shape)


def _encode_vec(a64: np.ndarray) -> np.ndarray:
    nan = np.isnan(a64)
    sign = np.where(np.signbit(a64), 0x80, 0).astype(np.int64)
    a = np.abs(np.where(nan, 0.0, a64))
    sat = a >= 464.0
    sub = a < 2.0 ** -6
    # normal range
    mant, exp2 = np.frexp(np.where(sub | sat, 1.0, a))
    e_unb = exp2.astype(np.int64) - 1
    quantum = np.ldexp(1.0, e_unb - 3)
    q = np.rint(np.where(sub | sat, 8.0, a) / quantum).astype(np.int64)  # rint = half-to-even
    carry = q == 16
    e_unb = np.where(carry, e_unb + 1, e_unb)
    q = np.where(carry, 8, q)
    code_norm = ((e_unb + 7) << 3) | (q - 8)
    code_sub = np.rint(np.where(sub, a, 0.0) / 2.0 ** -9).astype(np.int64)
    code = np.where(sub, code_sub, code_norm)
    code = np.where(sat, 0x7E, code)
    code = code | sign
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def encode_scalar(x: float) -> int:
    """Scalar reference encoder (the definition, one value at a time)."""
    return _encode_one(float(x))
