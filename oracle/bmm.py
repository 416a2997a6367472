"""Batched FP8 GEMM with per-tensor or per-channel scales (oracle; test infrastructure only).

MATE FlashInfer-API page, section "GEMM", ``bmm_fp8``: A (batch, m, k) and B (batch, k, n) FP8, the
product A @ B per batch, FP32 scales for A and B that are either one tensorwise value or rank-3
channelwise tensors, BF16 or FP16 output. Readings: a channelwise A scale is one value per row of
each batch, shape (batch, m, 1); a channelwise B scale one value per column, shape (batch, 1, n);
a scale multiplies the decoded code. E4M3 only.

  ref[g, i, j] = sa[g, i] * sb[g, j] * sum_k deq(A[g, i, k]) * deq(B[g, k, j])

The k-sum is exact in float64 (every E4M3 product is a multiple of 2^-18 below 2^18, so fewer than
2^17 terms cannot lose a bit), and the product of two float32 scales is exact in float64.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import decode


def _per_batch(scale, batch: int, size: int, axis: int) -> np.ndarray:
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    if s.size == 1:
        return np.full((batch, size), float(s.reshape(-1)[0]))
    want = (batch, size, 1) if axis == 0 else (batch, 1, size)
    if s.shape != want:
        raise ValueError(f"scale shape {s.shape}, expected a scalar or {want}")
    return s.reshape(batch, size)


def bmm_fp8(a, b, a_scale, b_scale) -> np.ndarray:
    """float64 (batch, m, n) reference."""
    a, b = np.asarray(a), np.asarray(b)
    batch, m, k = a.shape
    if b.shape[:2] != (batch, k):
        raise ValueError("need a (batch,m,k) and b (batch,k,n)")
    n = b.shape[2]
    sa = _per_batch(a_scale, batch, m, 0)
    sb = _per_batch(b_scale, batch, n, 1)
    prod = np.stack([decode(a[g]) @ decode(b[g]) for g in range(batch)]) if batch else np.zeros((0, m, n))
    return prod * sa[:, :, None] * sb[:, None, :]
