"""Float64 references for the three groupwise FP8 GEMM forms (oracle; test infrastructure only).

Source: MATE FlashInfer-API page (mate-docs.mthreads.com/latest/api/flashinfer.html), section
"GEMM":
  * ``gemm_fp8_nt_groupwise``: a (m,k) and b (n,k) row-major FP8; the result is a @ b.T with
    groupwise FP32 scaling. a_scale is (m, k_blocks) when K-major or (k_blocks, m) when MN-major;
    b_scale is (n_blocks, k_blocks) or (k_blocks, n_blocks); one common layout for both; the default
    granularity (m, n, k) = (1, 128, 128).
  * ``group_deepgemm_fp8_nt_groupwise``: for every row i with m_indices[i] >= 0,
    out[i] = a[i] @ b[m_indices[i]].T; rows with m_indices == -1 are padding, output unspecified.
  * ``batch_deepgemm_fp8_nt_groupwise``: out[g, :masked_m[g]] = a[g, :masked_m[g]] @ b[g].T;
    rows at or beyond masked_m[g] are unspecified.

Definition written out (granularity (1,128,128), KB = k/128, deq = exact E4M3 value):

  ref[i, j] = sum_kb  sa[i, kb] * sb[j // 128, kb] * sum_{k in block kb} deq(a[i,k]) * deq(b[j,k])

The scale multiplies (dequantises) the code, the reading under which a scale of amax/448 makes
sense. Each inner block sum is formed by one float64 matrix product: every E4M3 value is a multiple
of 2^-9 below 2^9, so each product is a multiple of 2^-18 below 2^18 and a 128-term sum stays
below 2^43 units of 2^-18 -- exact in float64 in any summation order. sa*sb (two float32 values) is
exact in float64. Unspecified output rows are returned as NaN so that callers cannot compare them.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import MAX_FINITE as MAX_E4M3, decode, encode_rne

BLOCK = 128


def _scales_k_major(a_scale, b_scale, m, n_blocks, k_blocks, scale_major):
    sa = np.asarray(a_scale, dtype=np.float32)
    sb = np.asarray(b_scale, dtype=np.float32)
    if sb.ndim == 0:
        # a scalar b_scale is one scale for every (n block, k block)
        sb = np.full((n_blocks, k_blocks), sb, dtype=np.float32)
    if scale_major == "K":
        want_a, want_b = (m, k_blocks), (n_blocks, k_blocks)
    elif scale_major == "MN":
        want_a, want_b = (k_blocks, m), (k_blocks, n_blocks)
    else:
        raise ValueError("scale_major must be 'K' or 'MN'")
    if sa.shape != want_a or sb.shape != want_b:
        raise ValueError(f"scale shapes {sa.shape}, {sb.shape}; expected {want_a}, {want_b}")
    if scale_major == "MN":
        sa, sb = sa.T, sb.T
    return sa.astype(np.float64), sb.astype(np.float64)


def gemm_fp8_nt_groupwise(a, b, a_scale, b_scale, scale_major: str = "K") -> np.ndarray:
    """float64 (m, n) reference of a @ b.T with (1,128,128) groupwise scales."""
    a = np.asarray(a)
    b = np.asarray(b)
    m, k = a.shape
    n, kb_ = b.shape
    if kb_ != k or k % BLOCK:
        raise ValueError("need a (m,k), b (n,k), k a multiple of 128")
    # any n: column j uses b-scale block j // 128, so there are ceil(n/128) blocks
    k_blocks, n_blocks = k // BLOCK, -(-n // BLOCK)
    sa, sb = _scales_k_major(a_scale, b_scale, m, n_blocks, k_blocks, scale_major)
    ref = np.zeros((m, n), dtype=np.float64)
    for kb in range(k_blocks):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        block = decode(a[:, ks]) @ decode(b[:, ks]).T          # exact block sums
        scale = sa[:, kb][:, None] * np.repeat(sb[:, kb], BLOCK)[None, :n]
        ref += block * scale
    return ref


def fp8_output_codes(values, output_scale) -> np.ndarray:
    """E4M3 codes of the FP8-output variant (``output_scale`` of gemm_fp8_nt_groupwise): the value
    divided by the per-tensor scale in float32 (the precision the GPU decides the code in),
    saturated to +-448, rounded to nearest even; NaN stays NaN."""
    v32 = np.asarray(values, dtype=np.float64).astype(np.float32)
    q = v32 / np.float32(output_scale)
    q = np.where(np.isnan(q), q, np.clip(q, -MAX_E4M3, MAX_E4M3)).astype(np.float32)
    return encode_rne(q)


def group_gemm_contiguous(a, b, a_scale, b_scale, m_indices, rows=None) -> np.ndarray:
    """float64 reference of the contiguous grouped form; padding rows (index -1) are NaN.

    ``rows`` optionally restricts the computation to a subset of row indices (the result then has
    one row per entry of ``rows``). Rows are handled one expert at a time, whatever their order, so
    nothing here assumes 128-row alignment.
    """
    a = np.asarray(a)
    m_indices = np.asarray(m_indices, dtype=np.int64)
    m, k = a.shape
    groups, n, _ = b.shape
    k_blocks, n_blocks = k // BLOCK, n // BLOCK
    sa = np.asarray(a_scale, dtype=np.float32).reshape(m, k_blocks)
    sb = np.asarray(b_scale, dtype=np.float32).reshape(groups, n_blocks, k_blocks)
    rows = np.arange(m) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.full((rows.size, n), np.nan, dtype=np.float64)
    experts = m_indices[rows]
    for e in np.unique(experts):
        if e < 0 or e >= groups:
            continue
        sel = np.nonzero(experts == e)[0]
        r = rows[sel]
        out[sel] = gemm_fp8_nt_groupwise(a[r], b[e], sa[r], sb[e], "K")
    return out


def batch_gemm_masked(a, b, a_scale, b_scale, masked_m, groups=None, rows=None) -> np.ndarray:
    """float64 reference of the masked batched form; rows >= masked_m[g] are NaN.

    ``groups``/``rows`` optionally restrict the work to some groups and to some row indices within
    each group (the result keeps the full (G, max_m, n) shape; skipped entries are NaN).
    """
    a = np.asarray(a)
    num_groups, max_m, k = a.shape
    _, n, _ = b.shape
    k_blocks, n_blocks = k // BLOCK, n // BLOCK
    sa = np.asarray(a_scale, dtype=np.float32).reshape(num_groups, max_m, k_blocks)
    sb = np.asarray(b_scale, dtype=np.float32).reshape(num_groups, n_blocks, k_blocks)
    out = np.full((num_groups, max_m, n), np.nan, dtype=np.float64)
    for g in (range(num_groups) if groups is None else groups):
        # counts outside [0, max_m] are not defined by the page; they are clamped into range
        valid = min(max(int(masked_m[g]), 0), max_m)
        r = np.arange(valid) if rows is None else np.asarray([x for x in rows if x < valid], dtype=np.int64)
        if r.size == 0:
            continue
        out[g, r] = gemm_fp8_nt_groupwise(a[g, r], b[g], sa[g, r], sb[g], "K")
    return out
