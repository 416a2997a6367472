"""Stages of the FP8 block-scale MoE expert FFN (oracle; test infrastructure only).

Source: flashinfer-rs README, section "API Example: Fused MoE FP8 (cudarc)", DeepSeek FP8
block-scale mode: BF16 tokens, int32 token_selected (num_tokens, top_k), FP8 fc1 weights
[num_experts, fc1_inter, hidden] (fc1_inter = 2 x inter: gate and up), FP8 fc2 weights
[num_experts, hidden, inter], FP32 block scales, hidden and inter divisible by 128. The grouped
GEMM it runs on is the MATE page's ``group_deepgemm_fp8_nt_groupwise`` (section "GEMM").

Stages, in the order the path runs them:
  1. quantize_1x128   tokens -> E4M3 codes + one FP32 scale per 1x128 block (scale = amax/448).
  2. build_permutation  token/slot entries grouped by expert into 128-row-aligned regions,
                        padding rows marked -1 (the contiguous layout of the grouped GEMM).
  3. gather             permuted activation rows.
  4. fc1                contiguous grouped GEMM, BF16 out (oracle.gemm.group_gemm_contiguous).
  5. silu_mul           h = silu(gate) * up over the two halves of fc1's output columns.
  6. quantize_1x128     h -> E4M3 codes + 1x128 scales.
  7. fc2                contiguous grouped GEMM, BF16 out.
  8. combine            out[t] = sum over slots of weight[t, slot] * fc2_row(t, slot).

Precision points: the quantiser's decision (amax, scale = amax/448, x/scale, round to E4M3) is taken
in float32, the precision of the GPU kernel, so that both sides round the same numbers; everything
else is float64.
"""

from __future__ import annotations

import numpy as np

from . import e4m3, bf16
from .gemm import group_gemm_contiguous

BLOCK = 128


def quantize_1x128(x):
    """Row-wise 1x128 block quantisation: (codes uint8 (r,c), scales float32 (r, c/128)).

    scale = amax/448 computed in float32 (IEEE division); a block of zeros gets scale 1.
    codes = RNE_E4M3(float32(x / scale)).
    """
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    if cols % BLOCK:
        raise ValueError("columns must be a multiple of 128")
    blk = x32.reshape(rows, cols // BLOCK, BLOCK)
    amax = np.max(np.abs(blk), axis=2)
    scale = np.where(amax > 0, amax / np.float32(e4m3.MAX_FINITE), np.float32(1.0)).astype(np.float32)
    ratio = (blk / scale[:, :, None]).astype(np.float32)
    codes = e4m3.encode_rne(ratio).reshape(rows, cols)
    return codes, scale


def default_m_alloc(num_tokens: int, top_k: int, num_experts: int) -> int:
    """Rows that hold every expert region whatever the routing: sum(ceil(c_e/128)*128) is at most
    T*top_k + E*127, rounded up to a multiple of 128."""
    worst = num_tokens * top_k + num_experts * (BLOCK - 1)
    return (worst + BLOCK - 1) // BLOCK * BLOCK


def build_permutation(topk_ids, num_experts: int, m_alloc: int | None = None):
    """Group (token, slot) entries by expert.

    Expert e owns rows [offset_e, offset_e + ceil(count_e/128)*128), in expert order; its entries
    fill the first count_e rows in ascending (token, slot) order and the rest are padding.
    Returns dict(m_indices (m_alloc,) int32 with -1 for padding, row_of_entry (T, top_k) int32,
    src_token (m_alloc,) int32 with -1 for padding, counts (E,), offsets (E,), m_pad).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    num_tokens, top_k = ids.shape
    if m_alloc is None:
        m_alloc = default_m_alloc(num_tokens, top_k, num_experts)
    flat = ids.reshape(-1)
    # ids outside [0, E) are routed nowhere (the page does not define them); they get row -1
    valid = (flat >= 0) & (flat < num_experts)
    counts = np.bincount(flat[valid], minlength=num_experts)[:num_experts]
    padded = (counts + BLOCK - 1) // BLOCK * BLOCK
    offsets = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    m_pad = int(padded.sum())
    if m_pad > m_alloc:
        raise ValueError("m_alloc too small for this routing")
    m_indices = np.full(m_alloc, -1, dtype=np.int32)
    src_token = np.full(m_alloc, -1, dtype=np.int32)
    row_of_entry = np.full(flat.size, -1, dtype=np.int64)
    for e in range(num_experts):
        entries = np.nonzero(flat == e)[0]            # ascending entry index = (token, slot) order
        rows = offsets[e] + np.arange(entries.size)
        m_indices[rows] = e
        src_token[rows] = entries // top_k
        row_of_entry[entries] = rows
    return dict(m_indices=m_indices, row_of_entry=row_of_entry.reshape(num_tokens, top_k).astype(np.int32),
                src_token=src_token, counts=counts, offsets=offsets, m_pad=m_pad)


def gather_rows(codes, scales, src_token):
    """Permuted activation rows; padding rows (src -1) are zero codes with scale 1 here (the GPU
    leaves them unspecified, and no valid output depends on them)."""
    src = np.asarray(src_token, dtype=np.int64)
    valid = src >= 0
    out_c = np.zeros((src.size, codes.shape[1]), dtype=np.uint8)
    out_s = np.ones((src.size, scales.shape[1]), dtype=np.float32)
    out_c[valid] = codes[src[valid]]
    out_s[valid] = scales[src[valid]]
    return out_c, out_s


def silu_mul(y):
    """h = silu(y[:, :I]) * y[:, I:] with silu(g) = g / (1 + exp(-g)), in float64."""
    y = np.asarray(y, dtype=np.float64)
    inter = y.shape[1] // 2
    g, u = y[:, :inter], y[:, inter:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def combine(y2, row_of_entry, topk_weights):
    """out[t] = sum_slot w[t, slot] * y2[row_of_entry[t, slot]] in float64; row -1 adds nothing.
    ``topk_weights`` None means weight 1 (the per-tensor call of the flashinfer-rs README passes no
    routing weights)."""
    y2 = np.asarray(y2, dtype=np.float64)
    rows = np.asarray(row_of_entry, dtype=np.int64)
    w = np.ones(rows.shape) if topk_weights is None else np.asarray(topk_weights, dtype=np.float64)
    out = np.zeros((rows.shape[0], y2.shape[1]), dtype=np.float64)
    for slot in range(rows.shape[1]):
        r = rows[:, slot]
        live = r >= 0
        out[live] += w[live, slot:slot + 1] * y2[r[live]]
    return out


def moe_ffn(x, topk_ids, topk_weights, w1, s1, w2, s2, m_alloc=None):
    """All stages chained on the oracle's own intermediates; returns every stage's result.

    fc1/fc2 outputs are rounded to BF16 (the grouped GEMM's output type) before the next stage.
    """
    num_experts = w1.shape[0]
    xq, xs = quantize_1x128(x)
    perm = build_permutation(topk_ids, num_experts, m_alloc)
    a1, sa1 = gather_rows(xq, xs, perm["src_token"])
    y1 = bf16.round_to_bf16(group_gemm_contiguous(a1, w1, sa1, s1, perm["m_indices"]))
    h = silu_mul(np.nan_to_num(y1))
    a2, sa2 = quantize_1x128(h.astype(np.float32))
    y2 = bf16.round_to_bf16(group_gemm_contiguous(a2, w2, sa2, s2, perm["m_indices"]))
    out = combine(np.nan_to_num(y2), perm["row_of_entry"], topk_weights)
    return dict(xq=xq, xs=xs, perm=perm, a1=a1, sa1=sa1, y1=y1, h=h, a2=a2, sa2=sa2, y2=y2, out=out)


# ---- per-tensor FP8 mode (flashinfer-rs README, "API Example: Fused MoE FP8 (cudarc)", per-tensor) --
#
# Readings: the tokens arrive as E4M3 codes; fc1_dequant[e] and fc2_dequant[e] multiply the FP32
# sums of fc1 and fc2 of expert e (they hold the product of the activation's and the weights'
# scales, so fc1_input_dequant is not applied again); fc2_quant multiplies h before the E4M3 cast
# (the page's multiplicative quant-scale convention), one value or one per expert; values beyond
# +-448 saturate; fc1's value is not rounded to BF16 between the GEMM and the activation.


def fc1_act_per_tensor(x_codes, src_token, m_indices, w1, fc1_dequant, fc2_quant):
    """(h, q): h = silu(g) * u in float64 with g, u = fc1_dequant[e] * (x[src] @ w1[e] halves .T);
    q = float32(h) * fc2_quant (float32, the precision the code is decided in); NaN on padding rows."""
    x = np.asarray(x_codes)
    m_idx = np.asarray(m_indices, dtype=np.int64)
    src = np.asarray(src_token, dtype=np.int64)
    w1 = np.asarray(w1)
    inter = w1.shape[1] // 2
    d1 = np.asarray(fc1_dequant, dtype=np.float32).astype(np.float64)
    qs = np.asarray(fc2_quant, dtype=np.float32).reshape(-1)
    h = np.full((m_idx.size, inter), np.nan)
    q = np.full((m_idx.size, inter), np.nan, dtype=np.float32)
    for e in np.unique(m_idx[m_idx >= 0]):
        rows = np.nonzero(m_idx == e)[0]
        y = (e4m3.decode(x[src[rows]]) @ e4m3.decode(w1[e]).T) * d1[e]    # exact sums, one scaling
        h[rows] = silu_mul(y)
        q[rows] = h[rows].astype(np.float32) * qs[e if qs.size > 1 else 0]
    return h, q


def quantize_per_tensor(q):
    """E4M3 codes of float32 values already multiplied by their quantisation scale: saturated to
    +-448, round to nearest even, NaN kept."""
    q = np.asarray(q, dtype=np.float32)
    return e4m3.encode_rne(np.where(np.isnan(q), q, np.clip(q, -e4m3.MAX_FINITE, e4m3.MAX_FINITE)).astype(np.float32))


def fc2_per_tensor(a2_codes, m_indices, w2, fc2_dequant):
    """fc2_dequant[e] * (a2[i] @ w2[e].T) in float64 for rows with e = m_indices[i] >= 0, NaN else."""
    a2 = np.asarray(a2_codes)
    m_idx = np.asarray(m_indices, dtype=np.int64)
    w2 = np.asarray(w2)
    d2 = np.asarray(fc2_dequant, dtype=np.float32).astype(np.float64)
    out = np.full((m_idx.size, w2.shape[1]), np.nan)
    for e in np.unique(m_idx[m_idx >= 0]):
        rows = np.nonzero(m_idx == e)[0]
        out[rows] = (e4m3.decode(a2[rows]) @ e4m3.decode(w2[e]).T) * d2[e]
    return out


def moe_ffn_per_tensor(x_codes, topk_ids, w1, w2, fc1_dequant, fc2_quant, fc2_dequant, topk_weights=None,
                       m_alloc=None):
    """All per-tensor stages chained on the oracle's own intermediates (fc2's output rounded to BF16,
    the stored type, before the combine)."""
    perm = build_permutation(topk_ids, np.asarray(w1).shape[0], m_alloc)
    h, q = fc1_act_per_tensor(x_codes, perm["src_token"], perm["m_indices"], w1, fc1_dequant, fc2_quant)
    a2 = quantize_per_tensor(np.nan_to_num(q))
    y2 = bf16.round_to_bf16(fc2_per_tensor(a2, perm["m_indices"], w2, fc2_dequant))
    out = combine(np.nan_to_num(y2), perm["row_of_entry"], topk_weights)
    return dict(perm=perm, h=h, q=q, a2=a2, y2=y2, out=out)
