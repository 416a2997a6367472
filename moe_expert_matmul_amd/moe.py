"""FP8 block-scale expert FFN on the contiguous grouped GEMM (argument marshalling only).

Follows the DeepSeek FP8 block-scale mode of the flashinfer-rs README (section "API Example: Fused
MoE FP8 (cudarc)"): BF16 tokens, int32 top-k expert ids, FP8 fc1 weights (E, 2*inter, hidden) whose
first ``inter`` rows are the gate and the next ``inter`` the up projection, FP8 fc2 weights
(E, hidden, inter), 128x128 FP32 block scales, and the top-k routing weights for the combine.

Five library calls on the current stream, no host synchronisation:
  permutation (three kernels) -> quantise the tokens -> fc1 grouped GEMM reading the token rows through the
  permutation, with SiLU-mul+quantise in its epilogue -> fc2 grouped GEMM -> combine
(``fuse_activation=False`` runs fc1 and the activation as two calls, with the same result).
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib
from .gemm import (_FP8_DTYPES, _GRAN, _OUT_DTYPES, _check, _major, _out_code, _ptr, _require_cuda, _stream,
                   fp8_group_gemm_contiguous, fp8_group_gemm_contiguous_gather)


def default_m_alloc(num_tokens: int, top_k: int, num_experts: int) -> int:
    """Rows that hold every expert region for any routing (each region is padded to 128 rows)."""
    worst = num_tokens * top_k + num_experts * 127
    return (worst + 127) // 128 * 128


@dataclass
class MoeWorkspace:
    """Device buffers of one expert-FFN call (allocated once, reused across calls)."""

    m_indices: torch.Tensor
    src_token: torch.Tensor
    row_of_entry: torch.Tensor
    perm_scratch: torch.Tensor  # the permutation's per-chunk expert counts
    a1: torch.Tensor  # the tokens, 1x128-quantised (num_tokens rows, in token order)
    sa1: torch.Tensor
    y1: torch.Tensor
    a2: torch.Tensor
    sa2: torch.Tensor
    y2: torch.Tensor

    @staticmethod
    def allocate(num_tokens, top_k, num_experts, hidden, inter, device) -> "MoeWorkspace":
        m_alloc = default_m_alloc(num_tokens, top_k, num_experts)
        e = dict(device=device)
        return MoeWorkspace(
            m_indices=torch.empty(m_alloc, dtype=torch.int32, **e),
            src_token=torch.empty(m_alloc, dtype=torch.int32, **e),
            row_of_entry=torch.empty((num_tokens, top_k), dtype=torch.int32, **e),
            perm_scratch=torch.empty(max(permutation_workspace_bytes(num_tokens, top_k, num_experts), 4),
                                     dtype=torch.uint8, **e),
            a1=torch.empty((num_tokens, hidden), dtype=torch.uint8, **e),
            sa1=torch.empty((num_tokens, hidden // 128), dtype=torch.float32, **e),
            y1=torch.empty((m_alloc, 2 * inter), dtype=torch.bfloat16, **e),
            a2=torch.empty((m_alloc, inter), dtype=torch.uint8, **e),
            sa2=torch.empty((m_alloc, inter // 128), dtype=torch.float32, **e),
            y2=torch.empty((m_alloc, hidden), dtype=torch.bfloat16, **e),
        )

    @property
    def m_alloc(self) -> int:
        return self.m_indices.shape[0]


def permutation_workspace_bytes(num_tokens: int, top_k: int, num_experts: int) -> int:
    """Device scratch the permutation needs: one int32 per (chunk of 1024 routing entries, expert)."""
    n = _lib.load().fp8_moe_permutation_workspace_size(num_tokens, top_k, num_experts)
    if n < 0:
        raise ValueError(f"invalid permutation sizes ({num_tokens}, {top_k}, {num_experts})")
    return n


def moe_build_permutation(topk_ids, num_experts, m_indices, src_token, row_of_entry, workspace=None):
    """``workspace``: a uint8 device tensor of at least permutation_workspace_bytes(...) bytes (allocated
    here when None)."""
    dev = _require_cuda(topk_ids)
    t, k = topk_ids.shape
    m_alloc = m_indices.shape[0]
    _check(topk_ids, "topk_ids", (torch.int32,), (t, k), dev)
    _check(m_indices, "m_indices", (torch.int32,), (m_alloc,), dev)
    _check(src_token, "src_token", (torch.int32,), (m_alloc,), dev)
    _check(row_of_entry, "row_of_entry", (torch.int32,), (t, k), dev)
    if workspace is None:
        workspace = torch.empty(max(permutation_workspace_bytes(t, k, num_experts), 4), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", (torch.uint8,), (workspace.numel(),), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_moe_build_permutation(topk_ids.data_ptr(), t, k, num_experts, m_alloc,
                                                   m_indices.data_ptr(), src_token.data_ptr(),
                                                   row_of_entry.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                                   _stream(dev))
    _lib.check(st, "fp8_moe_build_permutation")


def moe_build_permutation_noalloc(topk_ids, num_experts, m_indices, src_token, row_of_entry):
    """moe_build_permutation with the library's own scratch (no workspace, nothing allocated); calls
    that overlap on one device race on that scratch."""
    dev = _require_cuda(topk_ids)
    t, k = topk_ids.shape
    m_alloc = m_indices.shape[0]
    _check(topk_ids, "topk_ids", (torch.int32,), (t, k), dev)
    _check(m_indices, "m_indices", (torch.int32,), (m_alloc,), dev)
    _check(src_token, "src_token", (torch.int32,), (m_alloc,), dev)
    _check(row_of_entry, "row_of_entry", (torch.int32,), (t, k), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_moe_build_permutation_noalloc(topk_ids.data_ptr(), t, k, num_experts, m_alloc,
                                                           m_indices.data_ptr(), src_token.data_ptr(),
                                                           row_of_entry.data_ptr(), _stream(dev))
    _lib.check(st, "fp8_moe_build_permutation_noalloc")


def moe_gather_quant(x, src_token, a_out, a_scale_out):
    """Row r of a_out/a_scale_out: x[src_token[r]] quantised per 1x128 block (rows with -1 untouched).

    With ``src_token=None`` row r quantises token r (a_out holds at most num_tokens rows)."""
    dev = _require_cuda(x)
    t, h = x.shape
    m_alloc = a_out.shape[0] if src_token is None else src_token.shape[0]
    _check(x, "x", (torch.bfloat16,), (t, h), dev)
    if src_token is not None:
        _check(src_token, "src_token", (torch.int32,), (m_alloc,), dev)
    _check(a_out, "a_out", (torch.uint8, torch.float8_e4m3fn), (m_alloc, h), dev)
    _check(a_scale_out, "a_scale_out", (torch.float32,), (m_alloc, h // 128), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_moe_gather_quant(x.data_ptr(), None if src_token is None else src_token.data_ptr(),
                                              t, h, m_alloc, a_out.data_ptr(), a_scale_out.data_ptr(), _stream(dev))
    _lib.check(st, "fp8_moe_gather_quant")


def moe_silu_mul_quant(y, m_indices, a_out, a_scale_out):
    dev = _require_cuda(y)
    rows, two_i = y.shape
    inter = two_i // 2
    _check(y, "y", (torch.bfloat16,), (rows, 2 * inter), dev)
    _check(m_indices, "m_indices", (torch.int32,), (rows,), dev)
    _check(a_out, "a_out", (torch.uint8, torch.float8_e4m3fn), (rows, inter), dev)
    _check(a_scale_out, "a_scale_out", (torch.float32,), (rows, inter // 128), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_moe_silu_mul_quant(y.data_ptr(), m_indices.data_ptr(), rows, inter,
                                                a_out.data_ptr(), a_scale_out.data_ptr(), _stream(dev))
    _lib.check(st, "fp8_moe_silu_mul_quant")


def moe_fc1_silu_quant(a, a_scale, a_rows, w1, w1_scale, m_indices, q_out, q_scale_out, scale_major="K"):
    """fc1 and SiLU(gate)*up -> 1x128 E4M3 in one pass (rows of a read through a_rows, or a itself if None)."""
    dev = _require_cuda(a)
    rows_total, hidden = a.shape
    m = m_indices.shape[0]
    num_experts, two_inter, _ = w1.shape
    inter = two_inter // 2
    kb, nb = hidden // 128, two_inter // 128
    major = _major(scale_major)
    _check(a, "a", _FP8_DTYPES, (rows_total, hidden), dev)
    _check(a_scale, "a_scale", (torch.float32,), (rows_total, kb) if major == 0 else (kb, rows_total), dev)
    if a_rows is None:
        if rows_total != m:
            raise ValueError(f"without a_rows, a must have m = {m} rows")
    else:
        _check(a_rows, "a_rows", (torch.int32,), (m,), dev)
    _check(w1, "w1", _FP8_DTYPES, (num_experts, two_inter, hidden), dev)
    _check(w1_scale, "w1_scale", (torch.float32,), (num_experts, nb, kb) if major == 0 else (num_experts, kb, nb), dev)
    _check(m_indices, "m_indices", (torch.int32,), (m,), dev)
    _check(q_out, "q_out", (torch.uint8, torch.float8_e4m3fn), (m, inter), dev)
    _check(q_scale_out, "q_scale_out", (torch.float32,), (m, inter // 128), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_moe_fc1_silu_quant(_ptr(a), _ptr(a_scale), rows_total,
                                                None if a_rows is None else _ptr(a_rows), _ptr(w1), _ptr(w1_scale),
                                                _ptr(m_indices), _ptr(q_out), _ptr(q_scale_out), m, inter, hidden,
                                                num_experts, major, *_GRAN, _stream(dev))
    _lib.check(st, "fp8_moe_fc1_silu_quant")


def moe_combine(y, row_of_entry, topk_weights, out):
    """out (T, hidden) bf16 or fp16 = sum over slots of topk_weights * y[row_of_entry] (weight 1 when
    topk_weights is None)."""
    dev = _require_cuda(y)
    m_alloc, h = y.shape
    t, k = row_of_entry.shape
    _check(y, "y", (torch.bfloat16,), (m_alloc, h), dev)
    _check(row_of_entry, "row_of_entry", (torch.int32,), (t, k), dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", (torch.float32,), (t, k), dev)
    _check(out, "out", _OUT_DTYPES, (t, h), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_moe_combine(y.data_ptr(), row_of_entry.data_ptr(), _ptr(topk_weights), t, k, h,
                                         m_alloc, out.data_ptr(), _out_code(out), _stream(dev))
    _lib.check(st, "fp8_moe_combine")


def moe_ffn_fp8_block_scale(x, topk_ids, topk_weights, w1, s1, w2, s2, out=None, workspace=None,
                            fuse_activation=True):
    """Expert FFN: out (T, hidden) bf16. ``workspace`` (MoeWorkspace) keeps every intermediate.

    ``fuse_activation`` runs fc1 and SiLU-mul+requant as one pass (workspace.y1 is then not written);
    the result is bit-identical either way."""
    num_tokens, hidden = x.shape
    num_experts, two_inter, _ = w1.shape
    inter = two_inter // 2
    top_k = topk_ids.shape[1]
    if w2.shape != (num_experts, hidden, inter):
        raise ValueError(f"w2 has shape {tuple(w2.shape)}, expected {(num_experts, hidden, inter)}")
    ws = workspace or MoeWorkspace.allocate(num_tokens, top_k, num_experts, hidden, inter, x.device)
    if out is None:
        out = torch.empty((num_tokens, hidden), dtype=torch.bfloat16, device=x.device)
    moe_build_permutation(topk_ids, num_experts, ws.m_indices, ws.src_token, ws.row_of_entry, ws.perm_scratch)
    moe_gather_quant(x, None, ws.a1, ws.sa1)
    if fuse_activation:
        moe_fc1_silu_quant(ws.a1, ws.sa1, ws.src_token, w1, s1, ws.m_indices, ws.a2, ws.sa2)
    else:
        fp8_group_gemm_contiguous_gather(ws.a1, ws.sa1, ws.src_token, w1, s1, ws.m_indices, ws.y1)
        moe_silu_mul_quant(ws.y1, ws.m_indices, ws.a2, ws.sa2)
    fp8_group_gemm_contiguous(ws.a2, w2, ws.sa2, s2, ws.m_indices, ws.y2)
    moe_combine(ws.y2, ws.row_of_entry, topk_weights, out)
    return out


# ---- per-tensor FP8 expert FFN ----------------------------------------------------------------------


@dataclass
class MoePerTensorWorkspace:
    """Device buffers of one per-tensor expert-FFN call (allocated once, reused across calls)."""

    m_indices: torch.Tensor
    src_token: torch.Tensor
    row_of_entry: torch.Tensor
    perm_scratch: torch.Tensor  # the permutation's per-chunk expert counts
    a2: torch.Tensor  # fc2's E4M3 input, written by fc1's epilogue
    y2: torch.Tensor

    @staticmethod
    def allocate(num_tokens, top_k, num_experts, hidden, inter, device) -> "MoePerTensorWorkspace":
        m_alloc = default_m_alloc(num_tokens, top_k, num_experts)
        e = dict(device=device)
        return MoePerTensorWorkspace(
            m_indices=torch.empty(m_alloc, dtype=torch.int32, **e),
            src_token=torch.empty(m_alloc, dtype=torch.int32, **e),
            row_of_entry=torch.empty((num_tokens, top_k), dtype=torch.int32, **e),
            perm_scratch=torch.empty(max(permutation_workspace_bytes(num_tokens, top_k, num_experts), 4),
                                     dtype=torch.uint8, **e),
            a2=torch.empty((m_alloc, inter), dtype=torch.uint8, **e),
            y2=torch.empty((m_alloc, hidden), dtype=torch.bfloat16, **e),
        )

    @property
    def m_alloc(self) -> int:
        return self.m_indices.shape[0]


def fp8_group_gemm_contiguous_per_tensor(a, a_rows, b, b_dequant, m_indices, out):
    """out[i] = b_dequant[e] * (a[a_rows[i]] @ b[e].T) for rows with e = m_indices[i] >= 0 (a_rows None:
    row i of a); FP32 sum over k, bf16 or fp16 out."""
    dev = _require_cuda(a)
    rows_total, k = a.shape
    m = m_indices.shape[0]
    groups, n, _ = b.shape
    _check(a, "a", _FP8_DTYPES, (rows_total, k), dev)
    if a_rows is not None:
        _check(a_rows, "a_rows", (torch.int32,), (m,), dev)
    _check(b, "b", _FP8_DTYPES, (groups, n, k), dev)
    _check(b_dequant, "b_dequant", (torch.float32,), (groups,), dev)
    _check(m_indices, "m_indices", (torch.int32,), (m,), dev)
    _check(out, "out", _OUT_DTYPES, (m, n), dev)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_group_gemm_contiguous_per_tensor(_ptr(a), rows_total, _ptr(a_rows), _ptr(b),
                                                              _ptr(b_dequant), _ptr(m_indices), _ptr(out),
                                                              _out_code(out), m, n, k, groups, _stream(dev))
    _lib.check(st, "fp8_group_gemm_contiguous_per_tensor")
    return out


def moe_fc1_silu_quant_per_tensor(a, a_rows, w1, fc1_dequant, fc2_quant, m_indices, q_out):
    """q_out = E4M3(saturate(silu(gate) * up * fc2_quant)), gate/up = fc1_dequant[e] * (a[a_rows] @ w1[e].T)
    halves; fc2_quant holds one value or one per expert."""
    dev = _require_cuda(a)
    rows_total, hidden = a.shape
    m = m_indices.shape[0]
    num_experts, two_inter, _ = w1.shape
    inter = two_inter // 2
    _check(a, "a", _FP8_DTYPES, (rows_total, hidden), dev)
    if a_rows is not None:
        _check(a_rows, "a_rows", (torch.int32,), (m,), dev)
    _check(w1, "w1", _FP8_DTYPES, (num_experts, 2 * inter, hidden), dev)
    _check(fc1_dequant, "fc1_dequant", (torch.float32,), (num_experts,), dev)
    if fc2_quant.numel() not in (1, num_experts):
        raise ValueError(f"fc2_quant must hold 1 or {num_experts} values, got {fc2_quant.numel()}")
    _check(fc2_quant, "fc2_quant", (torch.float32,), tuple(fc2_quant.shape), dev)
    _check(m_indices, "m_indices", (torch.int32,), (m,), dev)
    _check(q_out, "q_out", _FP8_DTYPES, (m, inter), dev)
    per_expert = int(fc2_quant.numel() == num_experts and num_experts > 1)
    with torch.cuda.device(dev):
        st = _lib.load().fp8_moe_fc1_silu_quant_per_tensor(_ptr(a), rows_total, _ptr(a_rows), _ptr(w1),
                                                           _ptr(fc1_dequant), _ptr(fc2_quant), per_expert,
                                                           _ptr(m_indices), _ptr(q_out), m, inter, hidden,
                                                           num_experts, _stream(dev))
    _lib.check(st, "fp8_moe_fc1_silu_quant_per_tensor")
    return q_out


def moe_ffn_fp8_per_tensor(x_fp8, topk_ids, w1, w2, fc1_dequant, fc2_quant, fc2_dequant, fc1_input_dequant=None,
                           topk_weights=None, out=None, out_dtype=torch.bfloat16, workspace=None):
    """Per-tensor FP8 expert FFN with the argument list of the flashinfer-rs README (section "API
    Example: Fused MoE FP8 (cudarc)", per-tensor FP8 mode): x_fp8 (T, hidden) E4M3 tokens, topk_ids
    (T, top_k) int32, w1 (E, 2*inter, hidden) gate then up, w2 (E, hidden, inter), fc1_dequant (E,),
    fc2_quant (1 or E,), fc2_dequant (E,), out (T, hidden) bf16 or fp16. ``fc1_input_dequant`` (the
    tokens' own scale, already a factor of fc1_dequant) is accepted and not applied; the README's call
    takes no routing weights, so the expert outputs are summed with weight 1 unless ``topk_weights``
    is given. Four library calls: permutation -> fc1 + SiLU-mul + quantise -> fc2 -> combine."""
    num_tokens, hidden = x_fp8.shape
    num_experts, two_inter, _ = w1.shape
    inter = two_inter // 2
    top_k = topk_ids.shape[1]
    if w2.shape != (num_experts, hidden, inter):
        raise ValueError(f"w2 has shape {tuple(w2.shape)}, expected {(num_experts, hidden, inter)}")
    ws = workspace or MoePerTensorWorkspace.allocate(num_tokens, top_k, num_experts, hidden, inter, x_fp8.device)
    if out is None:
        out = torch.empty((num_tokens, hidden), dtype=out_dtype, device=x_fp8.device)
    moe_build_permutation(topk_ids, num_experts, ws.m_indices, ws.src_token, ws.row_of_entry, ws.perm_scratch)
    moe_fc1_silu_quant_per_tensor(x_fp8, ws.src_token, w1, fc1_dequant, fc2_quant, ws.m_indices, ws.a2)
    fp8_group_gemm_contiguous_per_tensor(ws.a2, None, w2, fc2_dequant, ws.m_indices, ws.y2)
    moe_combine(ws.y2, ws.row_of_entry, topk_weights, out)
    return out
