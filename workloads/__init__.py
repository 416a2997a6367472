"""Seeded synthetic inputs for the FP8 groupwise GEMM forms and the MoE expert FFN.

Shared by the tests, the smoke check and the benchmark, on both sides of every comparison: the GPU
path and the CPU oracle read the very same bytes. This module holds input synthesis only -- random
draws, the 1x128 / 128x128 block quantisation that turns N(0,1) data into E4M3 codes with
scale = amax/448 (through torch's own float8_e4m3fn cast), the expert-size draw and the router --
and none of the GEMM's arithmetic.

Workloads (all seed-fixed):
  plain        A (m,k), B (n,k) ~ N(0,1) float32, A quantised per 1x128 block, B per 128x128
               block, K-major FP32 scales.
  contiguous   expert sizes ~ multinomial(rows, p_e ~ (e+1)^-s) (Zipf, s = 1.1), rows sorted by
               expert, each expert region padded to a multiple of 128 with m_indices = -1.
  masked       masked_m ~ uniform integers on [0, max_m], A (G,max_m,k), B (G,n,k).
  moe          router logits ~ N(0,1) (T,E); p = softmax; top-k by p (ties -> lower expert index);
               weights = p at the chosen experts (not renormalised); X ~ N(0,1) in BF16;
               W1 (E, 2I, H) and W2 (E, H, I) ~ N(0,1) quantised per 128x128 block.
  moe (per-tensor)  x, W1, W2 ~ N(0,1) as E4M3 with one scale per tensor (per expert for the
               weights); fixed activation scale 16 * hidden / 448.
  bmm          A (B,m,k), B (B,k,n) ~ N(0,1) quantised with amax/448 per row of A / per column of B
               (channelwise) or per tensor.
  norm         add-RMSNorm input ~ N(0,1), residual ~ N(0,1) times a per-row log-uniform scale,
               weight ~ U(0.5, 1.5), all BF16.

Small structural draws (sizes, counts, logits) use numpy's default_rng(seed); bulk tensors use a
torch.Generator seeded with the same seed on the target device, so that full-size inputs are
produced where they are used. The same (seed, device) always gives the same bytes.
"""

from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0
BLOCK = 128


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, gen, device) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def quantize_blocks(x: torch.Tensor, block_rows: int, block_cols: int):
    """Quantise the last two dims of float32 ``x`` in (block_rows x block_cols) blocks.

    Returns (codes uint8 same shape as x, scales float32 of shape (..., R/block_rows, C/block_cols)).
    scale = amax/448 per block (1 for an all-zero block); codes = float8_e4m3fn(x / scale).
    """
    *lead, rows, cols = x.shape
    if rows % block_rows or cols % block_cols:
        raise ValueError("shape not divisible by the block")
    xb = x.reshape(*lead, rows // block_rows, block_rows, cols // block_cols, block_cols)
    amax = xb.abs().amax(dim=(-3, -1))
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (xb / scale[..., :, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(x.shape).contiguous(), scale.contiguous()


def _quantized_matrix(shape, block_rows, gen, device):
    x = _normal(shape, gen, device)
    codes, scales = quantize_blocks(x, block_rows, BLOCK)
    del x
    return codes, scales


def plain(m: int, n: int, k: int, seed: int = 0, device="cpu"):
    """Plain form inputs: a (m,k), b (n,k) E4M3 codes; a_scale (m,k/128), b_scale (ceil(n/128),k/128).
    When n is not a multiple of 128, b is drawn and quantised with whole 128-row blocks and cut to
    its first n rows (the last block's scale then covers its n % 128 remaining rows)."""
    g = _gen(seed, device)
    a, sa = _quantized_matrix((m, k), 1, g, device)
    n_pad = -(-n // BLOCK) * BLOCK
    b, sb = _quantized_matrix((n_pad, k), BLOCK, g, device)
    if n_pad != n:
        b = b[:n].contiguous()
    return dict(a=a, b=b, a_scale=sa, b_scale=sb, m=m, n=n, k=k)


def zipf_counts(num_groups: int, rows: int, s: float, seed: int) -> np.ndarray:
    p = np.arange(1, num_groups + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return np.random.default_rng(seed).multinomial(rows, p)


def contiguous_layout(counts) -> np.ndarray:
    """m_indices for experts of the given sizes, each region padded to a multiple of 128."""
    parts = []
    for e, c in enumerate(np.asarray(counts)):
        padded = (int(c) + BLOCK - 1) // BLOCK * BLOCK
        parts.append(np.concatenate([np.full(int(c), e, np.int32), np.full(padded - int(c), -1, np.int32)]))
    return np.concatenate(parts) if parts else np.zeros(0, np.int32)


def contiguous(num_groups: int = 32, rows: int = 8192, n: int = 4096, k: int = 7168,
               zipf_s: float = 1.1, seed: int = 0, device="cpu", counts=None):
    """Contiguous grouped inputs. ``counts`` overrides the Zipf draw (for edge cases)."""
    if counts is None:
        counts = zipf_counts(num_groups, rows, zipf_s, seed)
    counts = np.asarray(counts, dtype=np.int64)
    m_indices = contiguous_layout(counts)
    m = m_indices.size
    g = _gen(seed, device)
    a, sa = _quantized_matrix((m, k), 1, g, device)
    b, sb = _quantized_matrix((num_groups, n, k), BLOCK, g, device)
    return dict(a=a, b=b, a_scale=sa, b_scale=sb,
                m_indices=torch.from_numpy(m_indices).to(device), counts=counts,
                m=m, n=n, k=k, num_groups=num_groups)


def masked(num_groups: int = 16, max_m: int = 256, n: int = 4096, k: int = 7168,
           expected_m: int = 128, seed: int = 0, device="cpu", masked_m=None):
    """Masked batched inputs. ``masked_m`` overrides the uniform draw (for edge cases)."""
    if masked_m is None:
        masked_m = np.random.default_rng(seed).integers(0, max_m + 1, num_groups)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    g = _gen(seed, device)
    a, sa = _quantized_matrix((num_groups, max_m, k), 1, g, device)
    b, sb = _quantized_matrix((num_groups, n, k), BLOCK, g, device)
    return dict(a=a, b=b, a_scale=sa, b_scale=sb, masked_m=torch.from_numpy(masked_m).to(device),
                expected_m=int(expected_m), num_groups=num_groups, max_m=max_m, n=n, k=k)


def router(num_tokens: int, num_experts: int, top_k: int, seed: int):
    """Softmax top-k routing of N(0,1) logits: (ids int32 (T,k), weights float32 (T,k))."""
    logits = np.random.default_rng(seed).standard_normal((num_tokens, num_experts))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :top_k]
    w = np.take_along_axis(p, ids, axis=1)
    return ids.astype(np.int32), w.astype(np.float32)


def moe(num_tokens: int = 4096, hidden: int = 7168, num_experts: int = 64, top_k: int = 8,
        inter: int = 2048, seed: int = 0, device="cpu"):
    """Expert-FFN inputs: x (T,H) bf16, routing, W1 (E,2I,H)/W2 (E,H,I) codes with 128x128 scales."""
    ids, w = router(num_tokens, num_experts, top_k, seed)
    g = _gen(seed, device)
    x = _normal((num_tokens, hidden), g, device).to(torch.bfloat16)
    w1, s1 = _quantized_matrix((num_experts, 2 * inter, hidden), BLOCK, g, device)
    w2, s2 = _quantized_matrix((num_experts, hidden, inter), BLOCK, g, device)
    return dict(x=x, topk_ids=torch.from_numpy(ids).to(device), topk_weights=torch.from_numpy(w).to(device),
                w1=w1, s1=s1, w2=w2, s2=s2, num_tokens=num_tokens, hidden=hidden,
                num_experts=num_experts, top_k=top_k, inter=inter)


def moe_per_tensor(num_tokens: int = 4096, hidden: int = 7168, num_experts: int = 64, top_k: int = 8,
                   inter: int = 2048, seed: int = 0, device="cpu"):
    """Per-tensor FP8 expert-FFN inputs: x ~ N(0,1) as E4M3 codes with one scale amax/448 over the
    tensor, W1/W2 ~ N(0,1) with one scale per expert, the router of ``moe``. The dequantisation
    scales are fc1_dequant[e] = s_x * s_w1[e] and fc2_dequant[e] = s_act * s_w2[e], with a fixed
    activation scale s_act = 16 * hidden / 448 (h = silu(g) * u has a spread of about hidden for
    unit-variance codes; larger values saturate) and fc2_quant = 1 / s_act."""
    ids, w = router(num_tokens, num_experts, top_k, seed)
    g = _gen(seed, device)

    def quant(t, dims):
        amax = t.abs().amax(dim=dims, keepdim=True)
        scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        return (t / scale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), scale.reshape(-1)

    x, sx = quant(_normal((num_tokens, hidden), g, device), (0, 1))
    w1, sw1 = quant(_normal((num_experts, 2 * inter, hidden), g, device), (1, 2))
    w2, sw2 = quant(_normal((num_experts, hidden, inter), g, device), (1, 2))
    s_act = 16.0 * hidden / E4M3_MAX
    return dict(x=x, topk_ids=torch.from_numpy(ids).to(device), topk_weights=torch.from_numpy(w).to(device),
                w1=w1, w2=w2, fc1_dequant=(sx * sw1).float().contiguous(),
                fc2_quant=torch.tensor([1.0 / s_act], dtype=torch.float32, device=device),
                fc2_dequant=(s_act * sw2).float().contiguous(), fc1_input_dequant=sx.float().contiguous(),
                num_tokens=num_tokens, hidden=hidden, num_experts=num_experts, top_k=top_k, inter=inter)


def bmm(batch: int, m: int, n: int, k: int, channel_a: bool, channel_b: bool, seed: int = 0, device="cpu"):
    """Batched FP8 GEMM inputs: A (batch,m,k), B (batch,k,n) ~ N(0,1) as E4M3 codes, with scale =
    amax/448 per row of A / per column of B (channelwise, rank-3 scales (batch,m,1) / (batch,1,n)) or
    over the whole tensor (tensorwise, 0-d scales)."""
    g = _gen(seed, device)
    x = _normal((batch, m, k), g, device)
    y = _normal((batch, k, n), g, device)

    def quant(t, dims):
        amax = t.abs().amax(dim=dims, keepdim=True)
        scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        codes = (t / scale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
        return codes, scale.contiguous()

    a, sa = quant(x, (2,) if channel_a else (0, 1, 2))
    b, sb = quant(y, (1,) if channel_b else (0, 1, 2))
    if not channel_a:
        sa = sa.reshape(())
    if not channel_b:
        sb = sb.reshape(())
    return dict(a=a, b=b, a_scale=sa, b_scale=sb, batch=batch, m=m, n=n, k=k)


def norm(rows: int = 4096, hidden: int = 7168, seed: int = 0, device="cpu"):
    """Add-RMSNorm inputs: input ~ N(0,1), residual ~ N(0,1) * row scale (row scales log-uniform on
    [1/8, 8], a residual stream whose rows differ in size), weight ~ U(0.5, 1.5); all BF16."""
    g = _gen(seed, device)
    row_scale = torch.from_numpy(np.exp2(np.random.default_rng(seed).uniform(-3, 3, (rows, 1)))).float().to(device)
    inp = _normal((rows, hidden), g, device).to(torch.bfloat16)
    res = (_normal((rows, hidden), g, device) * row_scale).to(torch.bfloat16)
    w = (torch.rand(hidden, generator=g, device=device) + 0.5).to(torch.bfloat16)
    return dict(input=inp, residual=res, weight=w, rows=rows, hidden=hidden)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor; bf16 comes back as its uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
