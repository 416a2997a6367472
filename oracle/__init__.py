"""CPU oracle for the FP8 (E4M3) groupwise-scaled NT GEMM and the MoE expert FFN built on it.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the HIP library and its
Python binding in ``moe_expert_matmul_amd``) never imports, calls or links anything here, and this
package imports nothing from the product path: the two share no code, tables or constants.

What it computes follows the MATE FlashInfer-API page
(mate-docs.mthreads.com/latest/api/flashinfer.html, section "GEMM": ``gemm_fp8_nt_groupwise``,
``group_deepgemm_fp8_nt_groupwise``, ``batch_deepgemm_fp8_nt_groupwise``) and, for the expert FFN,
the fused-MoE API of the flashinfer-rs README (section "API Example: Fused MoE FP8 (cudarc)",
DeepSeek FP8 block-scale mode).

Arithmetic: E4M3 codes are decoded exactly from their bit fields, products are summed per 128-wide
K block in float64 (exact in any order, because every block sum is an integer multiple of 2^-18
below 2^43), and the per-block scales are applied in float64. Steps whose result the GPU decides in
FP32 (the 1x128 quantiser's scale and its division) are taken in float32 here as well.

Modules:
  e4m3  -- bit-level E4M3FN decode table and round-to-nearest-even encoder
  bf16  -- round-to-nearest-even float -> bfloat16 encoder
  gemm  -- plain, contiguous-grouped and masked-batched groupwise GEMM references
  moe   -- the expert-FFN stages (1x128 quantiser, permutation, SiLU-mul, weighted combine)
  bmm   -- batched FP8 GEMM with per-tensor or per-channel scales (bmm_fp8 of the MATE page)
  norm  -- fused add-RMSNorm with 1x128 FP8 quantisation (section "norm" of the MATE page)
"""

from . import e4m3, bf16, gemm, moe, norm, bmm  # noqa: F401
