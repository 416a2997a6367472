"""MI355X-native FP8 (E4M3) groupwise-scaled NT GEMM for MoE experts.

All computation happens in libfp8g.so (hand-written HIP kernels for gfx950 behind a C ABI declared
in include/fp8g.h); this package only marshals torch tensors into that ABI. Importing it does not
touch the GPU; the first call loads the library and fails loudly if it has not been built.
"""

from ._lib import Fp8gError, Fp8gInvalidArgument, Fp8gNotSupported, LIB_PATH, load  # noqa: F401
from .gemm import (  # noqa: F401
    batch_deepgemm_fp8_nt_groupwise,
    bmm_fp8,
    fp8_bmm,
    fp8_batch_gemm_masked,
    fp8_gemm_nt_groupwise,
    fp8_gemm_nt_groupwise_fp8_out,
    fp8_group_gemm_contiguous,
    fp8_group_gemm_contiguous_gather,
    gemm_fp8_nt_groupwise,
    group_deepgemm_fp8_nt_groupwise,
)
from .moe import (  # noqa: F401
    MoePerTensorWorkspace,
    MoeWorkspace,
    default_m_alloc,
    moe_build_permutation,
    moe_build_permutation_noalloc,
    fp8_group_gemm_contiguous_per_tensor,
    moe_combine,
    moe_fc1_silu_quant,
    moe_fc1_silu_quant_per_tensor,
    moe_ffn_fp8_block_scale,
    moe_ffn_fp8_per_tensor,
    moe_gather_quant,
    moe_silu_mul_quant,
    permutation_workspace_bytes,
)
from .quant import fp8_quantize_1x128, fused_add_rmsnorm_fp8_block_quant  # noqa: F401
