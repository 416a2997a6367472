"""ctypes loader for libfp8g.so and status -> exception mapping.

The library must have been built in-tree (``python -m moe_expert_matmul_amd.build``); there is no
fallback of any kind when it is missing.
"""

from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libfp8g.so")

OK, INVALID_ARGUMENT, NOT_SUPPORTED, HIP_ERROR, INTERNAL = 0, 1, 2, 3, 4
OUT_BF16, OUT_FP16 = 0, 1
SCALE_K_MAJOR, SCALE_MN_MAJOR = 0, 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

# Exported entry points and their argument types, in the order include/fp8g.h declares them.
SIGNATURES = {
    "fp8g_last_error": ([], ctypes.c_char_p),
    "fp8g_version": ([], _I32),
    "fp8g_clock_probe": ([_P, _I64, _P], _I32),
    "fp8g_gemm_clock_record": ([_P], _I32),
    "fp8g_wall_clock_khz": ([], _I64),
    "fp8_gemm_nt_groupwise": ([_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P], _I32),
    "fp8_gemm_nt_groupwise_fp8_out": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P], _I32),
    "fp8_group_gemm_contiguous": ([_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P],
                                  _I32),
    "fp8_group_gemm_contiguous_gather": ([_P, _P, _I64, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _I32, _I32,
                                          _I32, _I32, _P], _I32),
    "fp8_batch_gemm_masked": ([_P, _P, _P, _P, _P, _I64, _P, _I32, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32,
                               _P], _I32),
    "fp8_bmm": ([_P, _P, _P, _I32, _P, _I32, _P, _I32, _I64, _I64, _I64, _I64, _P], _I32),
    "fp8_quantize_1x128": ([_P, _I64, _I64, _P, _P, _I32, _P], _I32),
    "fp8_fused_add_rmsnorm_quant": ([_P, _P, _P, _P, _P, _P, ctypes.c_float, _I64, _I64, _I32, _P], _I32),
    "fp8_moe_permutation_workspace_size": ([_I64, _I64, _I64], _I64),
    "fp8_moe_build_permutation": ([_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _I64, _P], _I32),
    "fp8_moe_build_permutation_noalloc": ([_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P], _I32),
    "fp8_moe_gather_quant": ([_P, _P, _I64, _I64, _I64, _P, _P, _P], _I32),
    "fp8_moe_silu_mul_quant": ([_P, _P, _I64, _I64, _P, _P, _P], _I32),
    "fp8_moe_fc1_silu_quant": ([_P, _P, _I64, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32,
                                _P], _I32),
    "fp8_moe_combine": ([_P, _P, _P, _I64, _I64, _I64, _I64, _P, _I32, _P], _I32),
    "fp8_group_gemm_contiguous_per_tensor": ([_P, _I64, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _P], _I32),
    "fp8_moe_fc1_silu_quant_per_tensor": ([_P, _I64, _P, _P, _P, _P, _I32, _P, _P, _I64, _I64, _I64, _I64, _P], _I32),
}


class Fp8gError(RuntimeError):
    """A libfp8g call failed; ``status`` is the fp8g_status_t value."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Fp8gNotSupported(Fp8gError, NotImplementedError):
    pass


class Fp8gInvalidArgument(Fp8gError, ValueError):
    pass


_lib = None
POISON_LIB_PATH = os.path.join(_PKG_DIR, "libfp8g_poison_lds.so")


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    for name, (argtypes, restype) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return lib


def load_poison_lds() -> ctypes.CDLL:
    """The debug build whose GEMM kernels start with NaN-poisoned LDS (for the pipeline tests)."""
    if not os.path.exists(POISON_LIB_PATH):
        raise ImportError(f"{POISON_LIB_PATH} is missing: build with `python -m moe_expert_matmul_amd.build`")
    return _bind(ctypes.CDLL(POISON_LIB_PATH))


def load() -> ctypes.CDLL:
    """Load libfp8g.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_expert_matmul_amd.build` "
                              "(the HIP library is the only implementation)")
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def check(status: int, what: str) -> None:
    if status == OK:
        return
    msg = f"{what}: {load().fp8g_last_error().decode(errors='replace')}"
    if status == INVALID_ARGUMENT:
        raise Fp8gInvalidArgument(status, msg)
    if status == NOT_SUPPORTED:
        raise Fp8gNotSupported(status, msg)
    raise Fp8gError(status, msg)
