"""C-ABI checks that need no GPU: the library loads, exports every entry point the header declares,
and rejects bad arguments on the host before touching a device."""

import ctypes
import os
import re
import subprocess

import pytest

from moe_expert_matmul_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8g.h")


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"FP8G_API\s+[\w\s\*]+?\b(\w+)\s*\(", text))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfp8g.so is not built (run `python -m moe_expert_matmul_amd.build`)")
    return _lib.load()


def test_header_declares_the_three_gemm_forms_and_the_moe_steps():
    names = _declared()
    assert {"fp8_gemm_nt_groupwise", "fp8_group_gemm_contiguous", "fp8_batch_gemm_masked",
            "fp8g_last_error", "fp8_moe_build_permutation", "fp8_moe_gather_quant",
            "fp8_moe_silu_mul_quant", "fp8_moe_combine"} <= names
    assert names == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == _declared(), exported ^ _declared()


def test_version(lib):
    assert lib.fp8g_version() >= 100


GRAN = (1, 128, 128)
P = ctypes.c_void_p(16)  # a non-null, 16-byte aligned dummy (never dereferenced: validation fails first)


def _status(fn, *args):
    st = fn(*args)
    return st, _lib.load().fp8g_last_error().decode()


def test_plain_rejects_k_not_multiple_of_128(lib):
    st, msg = _status(lib.fp8_gemm_nt_groupwise, P, P, P, P, P, 0, 4, 128, 100, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "k (100)" in msg


def test_n_tails_only_in_the_plain_form(lib):
    # the plain form takes any n (validation passes; without a GPU the call stops at the device check)
    st, msg = _status(lib.fp8_gemm_nt_groupwise, P, P, P, P, P, 0, 4, 200, 128, 0, *GRAN, None)
    assert "n (200)" not in msg and st != _lib.OK
    st, msg = _status(lib.fp8_group_gemm_contiguous, P, P, P, P, P, P, 0, 128, 200, 128, 2, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "n (200)" in msg
    st, msg = _status(lib.fp8_batch_gemm_masked, P, P, P, P, P, 1, P, 0, 2, 64, 200, 128, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "n (200)" in msg


def test_fp8_output_needs_a_scale(lib):
    st, msg = _status(lib.fp8_gemm_nt_groupwise_fp8_out, P, P, P, P, P, None, 4, 128, 128, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "output_scale" in msg
    assert lib.fp8_gemm_nt_groupwise_fp8_out(None, None, None, None, None, P, 0, 128, 128, 0, *GRAN, None) == _lib.OK


def test_plain_rejects_negative_sizes_and_bad_layout(lib):
    assert lib.fp8_gemm_nt_groupwise(P, P, P, P, P, 0, -1, 128, 128, 0, *GRAN, None) == _lib.INVALID_ARGUMENT
    st, msg = _status(lib.fp8_gemm_nt_groupwise, P, P, P, P, P, 0, 4, 128, 128, 7, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "scale_major" in msg


def test_unsupported_granularity_is_not_supported(lib):
    st, msg = _status(lib.fp8_gemm_nt_groupwise, P, P, P, P, P, 0, 4, 128, 128, 0, 1, 64, 128, None)
    assert st == _lib.NOT_SUPPORTED and "granularity" in msg
    st, _ = _status(lib.fp8_group_gemm_contiguous, P, P, P, P, P, P, 0, 128, 128, 128, 2, 0, 128, 128, 128, None)
    assert st == _lib.NOT_SUPPORTED


def test_null_and_misaligned_pointers_are_rejected(lib):
    st, msg = _status(lib.fp8_gemm_nt_groupwise, None, P, P, P, P, 0, 4, 128, 128, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "non-null" in msg
    st, msg = _status(lib.fp8_gemm_nt_groupwise, P, P, P, P, None, 0, 4, 128, 0, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "out must be non-null" in msg
    st, msg = _status(lib.fp8_gemm_nt_groupwise, ctypes.c_void_p(17), P, P, P, P, 0, 4, 128, 128, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "aligned" in msg


def test_empty_problems_are_successful_no_ops(lib):
    assert lib.fp8_gemm_nt_groupwise(None, None, None, None, None, 0, 0, 128, 128, 0, *GRAN, None) == _lib.OK
    assert lib.fp8_gemm_nt_groupwise(None, None, None, None, None, 0, 5, 0, 128, 0, *GRAN, None) == _lib.OK
    assert lib.fp8_batch_gemm_masked(None, None, None, None, None, 0, None, 0, 0, 64, 128, 128, 0, *GRAN, None) == _lib.OK
    assert lib.fp8_group_gemm_contiguous(None, None, None, None, None, None, 0, 0, 128, 128, 4, 0, *GRAN, None) == _lib.OK
    assert lib.fp8g_last_error() == b""


def test_contiguous_requires_128_row_multiple(lib):
    st, msg = _status(lib.fp8_group_gemm_contiguous, P, P, P, P, P, P, 0, 100, 128, 128, 2, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "multiple of 128" in msg


def test_bad_out_dtype_is_rejected(lib):
    st, msg = _status(lib.fp8_gemm_nt_groupwise, P, P, P, P, P, 2, 4, 128, 128, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "out_dtype" in msg
    st, msg = _status(lib.fp8_batch_gemm_masked, P, P, P, P, P, 1, P, 7, 2, 64, 128, 128, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT and "out_dtype" in msg


def test_masked_rejects_negative_expected_m(lib):
    st, _ = _status(lib.fp8_batch_gemm_masked, P, P, P, P, P, -1, P, 0, 2, 64, 128, 128, 0, *GRAN, None)
    assert st == _lib.INVALID_ARGUMENT


def test_moe_steps_validate_sizes(lib):
    # m_alloc too small for 4 tokens x 2 slots over 3 experts (needs 128 * ceil((8 + 381) / 128) = 512)
    st, msg = _status(lib.fp8_moe_build_permutation, P, 4, 2, 3, 256, P, P, P, P, 1 << 20, None)
    assert st == _lib.INVALID_ARGUMENT and "m_alloc" in msg
    # the workspace holds one int32 per (chunk of 1024 entries, expert)
    assert lib.fp8_moe_permutation_workspace_size(4, 2, 3) == 12
    assert lib.fp8_moe_permutation_workspace_size(4096, 8, 64) == 32 * 64 * 4
    assert lib.fp8_moe_permutation_workspace_size(0, 8, 64) == 0
    assert lib.fp8_moe_permutation_workspace_size(4, 2, 1025) == -1
    st, msg = _status(lib.fp8_moe_build_permutation, P, 4, 2, 3, 512, P, P, P, P, 11, None)
    assert st == _lib.INVALID_ARGUMENT and "workspace" in msg
    st, _ = _status(lib.fp8_moe_gather_quant, P, P, 4, 100, 128, P, P, None)
    assert st == _lib.INVALID_ARGUMENT
    st, _ = _status(lib.fp8_moe_silu_mul_quant, P, P, 128, 100, P, P, None)
    assert st == _lib.INVALID_ARGUMENT
    st, _ = _status(lib.fp8_moe_combine, P, P, P, 4, 65, 128, 128, P, 0, None)
    assert st == _lib.INVALID_ARGUMENT


def test_error_message_is_cleared_by_the_next_successful_call(lib):
    lib.fp8_gemm_nt_groupwise(P, P, P, P, P, 0, 4, 128, 100, 0, *GRAN, None)
    assert lib.fp8g_last_error() != b""
    assert lib.fp8_gemm_nt_groupwise(None, None, None, None, None, 0, 0, 128, 128, 0, *GRAN, None) == _lib.OK
    assert lib.fp8g_last_error() == b""


def test_python_binding_refuses_cpu_tensors():
    import torch
    from moe_expert_matmul_amd import gemm_fp8_nt_groupwise
    a = torch.zeros((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        gemm_fp8_nt_groupwise(a, a, torch.ones(4, 1), torch.ones(1, 1))


def test_producers_validate_arguments(lib):
    st, msg = _status(lib.fp8_quantize_1x128, P, 4, 100, P, P, 0, None)
    assert st == _lib.INVALID_ARGUMENT and "cols (100)" in msg
    assert lib.fp8_quantize_1x128(None, 0, 256, None, None, 0, None) == _lib.OK
    f = lib.fp8_fused_add_rmsnorm_quant
    Q = ctypes.c_void_p(32)
    st, msg = _status(f, P, P, P, P, Q, P, 1e-6, 4, 100, 0, None)
    assert st == _lib.INVALID_ARGUMENT and "hidden (100)" in msg
    st, msg = _status(f, P, P, P, Q, Q, P, 1e-6, 4, 128, 0, None)
    assert st == _lib.INVALID_ARGUMENT and "alias" in msg
    st, msg = _status(f, P, P, P, P, Q, P, -1.0, 4, 128, 0, None)
    assert st == _lib.INVALID_ARGUMENT and "eps" in msg
    st, msg = _status(f, P, P, P, P, Q, P, float("nan"), 4, 128, 0, None)
    assert st == _lib.INVALID_ARGUMENT and "eps" in msg
    st, msg = _status(f, P, P, P, P, Q, P, 1e-6, 4, 128, 3, None)
    assert st == _lib.INVALID_ARGUMENT and "scale_major" in msg
    assert f(None, None, None, None, None, None, 1e-6, 0, 7168, 0, None) == _lib.OK


def test_missing_library_fails_loudly(tmp_path):
    # The package has no CPU fallback: without libfp8g.so the first call raises.
    code = ("import moe_expert_matmul_amd as m, moe_expert_matmul_amd._lib as L\n"
            f"L.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
            "try:\n    L.load()\nexcept ImportError as e:\n    print('raised', e)\n")
    r = subprocess.run(["python3", "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in r.stdout and "absent.so" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run(["python3", os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_header_and_library_work_from_plain_c(tmp_path):
    """The boundary is a C ABI: a C program compiled against include/fp8g.h and linked with
    libfp8g.so validates arguments and reports errors without Python."""
    exe = tmp_path / "abi_from_c"
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    build = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", lib_dir, "-lfp8g",
                            f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.returncode, run.stdout, run.stderr)


def test_validation_layer_under_host_asan_and_ubsan(tmp_path):
    """The library rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer on its host code, driven
    through every entry point's validation and error paths from C (no GPU is touched); any sanitizer
    report fails the run."""
    from moe_expert_matmul_amd import build as _build
    lib_dir = tmp_path / "hostsan"
    _build.build_host_sanitized(str(lib_dir))
    clang = os.path.join(os.path.dirname(os.path.realpath(_build._hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    exe = tmp_path / "validation_under_sanitizers"
    build = subprocess.run([clang, "-std=c99", "-Wall", "-Werror", "-g", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c", "validation_under_sanitizers.c"), "-L", str(lib_dir),
                            "-lfp8g", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and run.stdout.startswith("ok"), (run.returncode, run.stdout, run.stderr[-3000:])
