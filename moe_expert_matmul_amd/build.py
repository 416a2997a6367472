"""Build libfp8g.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m moe_expert_matmul_amd.build

Each source is compiled to an object in parallel, then linked into ``libfp8g.so`` beside this file.
Packed FP32 instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libfp8g.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
POISON_LIB_PATH = os.path.join(PKG_DIR, "libfp8g_poison_lds.so")  # debug build, NaN-poisoned LDS
SOURCES = ["api.hip", "gemm.hip", "moe.hip", "quant.hip", "clock.hip"]

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extra compiler flags (none at present).
SOURCE_FLAGS: dict = {}
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-command-line-argument",
                "-fvisibility=hidden",
                "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libfp8g.so")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature flag; that warning is expected
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if proc.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return lines


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for lines in ex.map(_run, jobs):
            if verbose:
                print("\n".join(lines))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    # debug build: the GEMM kernels start with NaN-poisoned LDS (the other objects are shared)
    poison_obj = os.path.join(BUILD_DIR, "gemm_poison.o")
    _run([hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, "-DFP8G_POISON_LDS=1", "-c", os.path.join(CSRC, "gemm.hip"), "-o",
          poison_obj])
    others = [o for o in objs if os.path.basename(o) != "gemm.o"]
    tmp = POISON_LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", poison_obj, *others, "-o", tmp])
    os.replace(tmp, POISON_LIB_PATH)
    return LIB_PATH


# Host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; device code untouched
# (each -fsanitize= applies to the host pass only). The library is linked without a sanitizer
# runtime: the program that loads it must be built with the same sanitizers, which provides one.
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build_host_sanitized(out_dir: str) -> str:
    """Compile every source with host-side ASan and UBSan into out_dir/libfp8g.so (for CPU tests of
    the validation layer); returns its path."""
    hipcc = _hipcc()
    os.makedirs(out_dir, exist_ok=True)
    objs, jobs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, *HOST_SANITIZE_FLAGS, "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        list(ex.map(_run, jobs))
    lib = os.path.join(out_dir, LIB_NAME)
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", lib])
    return lib


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
