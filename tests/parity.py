"""Helpers shared by the GPU parity tests: the tolerance check and host copies."""

from __future__ import annotations

import sys

import numpy as np
import torch

import workloads
from oracle import bf16

# |gpu - ref| <= REL * |ref| + ABS_RMS * rms(ref) on every valid output element, rms taken over all
# valid elements of the call. FP32 accumulation of 128-term blocks and the final BF16 rounding
# (relative error <= 2^-9 ~ 2e-3) stay well inside it.
REL = 8e-3
ABS_RMS = 1e-3


def say(*args):
    """Print a progress line that names the case before a GPU step (flushed at once)."""
    print("[case]", *args, file=sys.stderr, flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    return workloads.to_numpy(t)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    """float64 values of a BF16 device tensor."""
    return bf16.from_bf16_bits(workloads.to_numpy(t))


def assert_within_tolerance(gpu: np.ndarray, ref: np.ndarray, what: str, rms=None) -> None:
    """``ref`` holds NaN where the output is unspecified; those entries are not compared."""
    valid = ~np.isnan(ref)
    assert valid.any(), f"{what}: nothing to compare"
    if rms is None:
        rms = float(np.sqrt(np.mean(ref[valid] ** 2)))
    err = np.abs(gpu - ref)
    bound = REL * np.abs(ref) + ABS_RMS * rms
    bad = valid & ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: gpu {gpu[tuple(i)]!r} ref {ref[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {int(valid.sum())} valid outputs out of tolerance "
                             f"(rms {rms:.4g}); first: {detail}")


def fp16_values(t: torch.Tensor) -> np.ndarray:
    """float64 values of an FP16 device tensor."""
    return workloads.to_numpy(t).astype(np.float64)


def sentinel_like(shape, device, dtype=torch.bfloat16) -> torch.Tensor:
    """BF16 (or FP16) buffer filled with the bit pattern 0x7FC1 (a NaN in both) to detect stray writes."""
    return torch.full(shape, 0x7FC1, dtype=torch.int16, device=device).view(dtype)


def untouched(t: torch.Tensor) -> np.ndarray:
    """Boolean mask of the entries that still hold the sentinel."""
    return t.detach().cpu().view(torch.int16).numpy() == 0x7FC1
