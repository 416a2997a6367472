"""Helpers shared by the GPU parity tests: the tolerance check and host copies."""

from __future__ import annotations

import json
import os
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


def record(case: str, **values) -> None:
    """Print measured parity figures (code flips, errors in units of rms) and, when FP8G_PARITY_RECORD
    names a file, append them to it as one JSON line."""
    say(case, json.dumps(values))
    path = os.environ.get("FP8G_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": case, **values}) + "\n")


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


def combine_bound(y2_ref, row_of_entry, weights, out_ref):
    """Bound on |GPU combine - combine(y2_ref)| when the GPU's fc2 rows each lie within the GEMM
    tolerance of the exact y2_ref and the reference combine reads y2_ref rounded to BF16: per token
    and column, sum over slots of |w| * ((REL + 2^-9) |y2| + ABS_RMS * rms(y2)), plus the combine's own
    tolerance on its output. ``weights`` None means weight 1."""
    rows = np.asarray(row_of_entry, dtype=np.int64)
    live_rows = rows[rows >= 0]
    rms_y = float(np.sqrt(np.mean(y2_ref[live_rows] ** 2))) if live_rows.size else 0.0
    w = np.ones(rows.shape) if weights is None else np.abs(np.asarray(weights, dtype=np.float64))
    bound = np.zeros((rows.shape[0], y2_ref.shape[1]))
    for slot in range(rows.shape[1]):
        r = rows[:, slot]
        live = r >= 0
        bound[live] += w[live, slot:slot + 1] * ((REL + 2.0 ** -9) * np.abs(y2_ref[r[live]]) + ABS_RMS * rms_y)
    return bound + REL * np.abs(out_ref) + ABS_RMS * float(np.sqrt(np.mean(out_ref ** 2)))


def fp16_values(t: torch.Tensor) -> np.ndarray:
    """float64 values of an FP16 device tensor."""
    return workloads.to_numpy(t).astype(np.float64)


def sentinel_like(shape, device, dtype=torch.bfloat16) -> torch.Tensor:
    """BF16 (or FP16) buffer filled with the bit pattern 0x7FC1 (a NaN in both) to detect stray writes."""
    return torch.full(shape, 0x7FC1, dtype=torch.int16, device=device).view(dtype)


def untouched(t: torch.Tensor) -> np.ndarray:
    """Boolean mask of the entries that still hold the sentinel."""
    return t.detach().cpu().view(torch.int16).numpy() == 0x7FC1
