"""GPU parity of the batched FP8 GEMM with per-tensor / per-channel scales (MATE FlashInfer-API
page, section "GEMM", bmm_fp8) against the float64 oracle (MI355X only). Tolerance as for the
groupwise forms: |gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref)."""

import os

import numpy as np
import pytest
import torch

import moe_expert_matmul_amd as fp8g
import workloads
from oracle import bmm as obmm
from parity import assert_within_tolerance, bf16_values, fp16_values, host, say, sentinel_like, untouched

pytestmark = pytest.mark.gpu
DEV = "cuda"

# b is read as (k, n) slabs of the tile's columns: n below one tile (16, 48, 128), a last tile with
# one 16-column chunk (4112 = 16 * 257), and 25 K blocks
CASES = [(1, 1, 16, 128), (3, 37, 48, 256), (2, 64, 128, 256), (2, 300, 272, 512), (4, 129, 1040, 384),
         (8, 1000, 512, 1024), (1, 17, 4112, 3200)]


def _ref(d):
    return obmm.bmm_fp8(host(d["a"]), host(d["b"]), host(d["a_scale"]), host(d["b_scale"]))


@pytest.mark.parametrize("channel_a,channel_b", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("batch,m,n,k", CASES)
def test_bmm_matches_oracle(batch, m, n, k, channel_a, channel_b):
    say("bmm", batch, m, n, k, channel_a, channel_b)
    d = workloads.bmm(batch, m, n, k, channel_a, channel_b, seed=batch + m + n, device=DEV)
    out = fp8g.bmm_fp8(d["a"], d["b"], d["a_scale"], d["b_scale"], torch.bfloat16)
    torch.cuda.synchronize()
    assert out.shape == (batch, m, n) and out.dtype == torch.bfloat16
    assert_within_tolerance(bf16_values(out), _ref(d), f"bmm {batch}x{m}x{n}x{k} {channel_a} {channel_b}")


def test_bmm_fp16_every_element_written_and_tile_invariant():
    say("bmm fp16, tiles")
    d = workloads.bmm(3, 300, 272, 512, True, True, seed=5, device=DEV)
    outs = []
    try:
        for tile in ("256x256", "128x256", "256x128", "128x128"):
            os.environ["FP8G_TILE"] = tile
            out = sentinel_like((3, 300, 272), DEV, torch.float16)
            fp8g.bmm_fp8(d["a"], d["b"], d["a_scale"], d["b_scale"], torch.float16, out=out)
            torch.cuda.synchronize()
            assert not untouched(out).any()
            outs.append(host(out))
    finally:
        os.environ.pop("FP8G_TILE", None)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert_within_tolerance(outs[0].astype(np.float64), _ref(d), "bmm fp16")


def test_bmm_k_zero_writes_zeros():
    say("bmm k=0")
    a = torch.empty((2, 5, 0), dtype=torch.uint8, device=DEV)
    b = torch.empty((2, 0, 32), dtype=torch.uint8, device=DEV)
    out = fp8g.bmm_fp8(a, b, torch.tensor(2.0, device=DEV), torch.tensor(3.0, device=DEV), torch.bfloat16)
    torch.cuda.synchronize()
    assert np.all(bf16_values(out) == 0)


def test_bmm_full_size_sampled():
    batch, m, n, k = 8, 1024, 4096, 7168
    say("bmm full size", batch, m, n, k)
    d = workloads.bmm(batch, m, n, k, True, True, seed=0, device=DEV)
    out = fp8g.bmm_fp8(d["a"], d["b"], d["a_scale"], d["b_scale"], torch.bfloat16)
    torch.cuda.synchronize()
    got = bf16_values(out)
    rng = np.random.default_rng(0)
    a, b, sa, sb = host(d["a"]), host(d["b"]), host(d["a_scale"]), host(d["b_scale"])
    for g in (0, 7):
        rows = np.unique(np.concatenate([[0, 255, 256, 1023], rng.choice(m, 6, replace=False)]))
        ref = obmm.bmm_fp8(a[g:g + 1, rows], b[g:g + 1], sa[g:g + 1, rows], sb[g:g + 1])[0]
        assert_within_tolerance(got[g, rows], ref, f"bmm full size batch {g}")


def test_bmm_with_out_allocates_nothing_and_leaves_b_alone():
    """With out given and FP32 scales, the MATE-signature call allocates no device memory (b is read
    in place, as (batch, k, n)), leaves b unchanged, and gives the values of the call that
    allocates its own out; over two calls, the second smaller."""
    for batch, m, n, k in [(4, 129, 1040, 384), (2, 37, 48, 256)]:
        say("bmm allocation-free", batch, m, n, k)
        d = workloads.bmm(batch, m, n, k, True, True, seed=7 + m, device=DEV)
        b_before = d["b"].clone()
        own = fp8g.bmm_fp8(d["a"], d["b"], d["a_scale"], d["b_scale"], torch.bfloat16)
        out = torch.empty_like(own)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        before = torch.cuda.memory_allocated()
        fp8g.bmm_fp8(d["a"], d["b"], d["a_scale"], d["b_scale"], torch.bfloat16, out=out)
        torch.cuda.synchronize()
        assert torch.cuda.max_memory_allocated() == before
        assert torch.equal(own, out)
        assert torch.equal(d["b"], b_before)
