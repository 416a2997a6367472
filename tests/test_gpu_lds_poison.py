"""The GEMM kernels' LDS pipeline against a debug build whose kernels start with NaN-poisoned LDS
(every byte 0x7F: an E4M3 NaN code, 3.4e38 as an FP32 scale). A fragment or scale read that ran
ahead of the load filling it would carry the poison into the output, so every form must give the
same bytes with both builds (MI355X only)."""

import numpy as np
import pytest
import torch

import workloads
from moe_expert_matmul_amd import _lib
from parity import host, say, sentinel_like

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(call):
    """Run `call(lib)` with the normal and the poisoned build; returns the two host copies."""
    outs = []
    for lib in (_lib.load(), _lib.load_poison_lds()):
        out = call(lib)
        torch.cuda.synchronize()
        outs.append(host(out))
    return outs


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("m,n,k", [(4096, 4096, 1024), (300, 640, 1024), (129, 384, 256), (128, 256, 128)])
def test_plain_same_bytes_with_poisoned_lds(m, n, k):
    say("poisoned LDS: plain", m, n, k)
    d = workloads.plain(m, n, k, seed=11, device=DEV)

    def call(lib):
        out = sentinel_like((m, n), DEV)
        _lib.check(lib.fp8_gemm_nt_groupwise(d["a"].data_ptr(), d["b"].data_ptr(), d["a_scale"].data_ptr(),
                                             d["b_scale"].data_ptr(), out.data_ptr(), 0, m, n, k, 0, 1, 128, 128,
                                             _stream()), "plain")
        return out
    ref, got = _both(call)
    assert np.array_equal(ref, got)


def test_masked_same_bytes_with_poisoned_lds():
    say("poisoned LDS: masked")
    mm = np.array([256, 1, 130, 0, 200, 64, 255, 128], np.int32)
    d = workloads.masked(8, 256, 1024, 2048, 128, seed=12, device=DEV, masked_m=mm)

    def call(lib):
        out = sentinel_like((8, 256, 1024), DEV)
        _lib.check(lib.fp8_batch_gemm_masked(d["a"].data_ptr(), d["b"].data_ptr(), d["a_scale"].data_ptr(),
                                             d["b_scale"].data_ptr(), d["masked_m"].data_ptr(), 128, out.data_ptr(),
                                             0, 8, 256, 1024, 2048, 0, 1, 128, 128, _stream()), "masked")
        return out
    ref, got = _both(call)
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("k", [2048, 512])
def test_contiguous_same_bytes_with_poisoned_lds(k):
    """k = 2048 with large regions takes the 256-row tiles, k = 512 the 128-row ones."""
    counts = [700, 0, 5, 900, 129, 600]
    say("poisoned LDS: contiguous", counts, k)
    d = workloads.contiguous(len(counts), n=512, k=k, seed=13, device=DEV, counts=counts)

    def call(lib):
        out = sentinel_like((d["m"], 512), DEV)
        _lib.check(lib.fp8_group_gemm_contiguous(d["a"].data_ptr(), d["b"].data_ptr(), d["a_scale"].data_ptr(),
                                                 d["b_scale"].data_ptr(), d["m_indices"].data_ptr(), out.data_ptr(),
                                                 0, d["m"], 512, k, len(counts), 0, 1, 128, 128, _stream()),
                   "contiguous")
        return out
    ref, got = _both(call)
    assert np.array_equal(ref, got)


def test_fused_fc1_and_bmm_same_bytes_with_poisoned_lds():
    say("poisoned LDS: fused fc1 activation, bmm")
    d = workloads.moe(num_tokens=300, hidden=512, num_experts=5, top_k=3, inter=384, seed=14, device=DEV)
    import moe_expert_matmul_amd as fp8g
    ws = fp8g.MoeWorkspace.allocate(300, 3, 5, 512, 384, DEV)
    fp8g.moe_build_permutation(d["topk_ids"], 5, ws.m_indices, ws.src_token, ws.row_of_entry, ws.perm_scratch)
    fp8g.moe_gather_quant(d["x"], None, ws.a1, ws.sa1)

    def fc1(lib):
        q = torch.full((ws.m_alloc, 384), 0x11, dtype=torch.uint8, device=DEV)
        s = torch.full((ws.m_alloc, 3), -1.0, device=DEV)
        _lib.check(lib.fp8_moe_fc1_silu_quant(ws.a1.data_ptr(), ws.sa1.data_ptr(), 300, ws.src_token.data_ptr(),
                                              d["w1"].data_ptr(), d["s1"].data_ptr(), ws.m_indices.data_ptr(),
                                              q.data_ptr(), s.data_ptr(), ws.m_alloc, 384, 512, 5, 0, 1, 128, 128,
                                              _stream()), "fc1")
        return torch.cat([q.view(torch.float32).reshape(-1)[: q.numel() // 4], s.reshape(-1)])
    ref, got = _both(fc1)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))

    b = workloads.bmm(2, 256, 512, 1024, True, True, seed=15, device=DEV)

    def bmm(lib):
        out = torch.empty((2, 256, 512), dtype=torch.bfloat16, device=DEV)
        _lib.check(lib.fp8_bmm(b["a"].data_ptr(), b["b"].data_ptr(), b["a_scale"].data_ptr(), 1,
                               b["b_scale"].data_ptr(), 1, out.data_ptr(), 0, 2, 256, 512, 1024, _stream()), "bmm")
        return out
    ref, got = _both(bmm)
    assert np.array_equal(ref, got)
