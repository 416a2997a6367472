"""The allocation-free permutation (fp8_moe_build_permutation_noalloc) against the entry point that
takes a workspace, through the C ABI (MI355X only): bit for bit, on two calls in a row, the second
smaller than the first, so the library's scratch holds the first call's counts when the second starts."""

import ctypes

import numpy as np
import pytest
import torch

import moe_expert_matmul_amd as fp8g
from moe_expert_matmul_amd import _lib
from parity import host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _routing(num_tokens, top_k, num_experts, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, num_experts, (num_tokens, top_k)).astype(np.int32)
    drop = rng.random(ids.shape) < 0.05
    ids[drop] = rng.choice(np.array([-1, num_experts], np.int32), int(drop.sum()))
    return torch.from_numpy(ids).to(DEV)


def _permute(ids, num_experts, m_alloc, noalloc):
    lib = _lib.load()
    t, k = ids.shape
    outs = [torch.full((m_alloc,), 12345, dtype=torch.int32, device=DEV) for _ in range(2)]
    roe = torch.full((t, k), 12345, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = lib.fp8_moe_build_permutation_noalloc(ids.data_ptr(), t, k, num_experts, m_alloc, outs[0].data_ptr(),
                                                   outs[1].data_ptr(), roe.data_ptr(), stream)
    else:
        ws = torch.empty(max(lib.fp8_moe_permutation_workspace_size(t, k, num_experts), 4), dtype=torch.uint8,
                         device=DEV)
        st = lib.fp8_moe_build_permutation(ids.data_ptr(), t, k, num_experts, m_alloc, outs[0].data_ptr(),
                                           outs[1].data_ptr(), roe.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    _lib.check(st, "permutation")
    torch.cuda.synchronize()
    return host(outs[0]), host(outs[1]), host(roe)


def test_noalloc_permutation_equals_the_workspace_entry_point_on_two_calls():
    for num_tokens, top_k, num_experts, seed in [(65536, 8, 256, 1), (300, 6, 129, 2)]:
        say("no-alloc permutation", num_tokens, top_k, num_experts)
        ids = _routing(num_tokens, top_k, num_experts, seed)
        m_alloc = fp8g.default_m_alloc(num_tokens, top_k, num_experts)
        ref = _permute(ids, num_experts, m_alloc, noalloc=False)
        got = _permute(ids, num_experts, m_alloc, noalloc=True)
        for r, g, what in zip(ref, got, ("m_indices", "src_token", "row_of_entry")):
            assert np.array_equal(r, g), what


def test_noalloc_permutation_rejects_sizes_beyond_its_scratch():
    """ceil(entries/1024) * experts beyond 2^20 int32 is refused before anything is launched."""
    lib = _lib.load()
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    num_tokens, top_k, num_experts = 1 << 18, 8, 1024  # 2048 chunks x 1024 experts
    m_alloc = fp8g.default_m_alloc(num_tokens, top_k, num_experts)
    st = lib.fp8_moe_build_permutation_noalloc(p, num_tokens, top_k, num_experts, m_alloc, p, p, p, None)
    assert st == _lib.INVALID_ARGUMENT
    assert "scratch" in lib.fp8g_last_error().decode()
