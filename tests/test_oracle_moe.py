"""Pins for the oracle's expert-FFN stages and for the seeded workloads (CPU only)."""

import hashlib
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import bf16, e4m3, moe
from oracle import gemm as gemm_module
from oracle.gemm import gemm_fp8_nt_groupwise


def test_quantize_1x128_error_bound_and_block_max():
    rng = np.random.default_rng(20)
    x = (rng.standard_normal((37, 512)) * rng.uniform(0.01, 100, (37, 1))).astype(np.float32)
    codes, scales = moe.quantize_1x128(x)
    assert codes.shape == x.shape and scales.shape == (37, 4)
    deq = e4m3.decode(codes) * np.repeat(scales.astype(np.float64), 128, axis=1)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    # RNE to 3 mantissa bits: relative error <= 2^-4 for normals, absolute <= s*2^-10 for subnormals
    assert np.all(np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + s * 2.0 ** -10)
    blk_max = np.abs(x).reshape(37, 4, 128).max(axis=2)
    assert np.array_equal(scales, (blk_max / np.float32(448)).astype(np.float32))
    # the block's largest element lands on +-448 exactly
    amax_codes = np.abs(e4m3.decode(codes)).reshape(37, 4, 128).max(axis=2)
    assert np.all(amax_codes == 448.0)


def test_quantize_1x128_zero_block_gets_unit_scale():
    x = np.zeros((2, 256), np.float32)
    x[1, 200] = -3.0
    codes, scales = moe.quantize_1x128(x)
    assert scales.tolist() == [[1.0, 1.0], [1.0, np.float32(3.0) / np.float32(448)]]
    assert np.all(codes[0] == 0) and codes[1, 200] == 0xFE


def test_quantize_1x128_agrees_with_torch_cast_quantiser():
    # Library special case: the workload quantiser rounds through torch's float8_e4m3fn cast.
    g = torch.Generator().manual_seed(21)
    x = torch.randn(64, 1024, generator=g) * 7
    tc, ts = workloads.quantize_blocks(x, 1, 128)
    oc, os_ = moe.quantize_1x128(x.numpy())
    assert np.array_equal(ts.numpy(), os_)
    assert np.array_equal(tc.numpy(), oc)


def _brute_permutation(ids, num_experts):
    rows = []
    for e in range(num_experts):
        ent = [(t, s) for t in range(ids.shape[0]) for s in range(ids.shape[1]) if ids[t, s] == e]
        rows.extend([(e, t, s) for (t, s) in ent])
        pad = (-len(ent)) % 128
        rows.extend([(-1, -1, -1)] * pad)
    return rows


def test_permutation_matches_brute_force_and_is_valid():
    rng = np.random.default_rng(22)
    T, K, E = 50, 3, 5
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:, 0] = np.where(ids[:, 0] == 4, 3, ids[:, 0])  # expert 4 still appears in slots 1-2
    p = moe.build_permutation(ids, E)
    rows = _brute_permutation(ids, E)
    assert p["m_pad"] == len(rows)
    assert p["m_indices"].size == moe.default_m_alloc(T, K, E)
    for r, (e, t, s) in enumerate(rows):
        assert p["m_indices"][r] == e and p["src_token"][r] == t
        if e >= 0:
            assert p["row_of_entry"][t, s] == r
    assert np.all(p["m_indices"][len(rows):] == -1)
    # every region starts on a 128-row boundary
    assert np.all(p["offsets"] % 128 == 0)


def test_permutation_with_an_expert_that_gets_no_rows():
    ids = np.array([[0, 2], [2, 0], [0, 2]], dtype=np.int32)
    p = moe.build_permutation(ids, 3)
    assert p["counts"].tolist() == [3, 0, 3]
    assert p["offsets"].tolist() == [0, 128, 128] and p["m_pad"] == 256


def test_permutation_drops_ids_outside_the_expert_range():
    ids = np.array([[0, 5], [-1, 1], [1, 0]], dtype=np.int32)
    p = moe.build_permutation(ids, 2)
    assert p["counts"].tolist() == [2, 2]
    assert p["row_of_entry"].tolist() == [[0, -1], [-1, 128], [129, 1]]
    out = moe.combine(np.arange(2 * 256, dtype=np.float64).reshape(256, 2), p["row_of_entry"],
                      np.ones((3, 2), np.float32))
    assert out[0].tolist() == [0.0, 1.0] and out[1].tolist() == [256.0, 257.0]


def test_silu_mul_closed_forms():
    y = np.array([[0.0, 1.0, 40.0, -40.0, 5.0, 3.0, 2.0, 7.0]])
    h = moe.silu_mul(y)[0]
    assert h[0] == 0.0
    assert h[1] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)) * 3.0, rel=1e-15)
    assert h[2] == pytest.approx(40.0 * 2.0, rel=1e-15)   # silu(x) -> x for x >> 0
    assert abs(h[3]) < 1e-14                                # silu(x) -> 0 for x << 0


def test_combine_is_the_weighted_sum_of_rows():
    rng = np.random.default_rng(23)
    y2 = rng.standard_normal((10, 4))
    rows = np.array([[1, 4], [7, 0]])
    w = np.array([[0.25, 0.5], [1.0, 2.0]], dtype=np.float32)
    out = moe.combine(y2, rows, w)
    assert np.allclose(out[0], 0.25 * y2[1] + 0.5 * y2[4], rtol=1e-15)
    assert np.allclose(out[1], y2[7] + 2.0 * y2[0], rtol=1e-15)


def test_moe_ffn_small_end_to_end_is_consistent_stage_by_stage():
    d = workloads.moe(num_tokens=40, hidden=256, num_experts=4, top_k=2, inter=128, seed=3)
    x = workloads.to_numpy(d["x"])
    xf = bf16.from_bf16_bits(x)
    ids = d["topk_ids"].numpy()
    w = d["topk_weights"].numpy()
    w1, s1, w2, s2 = (d[k].numpy() for k in ("w1", "s1", "w2", "s2"))
    r = moe.moe_ffn(xf, ids, w, w1, s1, w2, s2)
    # fc1 row of (token 5, slot 1) equals the plain GEMM of that token against its expert
    t, s = 5, 1
    row = r["perm"]["row_of_entry"][t, s]
    e = ids[t, s]
    want = gemm_fp8_nt_groupwise(r["xq"][t:t + 1], w1[e], r["xs"][t:t + 1], s1[e])[0]
    assert np.array_equal(r["y1"][row], bf16.round_to_bf16(want))
    # output of token 7 is the weighted sum of its two fc2 rows
    t = 7
    rows = r["perm"]["row_of_entry"][t]
    assert np.allclose(r["out"][t], w[t, 0] * r["y2"][rows[0]] + w[t, 1] * r["y2"][rows[1]], rtol=1e-14)
    assert np.all(np.isfinite(r["out"]))


def _sha(d):
    h = hashlib.sha256()
    for k in sorted(d):
        v = d[k]
        if isinstance(v, torch.Tensor):
            h.update(v.contiguous().view(torch.uint8).numpy().tobytes() if v.dtype != torch.bfloat16
                     else workloads.to_numpy(v).tobytes())
    return h.hexdigest()


def test_workloads_are_deterministic_per_seed():
    assert _sha(workloads.plain(16, 256, 256, seed=1)) == _sha(workloads.plain(16, 256, 256, seed=1))
    assert _sha(workloads.plain(16, 256, 256, seed=1)) != _sha(workloads.plain(16, 256, 256, seed=2))
    m1, m2 = workloads.masked(4, 32, 128, 256, seed=5), workloads.masked(4, 32, 128, 256, seed=5)
    assert _sha(m1) == _sha(m2)


def test_workload_structure_at_full_configuration_sizes():
    counts = workloads.zipf_counts(32, 8192, 1.1, 0)
    assert counts.sum() == 8192 and workloads.contiguous_layout(counts).size == 9984
    mm = np.random.default_rng(0).integers(0, 257, 16)
    assert mm.min() >= 0 and mm.max() <= 256
    ids, w = workloads.router(4096, 64, 8, 0)
    assert ids.shape == (4096, 8) and np.all(np.diff(-w, axis=1) >= 0)
    assert all(len(set(r)) == 8 for r in ids[:200])
    p = moe.build_permutation(ids, 64)
    assert p["m_pad"] == 37248 and p["m_indices"].size == 40960


def test_workload_quantiser_blocks():
    d = workloads.plain(8, 256, 384, seed=4)
    assert d["a"].dtype == torch.uint8 and d["a_scale"].shape == (8, 3) and d["b_scale"].shape == (2, 3)
    # every 128x128 block of B has an element at +-448 and no NaN codes
    b = d["b"].numpy()
    assert not np.any((b & 0x7F) == 0x7F)
    dec = np.abs(e4m3.decode(b)).reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert np.all(dec == 448.0)


# ---- per-tensor FP8 mode -------------------------------------------------------------------------

def test_per_tensor_fc1_activation_closed_form():
    # all-ones codes, hidden 128, fc1_dequant 1/64: gate = up = 2, h = silu(2) * 2 = 4 / (1 + e^-2)
    # = 3.5232, whose nearest E4M3 value is 3.5 (code 0x46; 3.75 is 0x47).
    x = np.full((2, 128), 0x38, np.uint8)
    w1 = np.full((1, 256, 128), 0x38, np.uint8)
    h, q = moe.fc1_act_per_tensor(x, np.array([0, 1]), np.array([0, 0]), w1, np.array([1 / 64], np.float32),
                                  np.array([1.0], np.float32))
    assert np.allclose(h, 4.0 / (1.0 + math.exp(-2.0)), rtol=1e-15)
    assert np.all(moe.quantize_per_tensor(q) == 0x46)
    # a large quantisation scale saturates at 448 (0x7E)
    _, q = moe.fc1_act_per_tensor(x, np.array([0, 1]), np.array([0, 0]), w1, np.array([1 / 64], np.float32),
                                  np.array([1000.0], np.float32))
    assert np.all(moe.quantize_per_tensor(q) == 0x7E)


def test_per_tensor_fc1_gathers_rows_and_uses_each_experts_scales():
    rng = np.random.default_rng(70)
    x = rng.integers(0, 0x7E, (5, 256)).astype(np.uint8)
    w1 = rng.integers(0, 0x7E, (2, 256, 256)).astype(np.uint8)
    d1 = np.array([0.01, 0.02], np.float32)
    qs = np.array([0.5, 2.0], np.float32)
    src, m_idx = np.array([4, 0, -1, 2]), np.array([1, 0, -1, 1])
    h, q = moe.fc1_act_per_tensor(x, src, m_idx, w1, d1, qs)
    for i in (0, 1, 3):
        e = m_idx[i]
        y = (e4m3.decode(x[src[i]]) @ e4m3.decode(w1[e]).T) * float(d1[e])
        g, u = y[:128], y[128:]
        assert np.allclose(h[i], g / (1 + np.exp(-g)) * u, rtol=1e-13, atol=0)
        assert np.array_equal(q[i], (h[i].astype(np.float32) * qs[e]).astype(np.float32))
    assert np.all(np.isnan(h[2])) and np.all(np.isnan(q[2]))


def test_per_tensor_fc2_reduces_to_the_groupwise_form_with_constant_scales():
    rng = np.random.default_rng(71)
    a2 = rng.integers(0, 0x7E, (256, 256)).astype(np.uint8)
    w2 = rng.integers(0, 0x7E, (2, 384, 256)).astype(np.uint8)
    d2 = np.array([0.3, 1.7], np.float32)
    m_idx = np.array([0] * 128 + [1] * 100 + [-1] * 28)
    got = moe.fc2_per_tensor(a2, m_idx, w2, d2)
    sb = np.stack([np.full((3, 2), d, np.float32) for d in d2])
    want = gemm_module.group_gemm_contiguous(a2, w2, np.ones((256, 2), np.float32), sb, m_idx)
    np.testing.assert_allclose(got[m_idx >= 0], want[m_idx >= 0], rtol=1e-13)
    assert np.all(np.isnan(got[m_idx < 0]))


def test_combine_without_weights_sums_the_rows():
    y2 = np.arange(12, dtype=np.float64).reshape(4, 3)
    rows = np.array([[0, 3], [2, -1]])
    assert np.array_equal(moe.combine(y2, rows, None), np.array([y2[0] + y2[3], y2[2]]))


def test_per_tensor_chain_stage_identities():
    rng = np.random.default_rng(72)
    t, h_, e, k, i = 6, 256, 3, 2, 128
    x = rng.integers(0, 0x7E, (t, h_)).astype(np.uint8)
    ids = np.stack([rng.permutation(e)[:k] for _ in range(t)]).astype(np.int32)
    w1 = rng.integers(0, 0x7E, (e, 2 * i, h_)).astype(np.uint8)
    w2 = rng.integers(0, 0x7E, (e, h_, i)).astype(np.uint8)
    d1 = np.full(e, 1e-3, np.float32)
    qs = np.array([0.05], np.float32)
    d2 = np.full(e, 0.01, np.float32)
    r = moe.moe_ffn_per_tensor(x, ids, w1, w2, d1, qs, d2)
    perm = r["perm"]
    valid = perm["m_indices"] >= 0
    assert np.array_equal(r["a2"][valid], moe.quantize_per_tensor(r["q"][valid]))
    y2 = bf16.round_to_bf16(moe.fc2_per_tensor(r["a2"], perm["m_indices"], w2, d2))
    assert np.array_equal(np.nan_to_num(r["y2"]), np.nan_to_num(y2))
    assert np.array_equal(r["out"], moe.combine(np.nan_to_num(y2), perm["row_of_entry"], None))
