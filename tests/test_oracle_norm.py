"""Pins for the oracle's fused add-RMSNorm + 1x128 FP8 quantisation (CPU only).

MATE FlashInfer-API page, section "norm", fused_add_rmsnorm_fp8_block_quant: residual += input,
RMSNorm with a per-column weight, row-major 1x128 FP8 quantisation of the result.
"""

import numpy as np
import torch

from oracle import bf16, e4m3, norm


def _bits(values):
    return bf16.to_bf16_bits(np.asarray(values, dtype=np.float64))


def test_worked_example_sqrt2():
    # One 128-wide row: residual has 64 twos then 64 zeros, input is zero, weight one, eps zero.
    # mean square = 4*64/128 = 2, so the twos become 2/sqrt(2) = sqrt(2) -> bf16 1.4140625
    # (181 * 2^-7), the zeros stay zero; the block's amax 1.4140625 maps to code 0x7E (448).
    res = np.array([[2.0] * 64 + [0.0] * 64])
    r, n, codes, scales = norm.fused_add_rmsnorm_fp8_block_quant(_bits(np.zeros((1, 128))), _bits(res),
                                                                 _bits(np.ones(128)), eps=0.0)
    assert np.array_equal(bf16.from_bf16_bits(r), res)
    nv = bf16.from_bf16_bits(n)
    assert np.all(nv[0, :64] == 1.4140625) and np.all(nv[0, 64:] == 0.0)
    assert scales[0, 0] == np.float32(1.4140625) / np.float32(448)
    assert np.all(codes[0, :64] == 0x7E) and np.all(codes[0, 64:] == 0)


def test_worked_example_with_eps_and_weight():
    # residual row all 3 (input 1 + residual 2), eps 7: mean square 9, inv = 1/sqrt(16) = 0.25,
    # normed = 3 * 0.25 * w = 0.75 w; weight 2 on the first block, -1 on the second.
    inp = np.ones((1, 256))
    res = np.full((1, 256), 2.0)
    w = np.array([2.0] * 128 + [-1.0] * 128)
    r, n, codes, scales = norm.fused_add_rmsnorm_fp8_block_quant(_bits(inp), _bits(res), _bits(w), eps=7.0)
    assert np.all(bf16.from_bf16_bits(r) == 3.0)
    nv = bf16.from_bf16_bits(n)
    assert np.all(nv[0, :128] == 1.5) and np.all(nv[0, 128:] == -0.75)
    assert scales.tolist() == [[np.float32(1.5) / np.float32(448), np.float32(0.75) / np.float32(448)]]
    assert np.all(codes[0, :128] == 0x7E) and np.all(codes[0, 128:] == 0xFE)


def test_residual_add_rounds_once_to_nearest_even():
    # bf16 keeps 7 fraction bits: near 1 the spacing is 2^-7 (every operand here is a bf16 value).
    inp = np.array([1.0, 1.0, 1.0, -1.0, 256.0, 2.0 ** -20])
    res = np.array([2.0 ** -8, 3 * 2.0 ** -8, 2.0 ** -8 + 2.0 ** -14, 1.0, 1.0, 2.0 ** -20])
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, 0.0, 256.0, 2.0 ** -19])
    got = bf16.from_bf16_bits(norm.add_residual(_bits(inp), _bits(res)))
    assert np.array_equal(got, want)


def test_matches_torch_rms_norm_in_float64():
    # Library special case: torch's CPU rms_norm in float64, rounded by torch's bfloat16 cast.
    rng = np.random.default_rng(40)
    rows, hidden = 9, 640
    inp = _bits(rng.standard_normal((rows, hidden)) * 3)
    res = _bits(rng.standard_normal((rows, hidden)) * rng.uniform(0.1, 10, (rows, 1)))
    w = _bits(rng.uniform(-2, 2, hidden))
    r, n, _, _ = norm.fused_add_rmsnorm_fp8_block_quant(inp, res, w, eps=1e-6)
    rt = torch.from_numpy(bf16.from_bf16_bits(inp)).to(torch.bfloat16) + \
        torch.from_numpy(bf16.from_bf16_bits(res)).to(torch.bfloat16)
    assert np.array_equal(bf16.from_bf16_bits(r), rt.double().numpy())
    want = torch.nn.functional.rms_norm(rt.double(), (hidden,), torch.from_numpy(bf16.from_bf16_bits(w)),
                                        eps=float(np.float32(1e-6))).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16.from_bf16_bits(n), want)


def test_scale_invariance_and_unit_mean_square():
    rng = np.random.default_rng(41)
    rows, hidden = 6, 384
    res = rng.standard_normal((rows, hidden))
    zero = _bits(np.zeros((rows, hidden)))
    ones = _bits(np.ones(hidden))
    _, n1, c1, s1 = norm.fused_add_rmsnorm_fp8_block_quant(zero, _bits(res), ones, eps=0.0)
    _, n2, c2, s2 = norm.fused_add_rmsnorm_fp8_block_quant(zero, _bits(res * 2.0 ** 9), ones, eps=0.0)
    assert np.array_equal(n1, n2) and np.array_equal(c1, c2) and np.array_equal(s1, s2)
    ms = np.mean(bf16.from_bf16_bits(n1) ** 2, axis=1)
    assert np.all(np.abs(ms - 1.0) < 2.0 ** -7)


def test_weight_scales_columns():
    rng = np.random.default_rng(42)
    res = _bits(rng.standard_normal((4, 256)))
    zero = _bits(np.zeros((4, 256)))
    w = rng.uniform(0.5, 2, 256)
    _, n1, _, _ = norm.fused_add_rmsnorm_fp8_block_quant(zero, res, _bits(np.ones(256)), eps=1e-6)
    _, nw, _, _ = norm.fused_add_rmsnorm_fp8_block_quant(zero, res, _bits(w), eps=1e-6)
    a, b = bf16.from_bf16_bits(n1) * bf16.from_bf16_bits(_bits(w)), bf16.from_bf16_bits(nw)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-30)


def test_cancelled_rows_give_zero_codes_and_unit_scales():
    rng = np.random.default_rng(43)
    x = _bits(rng.standard_normal((3, 256)))
    neg = x ^ np.uint16(0x8000)
    r, n, codes, scales = norm.fused_add_rmsnorm_fp8_block_quant(x, neg, _bits(np.ones(256)), eps=1e-6)
    assert np.all(bf16.from_bf16_bits(r) == 0) and np.all(bf16.from_bf16_bits(n) == 0)
    assert np.all(codes == 0) and np.all(scales == 1.0)


def test_quantised_output_reconstructs_normed_rows():
    rng = np.random.default_rng(44)
    inp, res = _bits(rng.standard_normal((5, 512))), _bits(rng.standard_normal((5, 512)) * 4)
    _, n, codes, scales = norm.fused_add_rmsnorm_fp8_block_quant(inp, res, _bits(rng.uniform(-1, 1, 512)))
    nv = bf16.from_bf16_bits(n)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    deq = e4m3.decode(codes) * s
    assert np.all(np.abs(deq - nv) <= 2.0 ** -4 * np.abs(nv) + s * 2.0 ** -10)
    assert np.all(np.abs(e4m3.decode(codes)).reshape(5, 4, 128).max(axis=2) == 448.0)
