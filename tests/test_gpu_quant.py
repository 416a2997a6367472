"""GPU parity of the a-operand producers against the oracle (MI355X only).

The 1x128 quantiser is compared bit for bit (both sides decide each code in FP32). The fused
add-RMSNorm is checked in three parts:
  * the updated residual, bit for bit (one rounding of an exact sum);
  * normed_out: the GPU's FP32 sum of squares and products differ from the oracle's float64 by a few
    FP32 ulps, so a BF16 value may differ by one step where the exact value lies within 2^-15
    (relative) of the midpoint between two BF16 numbers; every other element must match;
  * out / block_scale, bit for bit against the oracle's quantiser fed the GPU's own normed_out.
"""

import numpy as np
import pytest
import torch

import moe_expert_matmul_amd as fp8g
import workloads
from oracle import bf16, e4m3, moe as omoe, norm as onorm
from parity import host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [(1, 128), (3, 384), (67, 1152), (130, 7168), (4096, 7168)]
# hidden beyond 64 blocks: two and four blocks per team in registers, and the re-reading kernel
WIDE = [(5, 12800), (3, 25600), (2, 38400)]


def _scales_k_major(scales: np.ndarray, major: str) -> np.ndarray:
    return scales.T if major == "MN" else scales


@pytest.mark.parametrize("major", ["K", "MN"])
@pytest.mark.parametrize("rows,cols", CASES[:4] + [(7, 2304), (0, 256), (2, 38400)])
def test_quantize_1x128_bit_exact(rows, cols, major):
    say("quantize_1x128", rows, cols, major)
    g = torch.Generator(device=DEV).manual_seed(rows * 7 + cols)
    x = (torch.randn(rows, cols, generator=g, device=DEV) *
         torch.exp2(torch.randint(-12, 12, (rows, 1), generator=g, device=DEV).float())).to(torch.bfloat16)
    if rows > 1:
        x[1, :128] = 0  # an all-zero block gets scale 1
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows, cols // 128) if major == "K" else (cols // 128, rows), dtype=torch.float32, device=DEV)
    fp8g.fp8_quantize_1x128(x, out, sc, major)
    torch.cuda.synchronize()
    codes, scales = omoe.quantize_1x128(bf16.from_bf16_bits(host(x)).astype(np.float32))
    assert np.array_equal(_scales_k_major(host(sc), major), scales)
    assert np.array_equal(host(out), codes)


def _near_midpoint_rows(seed=0):
    """BF16 rows whose quotients x / (amax/448) fall on or within two FP32 ulps of a rounding midpoint
    between E4M3 codes: the cases where a division off by one ulp would change the code. Each
    128-wide block starts with its amax, followed by such x values for that amax."""
    rng = np.random.default_rng(seed)
    codes = np.arange(0x7F, dtype=np.uint8)
    e4 = np.unique(e4m3.decode(codes))
    mids = ((e4[1:] + e4[:-1]) / 2).astype(np.float32)
    xs_bits = np.arange(1, 0x7F80, dtype=np.uint16)
    xs = (xs_bits.astype(np.uint32) << 16).view(np.float32)
    blocks = []
    for ab in rng.integers(0x3000, 0x5000, 1500).astype(np.uint16):
        amax = (np.array([ab], np.uint32) << 16).view(np.float32)[0]
        s = np.float32(amax) / np.float32(448)
        cand = xs_bits[xs <= amax]
        q = (xs[xs <= amax] / s).astype(np.float32)
        idx = np.clip(np.searchsorted(mids, q), 1, len(mids) - 1)
        near = np.zeros(q.shape, bool)
        for off in (0, -1):
            near |= np.abs(q.view(np.int32) - mids[idx + off].view(np.int32)) <= 2
        sel = cand[near][:127]
        if sel.size == 0:
            continue
        blk = np.zeros(128, np.uint16)
        blk[0] = ab
        blk[1:1 + sel.size] = sel
        signs = rng.random(128) < 0.5
        blk[1:] ^= np.where(signs[1:], np.uint16(0x8000), np.uint16(0))
        blocks.append(blk)
    rows = len(blocks) // 8
    return np.stack(blocks[:rows * 8]).reshape(rows, 8 * 128)


@pytest.mark.parametrize("major", ["K", "MN"])
def test_quantize_1x128_on_rounding_midpoints(major):
    """Quotients on or next to the E4M3 rounding midpoints: bit for bit against the oracle's IEEE
    float32 division, so the kernel's division must be correctly rounded there."""
    bits = _near_midpoint_rows()
    rows, cols = bits.shape
    say("quantize_1x128 midpoints", rows, cols, major)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows, cols // 128) if major == "K" else (cols // 128, rows), dtype=torch.float32, device=DEV)
    fp8g.fp8_quantize_1x128(x, out, sc, major)
    torch.cuda.synchronize()
    codes, scales = omoe.quantize_1x128(bf16.from_bf16_bits(bits).astype(np.float32))
    assert np.array_equal(_scales_k_major(host(sc), major), scales)
    assert np.array_equal(host(out), codes)


def _check_norm(d, res_gpu, normed_gpu, out_gpu, scale_gpu, major, eps):
    inp_bits, res_bits, w_bits = d["inp_bits"], d["res_bits"], d["w_bits"]
    res_ref = onorm.add_residual(inp_bits, res_bits)
    assert np.array_equal(host(res_gpu), res_ref), "updated residual differs"
    exact = onorm.rmsnorm_values(res_ref, w_bits, eps)
    want = bf16.to_bf16_bits(exact)
    got = host(normed_gpu)
    diff = got != want
    if diff.any():
        g, w, e = bf16.from_bf16_bits(got[diff]), bf16.from_bf16_bits(want[diff]), exact[diff]
        # one BF16 step apart, and the exact value next to the midpoint between them
        step = np.abs(g - w)
        assert np.all(step <= 2.0 ** -7 * np.maximum(np.abs(g), np.abs(w))), "normed_out off by more than one step"
        mid = (g + w) / 2
        assert np.all(np.abs(e - mid) <= 2.0 ** -15 * np.abs(e)), "normed_out flip away from a rounding midpoint"
    assert diff.mean() < 1e-2, f"too many normed_out flips: {diff.mean():.3g}"
    codes, scales = omoe.quantize_1x128(bf16.from_bf16_bits(got).astype(np.float32))
    assert np.array_equal(_scales_k_major(host(scale_gpu), major), scales), "block_scale differs"
    assert np.array_equal(host(out_gpu), codes), "out codes differ"
    return diff.mean()


def _norm_inputs(rows, hidden, seed):
    d = workloads.norm(rows, hidden, seed=seed, device=DEV)
    d["inp_bits"], d["res_bits"], d["w_bits"] = host(d["input"]), host(d["residual"]), host(d["weight"])
    return d


@pytest.mark.parametrize("major", ["K", "MN"])
@pytest.mark.parametrize("rows,hidden", CASES + WIDE)
def test_fused_add_rmsnorm_quant_matches_oracle(rows, hidden, major):
    say("fused_add_rmsnorm_quant", rows, hidden, major)
    d = _norm_inputs(rows, hidden, seed=rows + hidden)
    res = d["residual"].clone()
    normed = torch.empty_like(d["input"])
    out = torch.empty((rows, hidden), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows, hidden // 128) if major == "K" else (hidden // 128, rows), dtype=torch.float32,
                     device=DEV)
    fp8g.fused_add_rmsnorm_fp8_block_quant(out, sc, normed, d["input"], res, d["weight"], 1e-6, scale_major=major)
    torch.cuda.synchronize()
    _check_norm(d, res, normed, out, sc, major, 1e-6)


def test_fused_add_rmsnorm_normed_out_may_be_input_and_rows_may_cancel():
    say("fused_add_rmsnorm_quant aliasing")
    d = _norm_inputs(64, 2048, seed=5)
    d["residual"][3] = -d["input"][3]  # this row cancels to zero: normed 0, codes 0, scales 1
    d["res_bits"] = host(d["residual"])
    inp = d["input"].clone()
    res = d["residual"].clone()
    out = torch.empty((64, 2048), dtype=torch.uint8, device=DEV)
    sc = torch.empty((64, 16), dtype=torch.float32, device=DEV)
    fp8g.fused_add_rmsnorm_fp8_block_quant(out, sc, inp, inp, res, d["weight"], 1e-5)
    torch.cuda.synchronize()
    _check_norm(d, res, inp, out, sc, "K", 1e-5)
    assert np.all(host(out)[3] == 0) and np.all(host(sc)[3] == 1.0)


def test_fused_add_rmsnorm_feeds_the_gemm():
    # The producer's out / block_scale are the a / a_scale of the plain GEMM, in either layout.
    say("fused_add_rmsnorm_quant -> gemm")
    d = _norm_inputs(256, 1024, seed=9)
    b = workloads.plain(256, 512, 1024, seed=9, device=DEV)
    outs = []
    for major in ("K", "MN"):
        res = d["residual"].clone()
        normed = torch.empty_like(d["input"])
        a = torch.empty((256, 1024), dtype=torch.uint8, device=DEV)
        sa = torch.empty((256, 8) if major == "K" else (8, 256), dtype=torch.float32, device=DEV)
        fp8g.fused_add_rmsnorm_fp8_block_quant(a, sa, normed, d["input"], res, d["weight"], scale_major=major)
        sb = b["b_scale"] if major == "K" else b["b_scale"].T.contiguous()
        outs.append(host(fp8g.gemm_fp8_nt_groupwise(a, b["b"], sa, sb, scale_major_mode=major)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
