"""GPU parity of the per-tensor FP8 expert FFN (flashinfer-rs README, section "API Example: Fused MoE
FP8 (cudarc)", per-tensor FP8 mode) against the oracle, stage by stage (MI355X only).

fc1's activation codes: the GPU decides each code from its FP32 sums, the oracle from the exact
value; a code must be one the oracle gives somewhere in the band the GEMM tolerance allows around
the exact fc1 values (8e-3 |v| + 1e-3 rms(v) on gate and up), and almost all must be equal. fc2 and
the combine are held to the GEMM tolerance on the oracle fed the GPU's own inputs.
"""

import numpy as np
import pytest
import torch

import moe_expert_matmul_amd as fp8g
import workloads
from oracle import bf16, e4m3, moe as omoe
from parity import assert_within_tolerance, bf16_values, combine_bound, fp16_values, host, record, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _band_codes(d, perm, h_exact):
    """Lowest and highest code reachable within the tolerance band of gate and up."""
    x, w1 = host(d["x"]), host(d["w1"])
    m_idx, src = perm["m_indices"], perm["src_token"]
    inter = w1.shape[1] // 2
    d1 = host(d["fc1_dequant"]).astype(np.float64)
    qs = float(host(d["fc2_quant"]).reshape(-1)[0])
    lo = np.zeros(h_exact.shape, np.uint8)
    hi = np.zeros(h_exact.shape, np.uint8)
    for e in np.unique(m_idx[m_idx >= 0]):
        rows = np.nonzero(m_idx == e)[0]
        y = (e4m3.decode(x[src[rows]]) @ e4m3.decode(w1[e]).T) * d1[e]
        band = 8e-3 * np.abs(y) + 1e-3 * np.sqrt(np.mean(y ** 2))
        g, u, bg, bu = y[:, :inter], y[:, inter:], band[:, :inter], band[:, inter:]
        cands = []
        for gg in (g - bg, g, g + bg):
            for uu in (u - bu, u + bu):
                cands.append(gg / (1 + np.exp(-gg)) * uu)
        # silu has its minimum near g = -1.278 (value -0.2785): include it where the band crosses it
        gmin = -1.2784645
        inside = (g - bg <= gmin) & (gmin <= g + bg)
        for uu in (u - bu, u + bu):
            cands.append(np.where(inside, -0.27846454 * uu, cands[0]))
        c = np.stack(cands)
        lo[rows] = omoe.quantize_per_tensor((c.min(axis=0) * qs).astype(np.float32))
        hi[rows] = omoe.quantize_per_tensor((c.max(axis=0) * qs).astype(np.float32))
    return lo, hi


@pytest.mark.parametrize("case", ["small", "ffn_workload"])
def test_per_tensor_ffn_stages(case):
    if case == "small":
        d = workloads.moe_per_tensor(300, 512, 8, 3, 256, seed=3, device=DEV)
    else:
        d = workloads.moe_per_tensor(seed=0, device=DEV)
    say("per-tensor ffn", case)
    ws = fp8g.MoePerTensorWorkspace.allocate(d["num_tokens"], d["top_k"], d["num_experts"], d["hidden"],
                                             d["inter"], DEV)
    out = fp8g.moe_ffn_fp8_per_tensor(d["x"], d["topk_ids"], d["w1"], d["w2"], d["fc1_dequant"], d["fc2_quant"],
                                      d["fc2_dequant"], d["fc1_input_dequant"], workspace=ws)
    torch.cuda.synchronize()
    perm = omoe.build_permutation(host(d["topk_ids"]), d["num_experts"], ws.m_alloc)
    assert np.array_equal(host(ws.m_indices), perm["m_indices"])
    valid = perm["m_indices"] >= 0
    # (i) fc1 + activation + quantisation
    rows = np.nonzero(valid)[0]
    if case != "small":  # sample the full workload: every expert's first and last rows, and a spread
        rng = np.random.default_rng(0)
        rows = np.unique(np.concatenate([rng.choice(rows, 128, replace=False), rows[:4], rows[-4:]]))
    sub = dict(perm)
    sub["m_indices"] = perm["m_indices"][rows]
    sub["src_token"] = perm["src_token"][rows]
    h, q = omoe.fc1_act_per_tensor(host(d["x"]), sub["src_token"], sub["m_indices"], host(d["w1"]),
                                   host(d["fc1_dequant"]), host(d["fc2_quant"]))
    got = host(ws.a2)[rows]
    lo, hi = _band_codes(d, sub, h)
    gv = e4m3.decode(got)
    assert np.all((gv >= e4m3.decode(lo)) & (gv <= e4m3.decode(hi))), "activation code outside the band"
    assert np.mean(got != omoe.quantize_per_tensor(q)) < 1e-2
    # (ii) fc2 on the GPU's own codes
    y2_ref = omoe.fc2_per_tensor(host(ws.a2)[rows], sub["m_indices"], host(d["w2"]), host(d["fc2_dequant"]))
    assert_within_tolerance(bf16.from_bf16_bits(host(ws.y2)[rows]), y2_ref, f"per-tensor fc2 {case}")
    # (iii) combine (weight 1) on the GPU's own fc2 output
    # padding rows of y2 are unspecified: their bits are masked before the BF16 decode
    y2 = bf16.from_bf16_bits(np.where(valid[:, None], host(ws.y2), np.uint16(0)))
    ref = omoe.combine(y2, perm["row_of_entry"], None)
    assert_within_tolerance(bf16_values(out), ref, f"per-tensor combine {case}")


def test_per_tensor_fc2_quant_per_expert_and_fp16_out_with_weights():
    say("per-tensor ffn, per-expert fc2_quant, fp16, weights")
    d = workloads.moe_per_tensor(200, 256, 4, 2, 128, seed=4, device=DEV)
    qs = torch.tensor([0.5, 1.0, 2.0, 4.0], device=DEV) * d["fc2_quant"]
    ws = fp8g.MoePerTensorWorkspace.allocate(200, 2, 4, 256, 128, DEV)
    out = fp8g.moe_ffn_fp8_per_tensor(d["x"], d["topk_ids"], d["w1"], d["w2"], d["fc1_dequant"], qs,
                                      d["fc2_dequant"], topk_weights=d["topk_weights"], out_dtype=torch.float16,
                                      workspace=ws)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    perm = omoe.build_permutation(host(d["topk_ids"]), 4, ws.m_alloc)
    valid = perm["m_indices"] >= 0
    h, q = omoe.fc1_act_per_tensor(host(d["x"]), perm["src_token"], perm["m_indices"], host(d["w1"]),
                                   host(d["fc1_dequant"]), host(qs))
    got = host(ws.a2)[valid]
    assert np.mean(got != omoe.quantize_per_tensor(q[valid])) < 1e-2
    y2 = bf16.from_bf16_bits(np.where(valid[:, None], host(ws.y2), np.uint16(0)))  # padding rows: unspecified
    ref = omoe.combine(y2, perm["row_of_entry"], host(d["topk_weights"]))
    assert_within_tolerance(fp16_values(out), ref, "per-tensor combine fp16")


def test_per_tensor_end_to_end_against_the_oracle_chain():
    """The all-oracle chain differs from the GPU chain only through activation codes that flip near
    rounding midpoints (the GPU decides them from FP32 sums). That difference is reported, not graded;
    what is checked is the decomposition: the oracle's fc2 and combine run on the GPU's own codes give
    the GPU's output within the GEMM tolerance."""
    say("per-tensor end to end")
    d = workloads.moe_per_tensor(256, 512, 8, 2, 256, seed=6, device=DEV)
    ws = fp8g.MoePerTensorWorkspace.allocate(256, 2, 8, 512, 256, DEV)
    out = fp8g.moe_ffn_fp8_per_tensor(d["x"], d["topk_ids"], d["w1"], d["w2"], d["fc1_dequant"], d["fc2_quant"],
                                      d["fc2_dequant"], workspace=ws)
    torch.cuda.synchronize()
    r = omoe.moe_ffn_per_tensor(host(d["x"]), host(d["topk_ids"]), host(d["w1"]), host(d["w2"]),
                                host(d["fc1_dequant"]), host(d["fc2_quant"]), host(d["fc2_dequant"]),
                                m_alloc=ws.m_alloc)
    mi = r["perm"]["m_indices"]
    assert np.array_equal(host(ws.m_indices), mi)
    y2_exact = omoe.fc2_per_tensor(host(ws.a2), mi, host(d["w2"]), host(d["fc2_dequant"]))
    on_gpu_codes = omoe.combine(np.nan_to_num(bf16.round_to_bf16(y2_exact)), r["perm"]["row_of_entry"], None)
    got, ref = bf16_values(out), r["out"]
    bound = combine_bound(np.nan_to_num(y2_exact), r["perm"]["row_of_entry"], None, on_gpu_codes)
    bad = np.abs(got - on_gpu_codes) > bound
    assert not bad.any(), f"per-tensor end to end on the GPU's codes: {int(bad.sum())} outputs beyond the carried tolerance"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    valid = mi >= 0
    record("per-tensor moe T=256 H=512 E=8 k=2 I=256, end to end",
           codes_differing_from_oracle_chain=int((host(ws.a2)[valid] != r["a2"][valid]).sum()),
           codes=int(valid.sum()) * 256,
           max_err_vs_oracle_chain_rms=round(float(np.abs(got - ref).max()) / rms, 5),
           max_part_of_differing_codes_rms=round(float(np.abs(on_gpu_codes - ref).max()) / rms, 5))
