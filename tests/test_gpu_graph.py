"""The library under HIP graph capture (MI355X only): every entry point is a kernel launch on the
caller's stream with no host synchronisation and no allocation, so a caller can capture a whole
expert FFN (or a GEMM) once and replay it. Each replay must reproduce the eager result bit for bit,
with eager work on the same stream between the replays."""

import pytest
import torch

import moe_expert_matmul_amd as fp8g
import workloads
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _replays_match(run, out, eager_between):
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        run()  # warm-up on the capture stream, outside the graph
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        eager_between()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"


def test_plain_gemm_graph_replays():
    say("graph: plain GEMM")
    d = workloads.plain(512, 768, 1024, seed=51, device=DEV)
    out = torch.empty((512, 768), dtype=torch.bfloat16, device=DEV)
    scratch = torch.empty(1 << 20, device=DEV)
    _replays_match(lambda: fp8g.fp8_gemm_nt_groupwise(d["a"], d["b"], d["a_scale"], d["b_scale"], out), out,
                   lambda: scratch.normal_())


@pytest.mark.parametrize("mode", ["block", "per_tensor"])
def test_expert_ffn_graph_replays(mode):
    say("graph: expert FFN", mode)
    if mode == "block":
        d = workloads.moe(num_tokens=256, hidden=512, num_experts=8, top_k=2, inter=256, seed=52, device=DEV)
        ws = fp8g.MoeWorkspace.allocate(256, 2, 8, 512, 256, DEV)
        out = torch.empty((256, 512), dtype=torch.bfloat16, device=DEV)
        run = lambda: fp8g.moe_ffn_fp8_block_scale(d["x"], d["topk_ids"], d["topk_weights"], d["w1"], d["s1"],
                                                   d["w2"], d["s2"], out=out, workspace=ws)
    else:
        d = workloads.moe_per_tensor(256, 512, 8, 2, 256, seed=53, device=DEV)
        ws = fp8g.MoePerTensorWorkspace.allocate(256, 2, 8, 512, 256, DEV)
        out = torch.empty((256, 512), dtype=torch.bfloat16, device=DEV)
        run = lambda: fp8g.moe_ffn_fp8_per_tensor(d["x"], d["topk_ids"], d["w1"], d["w2"], d["fc1_dequant"],
                                                  d["fc2_quant"], d["fc2_dequant"], out=out, workspace=ws)
    scratch = torch.empty(1 << 20, device=DEV)
    _replays_match(run, out, lambda: scratch.normal_())
