"""Benchmark of the FP8 groupwise GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra]

The headline (``value``) times the plain 4096x4096x7168 groupwise GEMM (E4M3 inputs, 1x128 / 128x128
FP32 scales, BF16 out): W untimed launches, then exactly K launches bracketed by synchronisations and
timed with HIP events on the stream the kernel is launched on; an event between launches gives the
per-launch median and minimum beside the mean. value = algorithmic TFLOP/s (2*m*n*k per launch).
``roofline`` prices that against the dense FP8 matrix-core peak; ``traffic`` comes from the committed
rocprofv3 FETCH_SIZE/WRITE_SIZE summary when it was taken on the current kernel source, else null.
``sclk_mhz`` is the shader clock the last timed launch ran at (from the clock stamps the kernel's first
workgroup writes); ``frac_at_sclk`` prices the same time against the peak at that clock. The
part is held at its board power limit under this load, which sets that clock.
``sclk_after_timed_region_mhz`` is a one-wave probe right after the region (the clock recovers at
once, so it reads higher). ``cpu_baseline`` times the float64 CPU oracle on a bounded row sample.

``configs`` holds every workload of the benchmark, each with median and minimum per-launch time,
algorithmic TFLOP/s, the fraction of its binding roofline, and the SHA-256 of its generated inputs:
  1 plain 128x256x512 (launch-bound; back to back),
  2 plain 4096x4096x7168 (the headline, back to back),
  3 contiguous grouped over 32 Zipf-sized experts (8192 rows, n 4096, k 7168),
  4 masked batched over 16 groups (max_m 256, n 4096, k 7168, expected_m 128),
  5 the 4096-token expert FFN (hidden 7168, 64 experts, top-8, inter 2048), block scales.
Configs 3-5 stream their weights from HBM, so each of their launches starts with cold caches (a
512 MB read in between, not timed).

--extra adds the other workloads: the channelwise batched GEMM (8 x 1024x4096x7168, B read as
(k, n) in place), the add-RMSNorm + 1x128 quantiser and the plain quantiser over 4096x7168 BF16, the
per-tensor expert FFN, one GPU's share of the block-scale FFN under 8-way expert parallelism (8 of
the 64 experts), and two context lines timed back to back like the headline: the per-tensor
batched GEMM at batch 1 on the headline shape (the same matrix-core loop without per-block
promotion), and hipBLASLt's per-tensor FP8 GEMM (torch._scaled_mm) on that shape, not this path.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_DENSE_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix-core peak
NOMINAL_SCLK_MHZ = 2400.0        # the clock that peak is quoted at
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_plain_4096x4096x7168.json")
KERNEL_SOURCES = [os.path.join(ROOT, "moe_expert_matmul_amd", "csrc", f) for f in ("gemm.hip", "gemm_common.h")]


def kernel_source_hash() -> str:
    """sha256[:16] over the sources of the GEMM kernel (the traffic counters are tied to them)."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """Measured HBM bytes per launch, if the committed counters match the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def inputs_sha256(*tensors) -> str:
    """SHA-256 over the bytes of the generated inputs, in argument order."""
    import torch
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.detach().contiguous().view(torch.uint8).reshape(-1).cpu().numpy().tobytes())
    return h.hexdigest()


def sclk_probe(spin_us: int = 200):
    """Enqueue the one-wave clock probe on the current stream; returns a function giving MHz after a sync."""
    import torch
    from moe_expert_matmul_amd import _lib
    lib = _lib.load()
    buf = torch.zeros(2, dtype=torch.int64, device="cuda")
    _lib.check(lib.fp8g_clock_probe(buf.data_ptr(), spin_us, torch.cuda.current_stream().cuda_stream),
               "fp8g_clock_probe")

    def read():
        cycles, ticks = buf.tolist()
        khz = lib.fp8g_wall_clock_khz()
        return round(cycles / ticks * khz / 1000.0, 1) if ticks > 0 and khz > 0 else None
    return read


def gemm_clock_mhz():
    """Average shader clock of the most recent GEMM launch, from the stamps its first workgroup wrote."""
    import ctypes
    from moe_expert_matmul_amd import _lib
    lib = _lib.load()
    st = (ctypes.c_ulonglong * 4)()
    _lib.check(lib.fp8g_gemm_clock_record(st), "fp8g_gemm_clock_record")
    khz = lib.fp8g_wall_clock_khz()
    ticks = st[3] - st[1]
    return round((st[2] - st[0]) / ticks * khz / 1000.0, 1) if ticks > 0 and khz > 0 else None


def time_launches(fn, steps: int, warmup: int, probe: bool = False):
    """W untimed launches, then `steps` back-to-back launches between two events on the launching
    stream (the timed region: nothing else enters the stream between the launches), then `steps` more
    with an event before each, for the spread. Returns (mean ms per launch over the timed region,
    median and min ms per launch of the second pass), the wall time of the timed region, and the
    shader clock read right after it (when `probe`)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    read_clock = sclk_probe() if probe else None
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = start.elapsed_time(end) / steps
    clock = read_clock() if read_clock else None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(stream)
        fn()
    ev[steps].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return mean, per[len(per) // 2], per[0], wall, clock


def time_cold(fn, steps: int, warmup: int, flush):
    """Median and minimum per-launch time with a cache-evicting read before each launch (not timed)."""
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(steps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    return times[len(times) // 2], times[0]


def roofline_entry(med_ms, best_ms, flops, hbm_bytes, bound_us=None):
    """Per-config figures: algorithmic TFLOP/s and the fractions of the MFMA and HBM rooflines at the
    median time; ``bound_us`` overrides the roofline time (a chain of kernels: the sum of its stages')."""
    t_mfma = flops / FP8_DENSE_PEAK_TFLOPS / 1e6   # us
    t_hbm = hbm_bytes / HBM_PEAK_GBS / 1e3          # us
    t_roof = bound_us if bound_us is not None else max(t_mfma, t_hbm)
    us = med_ms * 1e3
    e = {"us_median": round(us, 2), "us_min": round(best_ms * 1e3, 2), "tflops": round(flops / us / 1e6, 2),
         "algorithmic_gflop": round(flops / 1e9, 3), "algorithmic_mb": round(hbm_bytes / 1e6, 2),
         "frac_mfma": round(t_mfma / us, 4), "frac_hbm": round(t_hbm / us, 4),
         "bound": "chain" if bound_us is not None else ("mfma" if t_mfma >= t_hbm else "hbm"),
         "roofline_us": round(t_roof, 2), "frac_roofline": round(t_roof / us, 4)}
    return e


def ffn_stage_roofline_us(rows, tokens, hidden, inter, experts, top_k):
    """Sum over the expert FFN's kernels of max(MFMA time, HBM time) at the peaks, each tensor moved
    once: token quantisation, fc1 (gathered rows, SiLU-mul and requantisation in its epilogue), fc2,
    combine (the permutation moves well under 1 MB)."""
    kb = lambda c: c // 128 * 4  # bytes of one row's 1x128 scales
    stages = [
        (0.0, tokens * hidden * 2 + tokens * hidden + tokens * kb(hidden)),
        (2.0 * rows * 2 * inter * hidden,
         rows * (hidden + kb(hidden)) + experts * 2 * inter * hidden + experts * (2 * inter // 128) * kb(hidden)
         + rows * (inter + kb(inter))),
        (2.0 * rows * hidden * inter,
         rows * (inter + kb(inter)) + experts * hidden * inter + experts * (hidden // 128) * kb(inter)
         + rows * hidden * 2),
        (0.0, rows * hidden * 2 + tokens * hidden * 2 + tokens * top_k * 8),
    ]
    return sum(max(f / FP8_DENSE_PEAK_TFLOPS / 1e6, b / HBM_PEAK_GBS / 1e3) for f, b in stages)


def cpu_baseline(d, flops_per_row):
    """Oracle on a bounded row sample of the plain workload (inputs are the GPU's bytes)."""
    import workloads
    from oracle import gemm as ogemm
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                      default=1)
    except Exception:  # threadpoolctl missing: numpy's BLAS uses every core by default
        threads = os.cpu_count()
    rows = 2048  # about 2 s of wall time on 16 host cores
    a = workloads.to_numpy(d["a"][:rows])
    sa = workloads.to_numpy(d["a_scale"][:rows])
    b = workloads.to_numpy(d["b"])
    sb = workloads.to_numpy(d["b_scale"])
    t0 = time.perf_counter()
    ogemm.gemm_fp8_nt_groupwise(a, b, sa, sb)
    dt = time.perf_counter() - t0
    return {"value": round(rows * flops_per_row / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {rows} of 4096 rows x all 4096 columns x k=7168 of the plain workload "
                      f"({rows * flops_per_row / 1e9:.1f} GFLOP, {dt:.1f} s wall on {int(threads)} threads, "
                      f"float64 BLAS per 128-wide K block)"}


def benchmark_configs(headline, steps, warmup):
    """The five workloads of the benchmark; ``headline`` carries config 2's own timing."""
    import numpy as np
    import torch
    import moe_expert_matmul_amd as fp8g
    import workloads
    dev = torch.device("cuda")
    res = {}
    cold_steps = max(5, steps // 2)

    d = workloads.plain(128, 256, 512, seed=0, device=dev)
    out = torch.empty((128, 256), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp8g.fp8_gemm_nt_groupwise(d["a"], d["b"], d["a_scale"], d["b_scale"], out)
    _, med, best, _, _ = time_launches(fn, max(steps, 20), warmup)
    e = roofline_entry(med, best, 2.0 * 128 * 256 * 512, 128 * 512 + 256 * 512 + 4 * (128 * 4 + 2 * 4) + 2 * 128 * 256)
    e["bound"] = "launch latency (parity-size case)"
    res["1_plain_m128_n256_k512"] = dict(e, timing="back to back", sclk_mhz=gemm_clock_mhz(), inputs_sha256=inputs_sha256(
        d["a"], d["b"], d["a_scale"], d["b_scale"]))
    del d, out

    res["2_plain_m4096_n4096_k7168"] = headline

    scratch = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
    # Reading 512 MB evicts L2 and the Infinity Cache. A write would leave dirty lines whose write-back
    # then overlaps the timed launch.
    flush = lambda: torch.amax(scratch)

    d = workloads.contiguous(32, 8192, 4096, 7168, 1.1, seed=0, device=dev)
    out = torch.empty((d["m"], d["n"]), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp8g.fp8_group_gemm_contiguous(d["a"], d["b"], d["a_scale"], d["b_scale"], d["m_indices"], out)
    med, best = time_cold(fn, cold_steps, 2, flush)
    valid = int(d["counts"].sum())
    hbm = d["a"].numel() + d["b"].numel() + 4 * (d["a_scale"].numel() + d["b_scale"].numel()) + d["m"] * 4 \
        + 2 * valid * 4096
    res["3_contiguous_32experts_zipf_8192rows_n4096_k7168"] = dict(
        roofline_entry(med, best, 2.0 * valid * 4096 * 7168, hbm), timing="cold caches", sclk_mhz=gemm_clock_mhz(),
        m_pad=d["m"],
        valid_rows=valid, inputs_sha256=inputs_sha256(d["a"], d["b"], d["a_scale"], d["b_scale"], d["m_indices"]))
    del d, out

    d = workloads.masked(16, 256, 4096, 7168, 128, seed=0, device=dev)
    out = torch.empty((16, 256, 4096), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp8g.fp8_batch_gemm_masked(d["a"], d["b"], d["a_scale"], d["b_scale"], d["masked_m"], 128, out)
    med, best = time_cold(fn, cold_steps, 2, flush)
    mm = workloads.to_numpy(d["masked_m"]).astype(np.int64)
    live = int((mm > 0).sum())
    rows = int(mm.sum())
    hbm = rows * 7168 + live * 4096 * 7168 + 2 * rows * 4096 + 4 * (rows * 56 + live * 32 * 56) + 16 * 4
    res["4_masked_16groups_maxm256_n4096_k7168"] = dict(
        roofline_entry(med, best, 2.0 * rows * 4096 * 7168, hbm), timing="cold caches", sclk_mhz=gemm_clock_mhz(),
        sum_masked_m=rows,
        inputs_sha256=inputs_sha256(d["a"], d["b"], d["a_scale"], d["b_scale"], d["masked_m"]))
    del d, out

    d = workloads.moe(seed=0, device=dev)
    ws = fp8g.MoeWorkspace.allocate(4096, 8, 64, 7168, 2048, dev)
    out = torch.empty((4096, 7168), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp8g.moe_ffn_fp8_block_scale(d["x"], d["topk_ids"], d["topk_weights"], d["w1"], d["s1"],
                                              d["w2"], d["s2"], out=out, workspace=ws)
    med, best = time_cold(fn, cold_steps, 2, flush)
    rows = int((d["topk_ids"] >= 0).sum().item())
    flops = 2.0 * rows * 4096 * 7168 + 2.0 * rows * 7168 * 2048
    bound = ffn_stage_roofline_us(rows, 4096, 7168, 2048, 64, 8)
    res["5_moe_ffn_4096tok_h7168_e64_top8_i2048"] = dict(
        roofline_entry(med, best, flops, 0.0, bound_us=bound), timing="cold caches", routed_rows=rows,
        sclk_mhz_fc2=gemm_clock_mhz(),
        note="roofline_us sums max(MFMA, HBM) time over the chain's kernels; tflops counts fc1 + fc2",
        inputs_sha256=inputs_sha256(d["x"], d["topk_ids"], d["topk_weights"], d["w1"], d["s1"], d["w2"], d["s2"]))
    del d, ws, out, scratch
    return res


def extra_configs(steps, warmup):
    import torch
    import moe_expert_matmul_amd as fp8g
    import workloads
    dev = torch.device("cuda")
    scratch = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
    flush = lambda: torch.amax(scratch)
    res = {}

    d = workloads.bmm(8, 1024, 4096, 7168, True, True, seed=0, device=dev)
    out = torch.empty((8, 1024, 4096), dtype=torch.bfloat16, device=dev)
    sa, sb = d["a_scale"].reshape(8, 1024), d["b_scale"].reshape(8, 4096)
    fn = lambda: fp8g.fp8_bmm(d["a"], d["b"], sa, sb, out, True, True)
    med, best = time_cold(fn, steps, warmup, flush)
    flops = 2.0 * 8 * 1024 * 4096 * 7168
    res["bmm_channelwise_8x1024x4096x7168"] = roofline_entry(med, best, flops, 8 * (1024 + 4096) * 7168 + 2 * 8 * 1024 * 4096)
    del d, out

    # The same matrix-core loop without per-block promotion (per-tensor scales, B read as (k, n)) on
    # the headline shape, and the vendor library's per-tensor FP8 GEMM (hipBLASLt through
    # torch._scaled_mm) on the same shape, for context: both back to back, like the headline.
    d = workloads.bmm(1, 4096, 4096, 7168, False, False, seed=0, device=dev)
    out = torch.empty((1, 4096, 4096), dtype=torch.bfloat16, device=dev)
    sa, sb = d["a_scale"].reshape(1), d["b_scale"].reshape(1)
    flops = 2.0 * 4096 * 4096 * 7168
    ms, med, best, _, _ = time_launches(lambda: fp8g.fp8_bmm(d["a"], d["b"], sa, sb, out, False, False), 50, 10)
    res["bmm_tensorwise_1x4096x4096x7168"] = {"us_mean": round(ms * 1e3, 2), "tflops": round(flops / ms / 1e9, 2),
                                              "frac_mfma": round(flops / ms / 1e9 / FP8_DENSE_PEAK_TFLOPS, 4)}
    try:
        a8 = d["a"][0].view(torch.float8_e4m3fn)
        b8 = d["b"][0].t().contiguous().view(torch.float8_e4m3fn)  # (n, k), K-major
        one = torch.tensor(1.0, device=dev)
        ms, _, _, _, _ = time_launches(lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one,
                                                                out_dtype=torch.bfloat16), 50, 10)
        res["reference_hipblaslt_fp8_tensorwise_4096x4096x7168"] = {
            "us_mean": round(ms * 1e3, 2), "tflops": round(flops / ms / 1e9, 2), "note": "vendor library, not this path"}
    except Exception as e:  # the reference is context only
        res["reference_hipblaslt_fp8_tensorwise_4096x4096x7168"] = {"error": f"{type(e).__name__}: {e}"[:200]}
    del d, out

    d = workloads.norm(4096, 7168, seed=0, device=dev)
    res_t = d["residual"].clone()
    normed = torch.empty_like(d["input"])
    q = torch.empty((4096, 7168), dtype=torch.uint8, device=dev)
    qs = torch.empty((4096, 56), dtype=torch.float32, device=dev)
    fn = lambda: fp8g.fused_add_rmsnorm_fp8_block_quant(q, qs, normed, d["input"], res_t, d["weight"])
    med, best = time_cold(fn, steps, warmup, flush)
    # reads input + residual (2 B each), writes residual + normed_out (2 B each), codes (1 B), scales
    res["add_rmsnorm_quant_4096x7168"] = roofline_entry(med, best, 0.0, 4096 * 7168 * 9 + 4096 * 56 * 4 + 7168 * 2)
    fn = lambda: fp8g.fp8_quantize_1x128(d["input"], q, qs)
    med, best = time_cold(fn, steps, warmup, flush)
    res["quantize_1x128_4096x7168"] = roofline_entry(med, best, 0.0, 4096 * 7168 * 3 + 4096 * 56 * 4)
    del d, res_t, normed, q, qs

    # One GPU's share under 8-way expert parallelism: experts 0-7 of the same 64 and every token's
    # routes; routes to other experts fall outside [0, 8) and are left to the other GPUs, so the
    # output is this GPU's partial sum (the part an all-to-all would return).
    d = workloads.moe(seed=0, device=dev)
    out = torch.empty((4096, 7168), dtype=torch.bfloat16, device=dev)
    shard = 8
    ws = fp8g.MoeWorkspace.allocate(4096, 8, shard, 7168, 2048, dev)
    fn = lambda: fp8g.moe_ffn_fp8_block_scale(d["x"], d["topk_ids"], d["topk_weights"], d["w1"][:shard],
                                              d["s1"][:shard], d["w2"][:shard], d["s2"][:shard], out=out,
                                              workspace=ws)
    med, best = time_cold(fn, steps, warmup, flush)
    rows = int((d["topk_ids"] < shard).sum().item())
    flops = 2.0 * rows * 4096 * 7168 + 2.0 * rows * 7168 * 2048
    res["moe_ffn_ep8_shard_8of64experts_4096tok_h7168_top8_i2048"] = dict(
        roofline_entry(med, best, flops, 0.0, bound_us=ffn_stage_roofline_us(rows, 4096, 7168, 2048, shard, 8)),
        local_rows=rows)
    del d, ws, out

    d = workloads.moe_per_tensor(seed=0, device=dev)
    ws = fp8g.MoePerTensorWorkspace.allocate(4096, 8, 64, 7168, 2048, dev)
    out = torch.empty((4096, 7168), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp8g.moe_ffn_fp8_per_tensor(d["x"], d["topk_ids"], d["w1"], d["w2"], d["fc1_dequant"],
                                             d["fc2_quant"], d["fc2_dequant"], d["fc1_input_dequant"], out=out,
                                             workspace=ws)
    med, best = time_cold(fn, steps, warmup, flush)
    rows = 4096 * 8
    flops = 2.0 * rows * 4096 * 7168 + 2.0 * rows * 7168 * 2048
    res["moe_ffn_per_tensor_4096tok_h7168_e64_top8_i2048"] = roofline_entry(med, best, flops, 0.0)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extra", "--configs", action="store_true", dest="extra",
                    help="also time the bmm, producer, per-tensor and expert-parallel workloads")
    ap.add_argument("--headline-only", action="store_true", help="time the headline GEMM only (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run five 1 GiB device-to-device copies (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); multi-GPU sharding is not built",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_expert_matmul_amd as fp8g
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "5 copies of 1 GiB (1073741824 B read + 1073741824 B written each)"}))
        return
    m = n = 4096
    k = 7168
    d = workloads.plain(m, n, k, seed=0, device=dev)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp8g.fp8_gemm_nt_groupwise(d["a"], d["b"], d["a_scale"], d["b_scale"], out)
    idle_clock = sclk_probe()
    torch.cuda.synchronize()
    idle_mhz = idle_clock()
    ms, med, best, wall, sclk_after = time_launches(fn, args.steps, args.warmup, probe=True)
    sclk = gemm_clock_mhz()  # the clock the last timed launch ran at
    flops = 2.0 * m * n * k
    tflops = flops / ms / 1e9
    frac = tflops / FP8_DENSE_PEAK_TFLOPS
    headline = dict(roofline_entry(med, best, flops, m * k + n * k + 4 * (m * 56 + 32 * 56) + 2 * m * n),
                    us_mean=round(ms * 1e3, 2), timing="back to back", sclk_mhz=sclk,
                    inputs_sha256=inputs_sha256(d["a"], d["b"], d["a_scale"], d["b_scale"]))
    line = {
        "metric": "FP8 groupwise GEMM TFLOP/s and % of MI355X dense-FP8 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_median": round(med, 5),
        "ms_min": round(best, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic: N(0,1) quantised to E4M3 per 1x128 (a) / 128x128 (b) block, seed 0",
        "config": {"workload": "plain FP8 NT groupwise GEMM m=4096 n=4096 k=7168, K-major FP32 scales, BF16 out",
                   "m": m, "n": n, "k": k},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP8_DENSE_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(frac, 4), "traffic": load_traffic()},
        "sclk_mhz": sclk,
        "sclk_after_timed_region_mhz": sclk_after,
        "sclk_idle_mhz": idle_mhz,
        "frac_at_sclk": round(frac * NOMINAL_SCLK_MHZ / sclk, 4) if sclk else None,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(d, 2.0 * n * k)
    del d, out
    torch.cuda.empty_cache()
    if not args.headline_only:
        line["configs"] = benchmark_configs(headline, args.steps, 2)
        torch.cuda.empty_cache()
        if args.extra:
            line["extra"] = extra_configs(max(5, args.steps // 5), 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
