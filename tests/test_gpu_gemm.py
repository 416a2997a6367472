"""GPU parity of the three groupwise FP8 GEMM forms against the float64 oracle (MI355X only).

Every case prints its name before it touches the GPU. Small cases compare every output element;
the full workload sizes (4096x4096x7168 plain, 32 Zipf-sized experts, 16 masked groups) compare
sampled rows and column blocks, computed by the oracle one sample at a time.
"""

import os

import numpy as np
import pytest
import torch

import moe_expert_matmul_amd as fp8g
import workloads
from oracle import bf16, e4m3, gemm as ogemm
from parity import assert_within_tolerance, bf16_values, fp16_values, host, say, sentinel_like, untouched

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _plain_call(d, major="K", out=None):
    a, b, sa, sb = d["a"], d["b"], d["a_scale"], d["b_scale"]
    if major == "MN":
        sa, sb = sa.t().contiguous(), sb.t().contiguous()
    if out is None:
        out = sentinel_like((a.shape[0], b.shape[0]), DEV)
    fp8g.fp8_gemm_nt_groupwise(a, b, sa, sb, out, major)
    torch.cuda.synchronize()
    return out


def _plain_ref(d, rows=None):
    a, sa = host(d["a"]), host(d["a_scale"])
    if rows is not None:
        a, sa = a[rows], sa[rows]
    return ogemm.gemm_fp8_nt_groupwise(a, host(d["b"]), sa, host(d["b_scale"]))


PLAIN_SHAPES = [(128, 256, 512), (1, 128, 128), (17, 128, 256), (129, 384, 256), (300, 640, 1024),
                (513, 768, 384), (1000, 1152, 640), (256, 256, 128)]


@pytest.mark.parametrize("m,n,k", PLAIN_SHAPES)
def test_plain_matches_oracle(m, n, k):
    say("plain", m, n, k)
    d = workloads.plain(m, n, k, seed=m + n + k, device=DEV)
    out = _plain_call(d)
    assert_within_tolerance(bf16_values(out), _plain_ref(d), f"plain {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(37, 100, 256), (300, 200, 512), (129, 130, 384), (513, 4100, 256), (1, 1, 128)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_plain_n_tails_match_oracle(m, n, k, dtype):
    """Any n in the plain form: the last b-scale block covers n % 128 rows; n % 4 != 0 takes the
    element-wise stores. Every element of out is written, in both scale layouts and every tile."""
    say("plain n tail", m, n, k, dtype)
    d = workloads.plain(m, n, k, seed=m + n, device=DEV)
    ref = _plain_ref(d)
    values = bf16_values if dtype == torch.bfloat16 else fp16_values
    outs = []
    try:
        for tile in ("256x256", "128x256", "256x128", "128x128"):
            os.environ["FP8G_TILE"] = tile
            for major in ("K", "MN"):
                out = _plain_call(d, major, out=sentinel_like((m, n), DEV, dtype))
                assert not untouched(out).any(), f"unwritten outputs ({tile}, {major})"
                outs.append(host(out))
    finally:
        os.environ.pop("FP8G_TILE", None)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert_within_tolerance(values(torch.from_numpy(outs[0].view(np.int16)).view(dtype)), ref, f"n tail {m}x{n}x{k}")


def _midpoint_distance(q):
    """Relative distance of float32 quotients to the nearest rounding midpoint between E4M3 codes."""
    table = np.sort(np.unique(np.abs(e4m3.decode(np.arange(256, dtype=np.uint8)))))
    table = table[np.isfinite(table)]
    mids = (table[1:] + table[:-1]) / 2
    aq = np.abs(q.astype(np.float64))
    idx = np.clip(np.searchsorted(mids, aq), 1, len(mids) - 1)
    near = np.minimum(np.abs(aq - mids[idx]), np.abs(aq - mids[idx - 1]))
    return near / np.maximum(aq, 1e-30)


@pytest.mark.parametrize("m,n,k,s", [(300, 384, 512, 0.37), (129, 200, 1024, 1.3), (64, 130, 256, 0.011)])
def test_fp8_output_bit_exact_on_exact_products(m, n, k, s):
    """output_scale (E4M3 output): out = E4M3(saturate(acc / s)). With integer codes in [-4, 4] and
    power-of-two scales every partial sum is exact in FP32, so the GPU's accumulator equals the exact
    value and every code -- saturated ones included -- must equal the oracle's."""
    say("fp8 output exact", m, n, k, s)
    rng = np.random.default_rng(m + n)
    ints = lambda shape: torch.from_numpy(rng.integers(-4, 5, shape).astype(np.float32))
    a = ints((m, k)).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
    b = ints((n, k)).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
    nb = -(-n // 128)
    sa = torch.from_numpy(np.exp2(rng.integers(-3, 4, (m, k // 128))).astype(np.float32)).to(DEV)
    sb = torch.from_numpy(np.exp2(rng.integers(-3, 4, (nb, k // 128))).astype(np.float32)).to(DEV)
    osc = torch.tensor([s], dtype=torch.float32, device=DEV)
    out = fp8g.gemm_fp8_nt_groupwise(a, b, sa, sb, output_scale=osc)
    torch.cuda.synchronize()
    assert out.dtype == torch.float8_e4m3fn
    ref = ogemm.gemm_fp8_nt_groupwise(host(a), host(b), host(sa), host(sb))
    want = ogemm.fp8_output_codes(ref, np.float32(s))
    assert np.array_equal(host(out.view(torch.uint8)), want)
    assert (np.abs(e4m3.decode(want)) == 448).any() and (np.abs(e4m3.decode(want)) < 448).any()


@pytest.mark.parametrize("m,n,k", [(300, 384, 512), (129, 200, 1024)])
def test_fp8_output_within_tolerance(m, n, k):
    """Random workload: the GPU decides each code from its FP32 accumulator, which may differ from
    the exact value by the GEMM tolerance (8e-3|ref| + 1e-3 rms). Its code must be one of the codes
    the oracle gives anywhere in that band around the exact value."""
    say("fp8 output tolerance", m, n, k)
    d = workloads.plain(m, n, k, seed=m * 3 + n, device=DEV)
    ref = _plain_ref(d)
    s = np.float32(np.abs(ref).max() / 600.0)  # the largest outputs saturate
    osc = torch.tensor([s], dtype=torch.float32, device=DEV)
    out = torch.empty((m, n), dtype=torch.uint8, device=DEV)
    fp8g.fp8_gemm_nt_groupwise_fp8_out(d["a"], d["b"], d["a_scale"], d["b_scale"], osc, out)
    torch.cuda.synchronize()
    gc = host(out)
    band = 8e-3 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    lo, hi = ogemm.fp8_output_codes(ref - band, s), ogemm.fp8_output_codes(ref + band, s)
    g = e4m3.decode(gc)
    assert np.all((g >= e4m3.decode(lo)) & (g <= e4m3.decode(hi))), "code outside the tolerance band"
    exact = ogemm.fp8_output_codes(ref, s)
    assert np.mean(gc != exact) < 1e-2
    assert (np.abs(g) == 448).any()


@pytest.mark.parametrize("m,n,k", [(300, 640, 1024), (4096, 512, 256)])
def test_mn_major_scales_give_bitwise_identical_output(m, n, k):
    say("plain K vs MN major", m, n, k)
    d = workloads.plain(m, n, k, seed=7, device=DEV)
    k_out = host(_plain_call(d, "K"))
    mn_out = host(_plain_call(d, "MN"))
    assert np.array_equal(k_out, mn_out)


@pytest.mark.parametrize("form", ["plain", "masked", "contiguous"])
def test_results_do_not_depend_on_the_tile_configuration(form):
    say("tile invariance", form)
    outs = []
    try:
        for tile in ("256x256", "128x256", "256x128", "128x128"):
            os.environ["FP8G_TILE"] = tile
            if form == "plain":
                d = workloads.plain(300, 640, 1024, seed=21, device=DEV)
                outs.append(host(_plain_call(d)))
            elif form == "masked":
                d = workloads.masked(3, 256, 384, 512, 128, seed=22, device=DEV,
                                     masked_m=np.array([256, 130, 5], np.int32))
                outs.append(host(_masked_call(d)))
            else:
                # 256-row tiles whose halves hold one expert, two experts, an expert and padding
                d = workloads.contiguous(5, n=384, k=512, seed=23, device=DEV, counts=[200, 100, 0, 129, 40])
                outs.append(host(_contig_call(d)))
    finally:
        os.environ.pop("FP8G_TILE", None)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("n", [2048, 1152, 256])
def test_contiguous_tile_order_does_not_change_results(n):
    """The contiguous form's tile order (row-tile groups, or bands of column tiles whose width
    need not divide the column tiles) only changes which workgroup computes a tile: every order
    gives the same bytes, with every valid row written (the output starts as NaN sentinels)."""
    say("contiguous tile order", n)
    d = workloads.contiguous(7, n=n, k=256, seed=61, device=DEV, counts=[300, 0, 513, 40, 128, 1000, 77])
    outs = []
    try:
        for gn in ("0", "1", "3", "8", "16"):
            os.environ["FP8G_GROUP_N"] = gn
            outs.append(host(_contig_call(d)))
    finally:
        os.environ.pop("FP8G_GROUP_N", None)
    valid = host(d["m_indices"]) >= 0
    assert not (outs[0][valid] == 0x7FC1).any()  # bf16 bit patterns: no valid row left unwritten
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("form", ["plain", "masked", "contiguous", "gathered"])
def test_long_k_scale_ring_every_tile_and_layout(form):
    """25 K blocks: a's row scales travel through their three-slot LDS ring in groups of 8 (4 on the
    256x128 tile), so the ring wraps and every part phase and swizzle occurs. Every tile and both
    scale layouts give one result, which matches the oracle."""
    k = 25 * 128
    say("long k scale ring", form, k)
    if form == "plain":
        d = workloads.plain(300, 384, k, seed=51, device=DEV)
        ref = _plain_ref(d)
        call = lambda major: _plain_call(d, major)
    elif form == "masked":
        mm = np.array([256, 70, 9], np.int32)
        d = workloads.masked(3, 256, 256, k, 128, seed=52, device=DEV, masked_m=mm)
        ref = _masked_ref(d, mm)
        call = lambda major: _masked_call(d, major=major)
    else:
        d = workloads.contiguous(4, n=256, k=k, seed=53, device=DEV, counts=[200, 129, 0, 60])
        ref = _contig_ref(d)
        if form == "contiguous":
            call = lambda major: _contig_call(d, major)
        else:
            # the same rows, gathered from a shuffled copy of a and of its scales
            perm = np.random.default_rng(53).permutation(d["m"]).astype(np.int32)
            inv = np.empty_like(perm)
            inv[perm] = np.arange(d["m"], dtype=np.int32)
            src = torch.from_numpy(perm).to(DEV).long()
            a_src, sa_src = d["a"][src].contiguous(), d["a_scale"][src].contiguous()
            rows = torch.from_numpy(inv).to(DEV)

            def call(major):
                sa, sb = sa_src, d["b_scale"]
                if major == "MN":
                    sa, sb = sa.t().contiguous(), sb.transpose(1, 2).contiguous()
                out = sentinel_like((d["m"], d["n"]), DEV)
                fp8g.fp8_group_gemm_contiguous_gather(a_src, sa, rows, d["b"], sb, d["m_indices"], out, major)
                torch.cuda.synchronize()
                return out
    first, outs = None, []
    try:
        for tile in ("256x256", "128x256", "256x128", "128x128"):
            os.environ["FP8G_TILE"] = tile
            for major in ("K", "MN"):
                out = call(major)
                first = out if first is None else first
                outs.append(host(out))
    finally:
        os.environ.pop("FP8G_TILE", None)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert_within_tolerance(bf16_values(first), ref, f"long k {form}")


@pytest.mark.parametrize("form", ["plain", "contiguous", "masked"])
def test_fp16_output_matches_oracle(form):
    """out_dtype FP16 (the page's other output type): same product, FP16 round-to-nearest-even."""
    say("fp16 output", form)
    if form == "plain":
        d = workloads.plain(300, 640, 1024, seed=41, device=DEV)
        out = sentinel_like((300, 640), DEV, torch.float16)
        fp8g.fp8_gemm_nt_groupwise(d["a"], d["b"], d["a_scale"], d["b_scale"], out)
        torch.cuda.synchronize()
        assert_within_tolerance(fp16_values(out), _plain_ref(d), "plain fp16")
        wrapped = fp8g.gemm_fp8_nt_groupwise(d["a"], d["b"], d["a_scale"], d["b_scale"], out_dtype=torch.float16)
        torch.cuda.synchronize()
        assert wrapped.dtype == torch.float16 and torch.equal(wrapped, out)
    elif form == "contiguous":
        d = workloads.contiguous(4, n=256, k=384, seed=42, device=DEV, counts=[130, 0, 5, 300])
        out = sentinel_like((d["m"], d["n"]), DEV, torch.float16)
        fp8g.fp8_group_gemm_contiguous(d["a"], d["b"], d["a_scale"], d["b_scale"], d["m_indices"], out)
        torch.cuda.synchronize()
        assert_within_tolerance(fp16_values(out), _contig_ref(d), "contiguous fp16")
        mi = host(d["m_indices"])
        assert untouched(out)[mi < 0].all() and not untouched(out)[mi >= 0].any()
    else:
        mm = np.array([0, 200, 77, 129], np.int32)
        d = workloads.masked(4, 200, 384, 512, 128, seed=43, device=DEV, masked_m=mm)
        out = sentinel_like((4, 200, 384), DEV, torch.float16)
        fp8g.fp8_batch_gemm_masked(d["a"], d["b"], d["a_scale"], d["b_scale"], d["masked_m"], 128, out)
        torch.cuda.synchronize()
        assert_within_tolerance(fp16_values(out), _masked_ref(d, mm), "masked fp16")


def test_fp16_output_overflows_to_inf():
    """448 * 448 * 128 = 25.7e6 is beyond FP16's 65504: the output is +inf (and -inf), as the
    oracle's FP16 rounding of the exact value gives."""
    say("fp16 overflow")
    k = 128
    a = torch.full((4, k), 0x7E, dtype=torch.uint8, device=DEV)  # +448
    b = torch.full((128, k), 0x7E, dtype=torch.uint8, device=DEV)
    b[64:] = 0xFE  # -448
    sa = torch.ones((4, 1), device=DEV)
    sb = torch.ones((1, 1), device=DEV)
    out = fp8g.gemm_fp8_nt_groupwise(a, b, sa, sb, out_dtype=torch.float16)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):  # the overflow to inf is the point
        ref = ogemm.gemm_fp8_nt_groupwise(host(a), host(b), host(sa), host(sb)).astype(np.float16)
    got = fp16_values(out)
    assert np.isinf(ref).all() and np.array_equal(got, ref.astype(np.float64))


def test_plain_full_size_sampled_rows():
    m, n, k = 4096, 4096, 7168
    say("plain full size", m, n, k)
    d = workloads.plain(m, n, k, seed=0, device=DEV)
    out = _plain_call(d)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 255, 256, 2047, 2048, 4094, 4095],
                                     rng.choice(m, 20, replace=False)]))
    ref = _plain_ref(d, rows)
    assert_within_tolerance(bf16_values(out)[rows], ref, "plain 4096x4096x7168 sampled rows")
    assert not untouched(out).any()


def _exact_case(m, n, k, seed):
    """Codes in {0, +-1, +-2} and power-of-two scales: every partial sum is exact in FP32."""
    rng = np.random.default_rng(seed)
    pal = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
    a = pal[rng.integers(0, 5, (m, k))]
    b = pal[rng.integers(0, 5, (n, k))]
    sa = np.ldexp(1.0, rng.integers(-3, 4, (m, k // 128))).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-3, 4, (n // 128, k // 128))).astype(np.float32)
    return a, b, sa, sb


def test_plain_power_of_two_scales_are_bit_exact():
    m, n, k = 257, 384, 1024
    say("plain bit-exact", m, n, k)
    a, b, sa, sb = _exact_case(m, n, k, 3)
    t = lambda x: torch.from_numpy(x).to(DEV)
    out = sentinel_like((m, n), DEV)
    fp8g.fp8_gemm_nt_groupwise(t(a), t(b), t(sa), t(sb), out)
    torch.cuda.synchronize()
    want = bf16.to_bf16_bits(ogemm.gemm_fp8_nt_groupwise(a, b, sa, sb))
    assert np.array_equal(host(out), want)


def test_all_ones_closed_form():
    m, n, k = 128, 256, 512
    say("plain all ones", m, n, k)
    alpha, beta = np.float32(0.375), np.float32(1.25)
    a = torch.full((m, k), 0x38, dtype=torch.uint8, device=DEV)
    b = torch.full((n, k), 0x38, dtype=torch.uint8, device=DEV)
    sa = torch.full((m, k // 128), float(alpha), device=DEV)
    sb = torch.full((n // 128, k // 128), float(beta), device=DEV)
    out = fp8g.gemm_fp8_nt_groupwise(a, b, sa, sb)
    torch.cuda.synchronize()
    assert np.all(bf16_values(out) == k * float(alpha) * float(beta))


def test_k_zero_writes_zeros():
    say("plain k=0")
    a = torch.empty((5, 0), dtype=torch.uint8, device=DEV)
    b = torch.empty((128, 0), dtype=torch.uint8, device=DEV)
    out = sentinel_like((5, 128), DEV)
    fp8g.fp8_gemm_nt_groupwise(a, b, torch.empty((5, 0), device=DEV), torch.empty((1, 0), device=DEV), out)
    torch.cuda.synchronize()
    assert np.all(bf16_values(out) == 0.0)


def test_p3_wrapper_scalar_b_scale_and_preallocated_out():
    m, n, k = 64, 256, 256
    say("plain wrapper scalar b_scale", m, n, k)
    d = workloads.plain(m, n, k, seed=11, device=DEV)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    got = fp8g.gemm_fp8_nt_groupwise(d["a"].view(torch.float8_e4m3fn), d["b"], d["a_scale"],
                                     torch.tensor(0.5, device=DEV), out=out)
    torch.cuda.synchronize()
    assert got is out
    ref = ogemm.gemm_fp8_nt_groupwise(host(d["a"]), host(d["b"]), host(d["a_scale"]), np.float32(0.5))
    assert_within_tolerance(bf16_values(out), ref, "scalar b_scale")


def test_side_stream_ordering():
    m, n, k = 512, 512, 512
    say("plain on a side stream", m, n, k)
    d = workloads.plain(m, n, k, seed=12, device=DEV)
    s = torch.cuda.Stream()
    out = sentinel_like((m, n), DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp8g.fp8_gemm_nt_groupwise(d["a"], d["b"], d["a_scale"], d["b_scale"], out)
    s.synchronize()
    assert_within_tolerance(bf16_values(out), _plain_ref(d), "side stream")


# ---------------------------------------------------------------------------------------------
# masked batched form


def _masked_call(d, masked_m=None, expected_m=None, major="K"):
    sa, sb = d["a_scale"], d["b_scale"]
    if major == "MN":
        sa, sb = sa.transpose(1, 2).contiguous(), sb.transpose(1, 2).contiguous()
    mm = d["masked_m"] if masked_m is None else masked_m
    out = sentinel_like((d["num_groups"], d["max_m"], d["n"]), DEV)
    fp8g.fp8_batch_gemm_masked(d["a"], d["b"], sa, sb, mm, d["expected_m"] if expected_m is None else expected_m,
                               out, major)
    torch.cuda.synchronize()
    return out


def _masked_ref(d, masked_m, groups=None, rows=None):
    return ogemm.batch_gemm_masked(host(d["a"]), host(d["b"]), host(d["a_scale"]), host(d["b_scale"]),
                                   masked_m, groups=groups, rows=rows)


@pytest.mark.parametrize("expected_m", [1, 128, 256])
def test_masked_matches_oracle_and_leaves_other_rows(expected_m):
    G, max_m, n, k = 4, 200, 384, 512
    mm = np.array([0, 200, 77, 129], np.int32)
    say("masked", G, max_m, n, k, mm.tolist(), "expected_m", expected_m)
    d = workloads.masked(G, max_m, n, k, expected_m, seed=5, device=DEV, masked_m=mm)
    out = _masked_call(d)
    ref = _masked_ref(d, mm)
    assert_within_tolerance(bf16_values(out), ref, "masked")
    keep = untouched(out)
    for g in range(G):
        assert keep[g, mm[g]:].all(), f"group {g}: rows at or beyond masked_m were written"
        assert not keep[g, :mm[g]].any()


@pytest.mark.parametrize("k", [128, 256, 384, 1152])
def test_masked_short_k_matches_oracle(k):
    """One to nine K blocks: the masked form's schedule carries each block's last column group
    into the next block, and its 256-row tiles load b two blocks ahead into three slots and a's
    row scales eight blocks at a time, so these cover loops that are all prologue and tail, every
    slot phase, and a second scale group (k = 1152), in both scale layouts."""
    G, max_m, n = 3, 256, 384
    mm = np.array([256, 70, 129], np.int32)
    say("masked short k", G, max_m, n, k, mm.tolist())
    for expected_m in (32, 256):  # 128- and 256-row tiles
        d = workloads.masked(G, max_m, n, k, expected_m, seed=11 + k, device=DEV, masked_m=mm)
        ref = _masked_ref(d, mm)
        for major in ("K", "MN"):
            out = _masked_call(d, major=major)
            assert_within_tolerance(bf16_values(out), ref, f"masked k={k} expected_m={expected_m} {major}")


def test_masked_expected_m_never_changes_results():
    G, max_m, n, k = 3, 256, 256, 384
    mm = np.array([256, 100, 3], np.int32)
    say("masked expected_m invariance")
    d = workloads.masked(G, max_m, n, k, 128, seed=6, device=DEV, masked_m=mm)
    outs = [host(_masked_call(d, expected_m=e)) for e in (0, 1, 64, 65, 128, 256, 10000)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_masked_ignores_poisoned_rows_beyond_masked_m():
    G, max_m, n, k = 2, 160, 256, 256
    mm = np.array([33, 150], np.int32)
    say("masked with NaN codes and scales beyond masked_m")
    d = workloads.masked(G, max_m, n, k, 64, seed=8, device=DEV, masked_m=mm)
    clean = _masked_call(d)
    for g in range(G):
        d["a"][g, mm[g]:] = 0x7F
        d["a_scale"][g, mm[g]:] = float("nan")
    poisoned = _masked_call(d)
    assert np.array_equal(host(clean), host(poisoned))


def test_masked_counts_outside_range_are_clamped():
    G, max_m, n, k = 2, 64, 128, 256
    say("masked clamp")
    d = workloads.masked(G, max_m, n, k, 32, seed=9, device=DEV, masked_m=np.array([300, -4], np.int32))
    out = _masked_call(d)
    ref = _masked_ref(d, np.array([64, 0]))
    assert_within_tolerance(bf16_values(out), ref, "masked clamp")
    assert untouched(out)[1].all()


def test_masked_mn_major_bitwise_equal():
    say("masked K vs MN")
    d = workloads.masked(3, 96, 256, 384, 64, seed=10, device=DEV, masked_m=np.array([96, 50, 7], np.int32))
    assert np.array_equal(host(_masked_call(d, major="K")), host(_masked_call(d, major="MN")))


def test_masked_full_size_sampled():
    say("masked full size 16x256 n=4096 k=7168")
    d = workloads.masked(16, 256, 4096, 7168, 128, seed=0, device=DEV)
    mm = host(d["masked_m"])
    out = _masked_call(d)
    vals = bf16_values(out)
    keep = untouched(out)
    rng = np.random.default_rng(1)
    groups = [g for g in range(16) if mm[g] > 0][:6]
    for g in range(16):
        assert keep[g, mm[g]:].all() and not keep[g, :mm[g]].any()
    rows = sorted(set([0, 1, 15, 16, 127, 128, 255]) | set(rng.integers(0, 256, 6).tolist()))
    ref = _masked_ref(d, mm, groups=groups, rows=rows)
    assert_within_tolerance(vals, ref, "masked full size sampled")


# ---------------------------------------------------------------------------------------------
# contiguous grouped form


def _contig_call(d, major="K"):
    sa, sb = d["a_scale"], d["b_scale"]
    if major == "MN":
        sa, sb = sa.t().contiguous(), sb.transpose(1, 2).contiguous()
    out = sentinel_like((d["m"], d["n"]), DEV)
    fp8g.fp8_group_gemm_contiguous(d["a"], d["b"], sa, sb, d["m_indices"], out, major)
    torch.cuda.synchronize()
    return out


def _contig_ref(d, rows=None, col_blocks=None):
    b, sb = host(d["b"]), host(d["b_scale"])
    if col_blocks is not None:
        cols = np.concatenate([np.arange(c * 128, c * 128 + 128) for c in col_blocks])
        b, sb = b[:, cols], sb[:, col_blocks]
    return ogemm.group_gemm_contiguous(host(d["a"]), b, host(d["a_scale"]), sb, host(d["m_indices"]), rows=rows)


def test_contiguous_matches_oracle_and_skips_padding():
    counts = [130, 0, 5, 300]
    say("contiguous", counts)
    d = workloads.contiguous(4, n=256, k=384, seed=4, device=DEV, counts=counts)
    out = _contig_call(d)
    ref = _contig_ref(d)
    assert_within_tolerance(bf16_values(out), ref, "contiguous")
    mi = host(d["m_indices"])
    keep = untouched(out)
    assert keep[mi < 0].all() and not keep[mi >= 0].any()


def test_contiguous_trailing_padding_tiles_and_poisoned_padding_rows():
    counts = [3, 129]
    say("contiguous trailing padding", counts)
    d = workloads.contiguous(2, n=128, k=256, seed=5, device=DEV, counts=counts)
    # two extra all-padding tiles at the end, and NaN codes/scales in every padding row
    extra = 256
    d["m_indices"] = torch.cat([d["m_indices"], torch.full((extra,), -1, dtype=torch.int32, device=DEV)])
    d["a"] = torch.cat([d["a"], torch.full((extra, 256), 0x7F, dtype=torch.uint8, device=DEV)])
    d["a_scale"] = torch.cat([d["a_scale"], torch.full((extra, 2), float("nan"), device=DEV)])
    d["m"] += extra
    pad = d["m_indices"] < 0
    d["a"][pad] = 0x7F
    d["a_scale"][pad] = float("nan")
    out = _contig_call(d)
    ref = _contig_ref(d)
    assert_within_tolerance(bf16_values(out), ref, "contiguous with padding")
    assert untouched(out)[host(pad)].all()


@pytest.mark.parametrize("tile", ["128x256", "256x256"])
def test_contiguous_out_of_range_ids_count_as_padding(tile):
    """Indices outside [-1, num_groups) inside an expert's region are padding: that expert's rows
    are still computed (a stray id larger than every expert must not take over the tile), and the
    stray rows are never written."""
    counts = [100, 40, 250, 7]
    say("contiguous out-of-range ids", counts, tile)
    d = workloads.contiguous(4, n=256, k=384, seed=41, device=DEV, counts=counts)
    mi = host(d["m_indices"]).copy()
    pad = np.nonzero(mi < 0)[0]
    rng = np.random.default_rng(41)
    stray = rng.choice(pad, min(len(pad), 40), replace=False)
    mi[stray] = rng.choice(np.array([4, 9, 1 << 20, -2, -(1 << 30)], np.int32), stray.size)
    d["m_indices"] = torch.from_numpy(mi).to(DEV)
    try:
        os.environ["FP8G_TILE"] = tile
        out = _contig_call(d)
    finally:
        os.environ.pop("FP8G_TILE", None)
    ref = _contig_ref(d)  # the oracle leaves rows with ids outside [0, 4) unspecified (NaN)
    assert_within_tolerance(bf16_values(out), ref, "contiguous with out-of-range ids")
    valid = (mi >= 0) & (mi < 4)
    keep = untouched(out)
    assert keep[~valid].all() and not keep[valid].any()


def test_contiguous_mn_major_bitwise_equal():
    say("contiguous K vs MN")
    d = workloads.contiguous(3, n=256, k=512, seed=6, device=DEV, counts=[200, 64, 1])
    assert np.array_equal(host(_contig_call(d, "K")), host(_contig_call(d, "MN")))


@pytest.mark.parametrize("major", ["K", "MN"])
def test_contiguous_gather_equals_contiguous_on_gathered_rows(major):
    """Rows of a read through a_rows (with -1 on padding rows) give exactly the contiguous result."""
    counts = [130, 0, 5, 300, 1]
    say("contiguous gather", counts, major)
    d = workloads.contiguous(len(counts), n=384, k=512, seed=31, device=DEV, counts=counts)
    m = d["m"]
    rng = np.random.default_rng(31)
    tokens = 97
    src = rng.integers(0, tokens, m).astype(np.int32)
    mi = host(d["m_indices"])
    src[mi < 0] = -1
    xa = workloads.plain(tokens, 128, 512, seed=32, device=DEV)  # token rows (a) and their scales
    a_tok, sa_tok = xa["a"], xa["a_scale"]
    src_d = torch.from_numpy(src).to(DEV)
    sa_arg = sa_tok if major == "K" else sa_tok.t().contiguous()
    out_g = sentinel_like((m, d["n"]), DEV)
    fp8g.fp8_group_gemm_contiguous_gather(a_tok, sa_arg, src_d, d["b"], d["b_scale"] if major == "K" else
                                          d["b_scale"].transpose(1, 2).contiguous(), d["m_indices"], out_g, major)
    torch.cuda.synchronize()
    g = torch.from_numpy(np.maximum(src, 0)).to(DEV).long()
    d2 = dict(d, a=a_tok[g].contiguous(), a_scale=sa_tok[g].contiguous())
    out_c = _contig_call(d2, major)
    assert np.array_equal(host(out_g), host(out_c))
    ref = _contig_ref(d2)
    assert_within_tolerance(bf16_values(out_g), ref, "contiguous gather")
    assert untouched(out_g)[mi < 0].all()


def test_contiguous_full_size_sampled():
    say("contiguous full size: 32 Zipf experts, 8192 rows, n=4096, k=7168")
    d = workloads.contiguous(32, 8192, 4096, 7168, 1.1, seed=0, device=DEV)
    out = _contig_call(d)
    mi = host(d["m_indices"])
    keep = untouched(out)
    assert keep[mi < 0].all() and not keep[mi >= 0].any()
    rng = np.random.default_rng(2)
    rows = []
    for e in (0, 1, 2, 7, 19, 31):
        r = np.nonzero(mi == e)[0]
        rows += [r[0], r[-1], r[len(r) // 2]]
    rows += rng.choice(np.nonzero(mi >= 0)[0], 6, replace=False).tolist()
    rows = np.unique(np.array(rows))
    col_blocks = [0, 13, 31]
    ref = _contig_ref(d, rows=rows, col_blocks=col_blocks)
    cols = np.concatenate([np.arange(c * 128, c * 128 + 128) for c in col_blocks])
    assert_within_tolerance(bf16_values(out)[rows][:, cols], ref, "contiguous full size sampled")


@pytest.mark.parametrize("form", ["plain", "contiguous", "masked"])
def test_repeated_launches_are_bitwise_identical(form):
    """The pipeline synchronises LDS stages with a fence-free barrier and counted waits on the LDS
    DMA loads; a missing wait would show up as launches that disagree. 40 back-to-back launches of
    each form at a multi-wave size must give the same bytes."""
    say("repeated launches", form)
    if form == "plain":
        d = workloads.plain(2048, 2048, 2048, seed=31, device=DEV)
        out = torch.empty((2048, 2048), dtype=torch.bfloat16, device=DEV)
        run = lambda: fp8g.fp8_gemm_nt_groupwise(d["a"], d["b"], d["a_scale"], d["b_scale"], out)
    elif form == "contiguous":
        d = workloads.contiguous(8, n=1024, k=2048, seed=32, device=DEV, counts=[300, 700, 0, 129, 800, 64, 200, 500])
        out = torch.zeros((d["m"], 1024), dtype=torch.bfloat16, device=DEV)
        run = lambda: fp8g.fp8_group_gemm_contiguous(d["a"], d["b"], d["a_scale"], d["b_scale"], d["m_indices"], out)
    else:
        d = workloads.masked(8, 256, 1024, 2048, 128, seed=33, device=DEV,
                             masked_m=np.array([256, 1, 130, 0, 200, 64, 255, 128], np.int32))
        out = torch.zeros((8, 256, 1024), dtype=torch.bfloat16, device=DEV)
        run = lambda: fp8g.fp8_batch_gemm_masked(d["a"], d["b"], d["a_scale"], d["b_scale"], d["masked_m"], 128, out)
    run()
    torch.cuda.synchronize()
    first = out.clone()
    for _ in range(40):
        run()
        assert torch.equal(out, first), f"{form}: a repeated launch changed the output"
    torch.cuda.synchronize()
