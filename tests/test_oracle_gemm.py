"""Pins for the oracle's groupwise GEMM references (CPU only).

Each pin is independent of the oracle's own code path: closed forms, an exact rational brute force
(values decoded by torch, sums in fractions.Fraction), a single float64 library matmul over the
whole K range, the reductions between the three forms, and invariants. A dropped K block, a wrong
scale index (j % 128 for j // 128, kb for nb), a sign error or a transposed operand each fails at
least the brute force, which uses two n blocks, two k blocks and distinct random scales.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm

ONE = 0x38  # E4M3 code of 1.0


def _torch_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().double().numpy()


def _random_codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A  # no NaN codes in valid data
    return c


def _random_scales(rng, shape):
    return rng.uniform(0.25, 4.0, shape).astype(np.float32)


def test_all_ones_closed_form_is_k_alpha_beta():
    m, n, k = 128, 256, 512
    a = np.full((m, k), ONE, np.uint8)
    b = np.full((n, k), ONE, np.uint8)
    alpha, beta = np.float32(0.37), np.float32(1.9)
    ref = gemm.gemm_fp8_nt_groupwise(a, b, np.full((m, 4), alpha, np.float32),
                                     np.full((2, 4), beta, np.float32))
    assert np.all(ref == k * float(alpha) * float(beta))


def test_all_ones_with_per_block_scales():
    rng = np.random.default_rng(4)
    m, n, k = 5, 384, 512
    kb, nb = k // 128, n // 128
    sa, sb = _random_scales(rng, (m, kb)), _random_scales(rng, (nb, kb))
    ref = gemm.gemm_fp8_nt_groupwise(np.full((m, k), ONE, np.uint8), np.full((n, k), ONE, np.uint8), sa, sb)
    for i in range(m):
        for j in range(n):
            want = sum(128.0 * float(sa[i, t]) * float(sb[j // 128, t]) for t in range(kb))
            assert ref[i, j] == pytest.approx(want, rel=1e-15)


@pytest.mark.parametrize("m,n,k", [(3, 128, 128), (2, 256, 256), (4, 256, 128), (1, 128, 256)])
def test_exact_rational_brute_force(m, n, k):
    rng = np.random.default_rng(m * 1000 + n + k)
    a, b = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sa, sb = _random_scales(rng, (m, k // 128)), _random_scales(rng, (n // 128, k // 128))
    av, bv = _torch_values(a), _torch_values(b)
    ref = gemm.gemm_fp8_nt_groupwise(a, b, sa, sb)
    for i in range(m):
        for j in range(n):
            exact, magnitude = Fraction(0), Fraction(0)
            for kb in range(k // 128):
                term = Fraction(0)
                for kk in range(kb * 128, kb * 128 + 128):
                    term += Fraction(av[i, kk]) * Fraction(bv[j, kk])
                term *= Fraction(float(sa[i, kb])) * Fraction(float(sb[j // 128, kb]))
                exact += term
                magnitude += abs(term)
            # float64 rounds each scaled block term and each partial sum once: 2*KB roundings
            err = abs(Fraction(ref[i, j]) - exact)
            assert err <= 2 * (k // 128) * magnitude * Fraction(1, 2 ** 53), (i, j)


def test_matches_one_float64_matmul_of_dequantised_operands():
    rng = np.random.default_rng(5)
    m, n, k = 64, 384, 640
    a, b = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sa, sb = _random_scales(rng, (m, k // 128)), _random_scales(rng, (n // 128, k // 128))
    a_deq = _torch_values(a) * np.repeat(sa.astype(np.float64), 128, axis=1)
    b_deq = _torch_values(b) * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0), 128, axis=1)
    lib = np.matmul(a_deq, b_deq.T)
    ref = gemm.gemm_fp8_nt_groupwise(a, b, sa, sb)
    assert np.allclose(ref, lib, rtol=1e-12, atol=1e-12 * np.abs(lib).max())


def test_mn_major_is_the_transposed_layout():
    rng = np.random.default_rng(6)
    m, n, k = 7, 256, 384
    a, b = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sa, sb = _random_scales(rng, (m, 3)), _random_scales(rng, (2, 3))
    k_major = gemm.gemm_fp8_nt_groupwise(a, b, sa, sb, "K")
    mn_major = gemm.gemm_fp8_nt_groupwise(a, b, np.ascontiguousarray(sa.T), np.ascontiguousarray(sb.T), "MN")
    assert np.array_equal(k_major, mn_major)
    with pytest.raises(ValueError):
        gemm.gemm_fp8_nt_groupwise(a, b, sa, sb, "MN")


def test_scalar_b_scale_broadcasts():
    rng = np.random.default_rng(7)
    a, b = _random_codes(rng, (3, 256)), _random_codes(rng, (128, 256))
    sa = _random_scales(rng, (3, 2))
    full = gemm.gemm_fp8_nt_groupwise(a, b, sa, np.full((1, 2), 1.5, np.float32))
    scalar = gemm.gemm_fp8_nt_groupwise(a, b, sa, np.float32(1.5))
    assert np.array_equal(full, scalar)


def test_invariants_row_permutation_scale_doubling_and_block_removal():
    rng = np.random.default_rng(8)
    m, n, k = 9, 256, 384
    a, b = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sa, sb = _random_scales(rng, (m, 3)), _random_scales(rng, (2, 3))
    ref = gemm.gemm_fp8_nt_groupwise(a, b, sa, sb)
    perm = rng.permutation(m)
    assert np.array_equal(gemm.gemm_fp8_nt_groupwise(a[perm], b, sa[perm], sb), ref[perm])
    sa2 = sa.copy()
    sa2[4] *= 2
    doubled = gemm.gemm_fp8_nt_groupwise(a, b, sa2, sb)
    assert np.array_equal(doubled[4], 2 * ref[4])
    assert np.array_equal(np.delete(doubled, 4, 0), np.delete(ref, 4, 0))
    # zeroing K block 1 removes exactly its term
    a0 = a.copy()
    a0[:, 128:256] = 0
    only_other = gemm.gemm_fp8_nt_groupwise(a0, b, sa, sb)
    blk1 = gemm.gemm_fp8_nt_groupwise(a[:, 128:256], b[:, 128:256], sa[:, 1:2], sb[:, 1:2])
    # float64 rounding: a few ulps of the largest block term
    assert np.max(np.abs(only_other + blk1 - ref)) <= 1e-13 * np.max(np.abs(blk1))


def test_contiguous_reduces_to_plain_per_expert_in_any_row_order():
    rng = np.random.default_rng(9)
    groups, n, k = 3, 256, 256
    m_indices = np.array([2, -1, 0, 0, 1, -1, 2, 1, 0, 2], dtype=np.int32)  # not aligned on purpose
    m = m_indices.size
    a, b = _random_codes(rng, (m, k)), _random_codes(rng, (groups, n, k))
    sa, sb = _random_scales(rng, (m, 2)), _random_scales(rng, (groups, 2, 2))
    out = gemm.group_gemm_contiguous(a, b, sa, sb, m_indices)
    assert np.all(np.isnan(out[m_indices < 0]))
    for i in range(m):
        e = m_indices[i]
        if e >= 0:
            want = gemm.gemm_fp8_nt_groupwise(a[i:i + 1], b[e], sa[i:i + 1], sb[e])[0]
            assert np.array_equal(out[i], want)
    sub = gemm.group_gemm_contiguous(a, b, sa, sb, m_indices, rows=[6, 2])
    assert np.array_equal(sub, out[[6, 2]])


def test_masked_reduces_to_plain_on_the_prefix():
    rng = np.random.default_rng(10)
    groups, max_m, n, k = 3, 6, 128, 256
    a, b = _random_codes(rng, (groups, max_m, k)), _random_codes(rng, (groups, n, k))
    sa, sb = _random_scales(rng, (groups, max_m, 2)), _random_scales(rng, (groups, 1, 2))
    masked_m = np.array([0, 6, 4], dtype=np.int32)
    out = gemm.batch_gemm_masked(a, b, sa, sb, masked_m)
    assert np.all(np.isnan(out[0]))
    assert np.array_equal(out[1], gemm.gemm_fp8_nt_groupwise(a[1], b[1], sa[1], sb[1]))
    assert np.array_equal(out[2, :4], gemm.gemm_fp8_nt_groupwise(a[2, :4], b[2], sa[2, :4], sb[2]))
    assert np.all(np.isnan(out[2, 4:]))
    part = gemm.batch_gemm_masked(a, b, sa, sb, masked_m, groups=[2], rows=[1, 5])
    assert np.array_equal(part[2, 1], out[2, 1]) and np.all(np.isnan(part[2, 5]))


def test_plain_equals_single_group_masked_and_contiguous():
    rng = np.random.default_rng(11)
    m, n, k = 128, 256, 256
    a, b = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sa, sb = _random_scales(rng, (m, 2)), _random_scales(rng, (2, 2))
    plain = gemm.gemm_fp8_nt_groupwise(a, b, sa, sb)
    masked = gemm.batch_gemm_masked(a[None], b[None], sa[None], sb[None], np.array([m]))[0]
    contig = gemm.group_gemm_contiguous(a, b[None], sa, sb[None], np.zeros(m, np.int32))
    assert np.array_equal(plain, masked) and np.array_equal(plain, contig)


def test_rejects_k_not_multiple_of_128():
    with pytest.raises(ValueError):
        gemm.gemm_fp8_nt_groupwise(np.zeros((2, 100), np.uint8), np.zeros((128, 100), np.uint8),
                                   np.ones((2, 1), np.float32), np.ones((1, 1), np.float32))


@pytest.mark.parametrize("n", [1, 100, 130, 200])
def test_n_tail_is_the_leading_columns_of_a_padded_b(n):
    # Column j uses b-scale block j // 128 whatever n is: the result for n columns equals the first n
    # columns of the product with b padded by arbitrary rows to whole 128-row blocks.
    rng = np.random.default_rng(n)
    m, k = 6, 256
    nb = -(-n // 128)
    a, b_full = _random_codes(rng, (m, k)), _random_codes(rng, (nb * 128, k))
    sa, sb = _random_scales(rng, (m, 2)), _random_scales(rng, (nb, 2))
    full = gemm.gemm_fp8_nt_groupwise(a, b_full, sa, sb)
    assert np.array_equal(gemm.gemm_fp8_nt_groupwise(a, b_full[:n], sa, sb), full[:, :n])
    assert np.array_equal(gemm.gemm_fp8_nt_groupwise(a, b_full[:n], sa.T.copy(), sb.T.copy(), "MN"), full[:, :n])


def test_n_tail_brute_force():
    rng = np.random.default_rng(9)
    a, b = _random_codes(rng, (2, 128)), _random_codes(rng, (3, 128))
    sa, sb = _random_scales(rng, (2, 1)), _random_scales(rng, (1, 1))
    av, bv = _torch_values(a), _torch_values(b)
    ref = gemm.gemm_fp8_nt_groupwise(a, b, sa, sb)
    for i in range(2):
        for j in range(3):
            exact = sum(Fraction(av[i, t]) * Fraction(bv[j, t]) for t in range(128))
            exact *= Fraction(float(sa[i, 0])) * Fraction(float(sb[0, 0]))
            assert Fraction(ref[i, j]) == exact or abs(Fraction(ref[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 52)


def test_fp8_output_codes_closed_forms():
    # E4M3: 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A, 256 = 0x78, 448 = 0x7E; NaN = 0x7F.
    vals = np.array([2.0, 2.125, 2.375, 512.0, 896.0, 1000.0, -1e30, np.inf, np.nan, 0.0, -2.0])
    codes = gemm.fp8_output_codes(vals, 2.0)
    # 2.125/2 = 1.0625 is the midpoint of 1 and 1.125 -> even 0x38; 2.375/2 = 1.1875 -> even 0x3A;
    # beyond 448 saturates; NaN stays NaN
    assert codes.tolist() == [0x38, 0x38, 0x3A, 0x78, 0x7E, 0x7E, 0xFE, 0x7E, 0x7F, 0x00, 0xB8]


def test_fp8_output_of_an_all_ones_product():
    # a = b = 1, k = 128, unit scales: every output is 128; with output scale 0.5 the code is 256
    # (0x78), with 0.25 the quotient 512 saturates to 448 (0x7E), with 1024 it is 0.125 (0x20).
    a = np.full((4, 128), ONE, np.uint8)
    vals = gemm.gemm_fp8_nt_groupwise(a, a, np.ones((4, 1), np.float32), np.ones((1, 1), np.float32))
    assert np.all(gemm.fp8_output_codes(vals, 0.5) == 0x78)
    assert np.all(gemm.fp8_output_codes(vals, 0.25) == 0x7E)
    assert np.all(gemm.fp8_output_codes(vals, 1024.0) == 0x20)
