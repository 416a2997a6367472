"""Pins for the oracle's batched FP8 GEMM with per-tensor / per-channel scales (CPU only).

MATE FlashInfer-API page, section "GEMM", bmm_fp8: A (batch,m,k) @ B (batch,k,n) with FP32 scales.
"""

import numpy as np
import pytest
import torch

from oracle import bmm, gemm

ONE = 0x38  # E4M3 code of 1.0


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return c


def _values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def test_all_ones_closed_form():
    a = np.full((2, 3, 256), ONE, np.uint8)
    b = np.full((2, 256, 5), ONE, np.uint8)
    ref = bmm.bmm_fp8(a, b, np.float32(0.5), np.float32(3.0))
    assert ref.shape == (2, 3, 5) and np.all(ref == 256 * 0.5 * 3.0)


def test_matches_torch_float64_bmm_of_dequantised_operands():
    # Library special case: torch's CPU bmm in float64 on the decoded values, scaled per channel.
    rng = np.random.default_rng(60)
    a, b = _codes(rng, (3, 17, 384)), _codes(rng, (3, 384, 40))
    sa = rng.uniform(0.1, 4, (3, 17, 1)).astype(np.float32)
    sb = rng.uniform(0.1, 4, (3, 1, 40)).astype(np.float32)
    want = torch.bmm(torch.from_numpy(_values(a)), torch.from_numpy(_values(b))).numpy()
    want = want * sa.astype(np.float64) * sb.astype(np.float64)
    assert np.array_equal(bmm.bmm_fp8(a, b, sa, sb), want)


@pytest.mark.parametrize("channel_a,channel_b", [(False, False), (True, False), (False, True), (True, True)])
def test_reduces_to_the_groupwise_form(channel_a, channel_b):
    # Scales constant along k are groupwise scales repeated over the K blocks: bmm[g] equals the
    # groupwise product of a[g] and b[g].T with a_scale = sa per row, unit b_scale, then scaled by sb
    # per column.
    rng = np.random.default_rng(61 + 2 * channel_a + channel_b)
    batch, m, k, n = 2, 9, 256, 256
    a, b = _codes(rng, (batch, m, k)), _codes(rng, (batch, k, n))
    sa = rng.uniform(0.5, 2, (batch, m, 1)).astype(np.float32) if channel_a else np.float32(1.7)
    sb = rng.uniform(0.5, 2, (batch, 1, n)).astype(np.float32) if channel_b else np.float32(0.3)
    ref = bmm.bmm_fp8(a, b, sa, sb)
    for g in range(batch):
        sa_g = (sa[g, :, 0] if channel_a else np.full(m, sa, np.float32)).astype(np.float32)
        sb_g = (sb[g, 0, :] if channel_b else np.full(n, sb, np.float32)).astype(np.float64)
        plain = gemm.gemm_fp8_nt_groupwise(a[g], b[g].T.copy(), np.repeat(sa_g[:, None], k // 128, axis=1),
                                           np.ones((n // 128, k // 128), np.float32))
        # the groupwise oracle rounds each scaled K-block term once in float64: a few 2^-53 of the
        # terms' magnitude
        np.testing.assert_allclose(ref[g], plain * sb_g[None, :], rtol=1e-13, atol=1e-13 * np.abs(ref[g]).max())


def test_rejects_wrong_scale_shapes():
    a = np.full((2, 3, 128), ONE, np.uint8)
    b = np.full((2, 128, 4), ONE, np.uint8)
    with pytest.raises(ValueError):
        bmm.bmm_fp8(a, b, np.ones((2, 1, 3), np.float32), np.float32(1))
    with pytest.raises(ValueError):
        bmm.bmm_fp8(a, b, np.float32(1), np.ones((2, 4, 1), np.float32))
