"""Pins for the oracle's E4M3FN and BF16 codecs (CPU only).

The decode table is checked against the format's published spot values (tests/golden) and against
torch's own float8_e4m3fn decoding, a library routine; the encoder against the scalar definition,
against torch's cast, and on exact round-to-nearest-even ties.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_spot_values.txt")


def _torch_decode_all():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()


def test_decode_table_matches_torch_for_all_256_codes():
    ours = e4m3.decode_table()
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_golden_spot_values():
    lut = e4m3.decode_table()
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        code = int(code, 16)
        if val == "nan":
            assert math.isnan(lut[code])
        else:
            v = float(val)
            assert lut[code] == v and math.copysign(1, lut[code]) == math.copysign(1, v), hex(code)
        n += 1
    assert n >= 16


def test_nan_only_at_7f_and_ff_and_253_distinct_finite_values():
    lut = e4m3.decode_table()
    assert set(np.nonzero(np.isnan(lut))[0]) == {0x7F, 0xFF}
    assert len(set(lut[~np.isnan(lut)].tolist())) == 253      # +0 and -0 compare equal
    assert np.nanmax(lut) == 448.0 and np.nanmin(lut) == -448.0


def test_positive_codes_are_monotonic():
    lut = e4m3.decode_table()
    assert np.all(np.diff(lut[:0x7F]) > 0)


def test_decode_rejects_non_uint8():
    with pytest.raises(TypeError):
        e4m3.decode(np.zeros(3, dtype=np.int32))


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes)
    assert np.array_equal(e4m3.encode_rne(vals), codes)
    assert all(e4m3.encode_scalar(v) == c for v, c in zip(vals, codes))


def test_encode_vectorised_matches_scalar_definition():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4000) * 30, rng.standard_normal(2000) * 1e-2,
                        rng.uniform(-500, 500, 2000), [0.0, -0.0, 464.0, -464.0, 463.99, 1e6, -1e6]])
    x = x.astype(np.float32)
    vec = e4m3.encode_rne(x)
    ref = np.array([e4m3.encode_scalar(v) for v in x], dtype=np.uint8)
    assert np.array_equal(vec, ref)


def test_encode_matches_torch_cast_within_range():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000),
                        rng.standard_normal(20000) * 2.0 ** -7]).astype(np.float32)
    ours = e4m3.encode_rne(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_encode_ties_go_to_even_mantissa():
    lut = e4m3.decode_table()
    for c in range(0, 0x7E):
        lo, hi = lut[c], lut[c + 1]
        mid = (lo + hi) / 2.0                       # exact in float64
        got = e4m3.encode_rne(np.array([mid]))[0]
        assert got in (c, c + 1)
        assert got % 2 == 0, (hex(c), mid, hex(got))
        assert e4m3.encode_rne(np.array([-mid]))[0] == (got | 0x80)


def test_encode_saturates_and_maps_nan():
    out = e4m3.encode_rne(np.array([448.0, 463.9, 464.0, 1e30, -1e30, np.nan]))
    assert out.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(50000) * 1e3, rng.standard_normal(20000) * 1e-30,
                        rng.standard_normal(20000) * 1e30]).astype(np.float32)
    ours = bf16.to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_ties_to_even_and_roundtrip():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7: ties to 1 (even mantissa).
    assert bf16.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies between 1 + 2^-7 (odd) and 1 + 2^-6 (even): goes up.
    assert bf16.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    vals = np.array([0.0, -2.5, 3.140625, 65280.0])
    assert np.array_equal(bf16.from_bf16_bits(bf16.to_bf16_bits(vals)), vals)
