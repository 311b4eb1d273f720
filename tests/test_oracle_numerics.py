"""Pins for oracle.numerics: exact decoding of fp16, bf16 and OCP e4m3 bytes.

The e4m3 table is checked against torch's float8_e4m3fn, a library decoding
of the same OCP format, on all 256 codes, plus spot values from the format's
definition. fp16/bf16 are checked against torch's own conversions.
"""

import numpy as np
import pytest
import torch

from oracle import numerics as N


def test_e4m3_table_matches_torch_on_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = N.e4m3_bytes_to_f64(np.arange(256))
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert (nan_ref == nan_got).all()
    assert sorted(np.nonzero(nan_got)[0].tolist()) == [0x7F, 0xFF]   # only S.1111.111 is NaN
    assert np.array_equal(ref[~nan_ref], got[~nan_got])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(got[~nan_got]))


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0),            # largest finite: 1.75 * 2^8
    (0xFE, -448.0),
    (0x08, 2.0 ** -6),        # smallest normal
    (0x01, 2.0 ** -9),        # smallest subnormal: 1/8 * 2^-6
    (0x07, 7 / 8 * 2.0 ** -6),
    (0x38, 1.0),              # exponent field 7 = bias
    (0x00, 0.0),
])
def test_e4m3_spot_values(code, value):
    assert N.e4m3_bytes_to_f64([code])[0] == value


def test_e4m3_has_no_infinity():
    assert np.isfinite(N.E4M3_TABLE[~np.isnan(N.E4M3_TABLE)]).all()
    assert np.nanmax(np.abs(N.E4M3_TABLE)) == 448.0


def test_f16_bits_decode_exactly():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    got = N.f16_bits_to_f64(bits)
    assert (np.isnan(ref) == np.isnan(got)).all()
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_bf16_bits_decode_exactly():
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = N.bf16_bits_to_f64(bits)
    assert (np.isnan(ref) == np.isnan(got)).all()
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    # spot values: 1.0 = 0x3F80, -2.0 = 0xC000, smallest normal 2^-126 = 0x0080
    assert list(N.bf16_bits_to_f64([0x3F80, 0xC000, 0x0080])) == [1.0, -2.0, 2.0 ** -126]


def test_every_e4m3_value_is_exact_in_bf16():
    # A fact the kernels rely on (fp8 -> bf16 conversion loses nothing); checked on the oracle's table.
    vals = N.E4M3_TABLE[~np.isnan(N.E4M3_TABLE)]
    as_bf16 = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, vals)


def test_f32le_bytes():
    v = np.array([1.5, -3.25e-3, 448.0], dtype="<f4")
    assert list(N.f32le_bytes_to_f64(v.view(np.uint8))) == [1.5, float(np.float32(-3.25e-3)), 448.0]
