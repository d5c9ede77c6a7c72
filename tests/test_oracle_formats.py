"""Pins of the oracle's number formats against library conversions and the
format definitions' fixed points (CPU only)."""
import numpy as np
import pytest
import torch

import oracle


def test_f16_decode_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(b) for b in bits.tolist()])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero survives
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode_array(np.arange(256))
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_fixed_points():
    # OCP E4M3: largest finite 448, least normal 2^-6, least subnormal 2^-9, one = 0x38
    assert oracle.e4m3_to_f64(0x7E) == 448.0
    assert oracle.e4m3_to_f64(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_f64(0x01) == 2.0 ** -9
    assert oracle.e4m3_to_f64(0x38) == 1.0
    assert oracle.e4m3_to_f64(0xB8) == -1.0
    vals = oracle.e4m3_decode_array(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0), "positive codes must be strictly increasing"


def test_e4m3_round_trip_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_to_f64(c)) == c, hex(c)


def test_e4m3_ties_go_to_even_code():
    vals = oracle.e4m3_decode_array(np.arange(0x7F))
    for c in range(0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)
        assert float(mid) == (vals[c] + vals[c + 1]) / 2  # exact in binary32
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == want, (hex(c), float(mid))
        assert oracle.e4m3_encode(-mid) == want | 0x80


def test_e4m3_saturates_and_keeps_nan():
    for y in (448.0, 448.5, 463.9, 464.0, 500.0, 1e30, float("inf")):
        assert oracle.e4m3_encode(y) == 0x7E
        assert oracle.e4m3_encode(-y) == 0xFE
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    assert oracle.e4m3_encode(-np.float32("nan")) == 0x7F  # a NaN's sign carries no meaning


@pytest.mark.parametrize("scale", [1.0, 0.012345678, 3.75])
def test_e4m3_quantise_matches_torch_on_all_f16_inputs(scale):
    inv = np.float32(1.0 / np.float64(np.float32(scale)))
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = np.isfinite(x)
    y = x[finite].astype(np.float32) * inv  # one binary32 multiply
    inrange = np.abs(y) <= 448.0
    ref = torch.from_numpy(y[inrange]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    xs = x[finite][inrange]
    got = np.array([oracle.e4m3_quantize(v, inv) for v in xs.tolist()], dtype=np.uint8)
    assert np.array_equal(got, ref)
    # beyond the range the store saturates
    big = x[finite][~inrange]
    got_big = np.array([oracle.e4m3_quantize(v, inv) for v in big.tolist()], dtype=np.uint8)
    assert np.all((got_big & 0x7F) == 0x7E)
