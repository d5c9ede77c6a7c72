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


@pytest.mark.parametrize("scale", [1.0, 0.012345678])
def test_e4m3_quantise_matches_torch_on_f32_inputs(scale):
    """f32 activations: random binary32 bit patterns (every exponent) and the
    binary32 neighbours of every rounding boundary, quantised with one
    binary32 multiply by the inverse scale."""
    inv = np.float32(1.0 / np.float64(np.float32(scale)))
    x = f32_store_inputs(np.random.default_rng(7))
    with np.errstate(over="ignore", invalid="ignore"):
        x = (x * np.float32(scale)).astype(np.float32)  # the boundaries near where the scale puts them
    finite = np.isfinite(x)
    y = x[finite] * inv
    inrange = np.abs(y) <= 448.0
    ref = torch.from_numpy(y[inrange]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_quantize(v, inv) for v in x[finite][inrange].tolist()], dtype=np.uint8)
    assert np.array_equal(got, ref)
    got_big = np.array([oracle.e4m3_quantize(v, inv) for v in x[finite][~inrange].tolist()], dtype=np.uint8)
    assert np.all((got_big & 0x7F) == 0x7E)


def f32_store_inputs(rng, n_random=16384):
    """binary32 inputs for the FP8 store: the neighbours (one ulp either side)
    of every E4M3 value and of every midpoint between neighbouring values,
    both signs; the saturation edge, infinities, NaN, zeros and binary32
    subnormals; then random bit patterns."""
    vals = np.array([oracle.e4m3_to_f64(c) for c in range(0x7F)], dtype=np.float32)
    pts = list(vals) + [np.float32((vals[c] + vals[c + 1]) / 2) for c in range(0x7E)]
    pts += [448.0, 464.0, 480.0, 1e30, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 1e-40]
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(-np.inf))])
    pts = np.concatenate([pts, -pts, np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, np.finfo(np.float32).max],
                                              dtype=np.float32)])
    rand = rng.integers(0, 2 ** 32, size=n_random, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return np.concatenate([pts.astype(np.float32), rand])
