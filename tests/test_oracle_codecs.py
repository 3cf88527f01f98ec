"""Pins for the oracle's number formats (CPU only).

The oracle's codecs are checked against things other than themselves:
numpy's binary16 decoding, torch's float8_e4m3fn decoding and rounding, the
closed-form anchor values of the OCP E4M3FN format, and the defining
inequalities of symmetric INT8 rounding.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_f16_value_matches_numpy_on_every_bit_pattern():
    L = oracle.lib()
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([L.orc_f16_value(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


def test_e4m3_decode_matches_torch_on_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0), (0x38, 1.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x00, 0.0), (0x80, -0.0), (0xFE, -448.0), (0x40, 2.0), (0x3F, 1.875), (0x77, 240.0)])
def test_e4m3_closed_form_anchors(code, value):
    # OCP E4M3FN: bias 7, three mantissa bits, subnormal step 2^-9, max 448.
    got = oracle.e4m3_value(code)
    assert got == value and math.copysign(1, got) == math.copysign(1, value)


def test_e4m3_decode_is_exact_in_f16():
    vals = np.array([oracle.e4m3_value(c) for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(vals.astype(np.float16).astype(np.float64), vals)


def test_e4m3_round_trip_all_codes():
    for c in range(256):
        v = oracle.e4m3_value(c)
        if math.isnan(v):
            assert oracle.e4m3_encode(v) & 0x7F == 0x7F
        else:
            assert oracle.e4m3_encode(v) == c, hex(c)


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_rounding_on_f16_sweep_and_midpoints():
    f16 = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    f16 = f16[np.isfinite(f16) & (np.abs(f16) < 464.0)]
    pos = np.array(sorted({oracle.e4m3_value(c) for c in range(0x7F)}))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)      # exact ties in fp32
    nudged = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rng = np.random.default_rng(7)
    rand = (rng.standard_normal(20000) * 50).astype(np.float32)
    x = np.concatenate([f16, mids, -mids, nudged, -nudged, rand[np.abs(rand) < 464]])
    got = oracle.e4m3_encode_array(x)
    ref = _torch_e4m3(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_ties_go_to_even_code():
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(float(mid)) == want
        assert oracle.e4m3_encode(float(-mid)) == want | 0x80


@pytest.mark.parametrize("x", [448.0, 450.0, 463.99, 464.0, 500.0, 1e6, float("inf")])
def test_e4m3_saturates(x):
    assert oracle.e4m3_encode(x) == 0x7E
    assert oracle.e4m3_encode(-x) == 0xFE


def test_e4m3_nan_and_signed_zero():
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-1e-9) == 0x80      # rounds to zero, keeps the sign


def _f16(a):
    return np.asarray(a, np.float16)


def test_int8_extreme_element_maps_to_127():
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = _f16(rng.standard_normal(128) * rng.uniform(0.01, 100))
        codes, sigma = oracle.int8_encode_row(x)
        i = np.argmax(np.abs(x.astype(np.float32)))
        assert abs(int(codes[i])) == 127
        assert np.sign(codes[i]) == np.sign(x[i])
        assert sigma == np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(127)


def test_int8_matches_torch_round_half_even():
    rng = np.random.default_rng(4)
    for _ in range(50):
        x = _f16(rng.standard_normal(128) * 3)
        codes, sigma = oracle.int8_encode_row(x)
        xt = torch.from_numpy(x.astype(np.float32))
        s = xt.abs().max() / torch.tensor(127.0, dtype=torch.float32)
        ref = torch.clamp(torch.round(xt / s), -127, 127).to(torch.int8).numpy()
        assert float(s) == sigma
        assert np.array_equal(ref, codes)


def test_int8_error_bound_and_zero_row():
    rng = np.random.default_rng(5)
    x = _f16(rng.uniform(-2, 2, 128))
    codes, sigma = oracle.int8_encode_row(x)
    err = np.abs(x.astype(np.float64) - sigma * codes.astype(np.float64))
    assert np.all(err <= sigma / 2 * (1 + 1e-6))
    codes, sigma = oracle.int8_encode_row(np.zeros(128, np.float16))
    assert sigma == 0.0 and not codes.any()


def test_int8_ties_round_to_even():
    # x / sigma lands exactly on k + 1/2: max 127 with elements 0.5, 1.5, 2.5 (sigma = 1)
    x = np.zeros(128, np.float16)
    x[0] = 127.0
    x[1:4] = [0.5, 1.5, 2.5]
    x[4:7] = [-0.5, -1.5, -2.5]
    codes, sigma = oracle.int8_encode_row(x)
    assert sigma == 1.0
    assert list(codes[1:7]) == [0, 2, 2, 0, -2, -2]
