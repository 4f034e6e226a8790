"""Pins the oracle's E4M3 decoder to the format definition, the pages' max-448
statement, and a library implementation (torch.float8_e4m3fn)."""
import math

import numpy as np
import pytest
import torch

from oracle import decode_e4m3fn
from workloads import encode_e4m3fn

ALL = np.arange(256, dtype=np.uint8)


def test_page_max_finite_is_448():
    # The page's format table: finite-only E4M3, largest value 448.
    v = decode_e4m3fn(ALL)
    assert np.nanmax(v) == 448.0
    assert np.nanmin(v) == -448.0
    assert decode_e4m3fn(np.array([0x7E]))[0] == 448.0


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x30, 0.5), (0x3C, 1.5), (0x39, 1.125),
    (0x08, 2.0 ** -6),            # smallest normal
    (0x01, 2.0 ** -9),            # smallest subnormal
    (0x07, 7 * 2.0 ** -9),        # largest subnormal
    (0x77, 1.875 * 2 ** 7),       # 240: exponent 14 is finite in this variant
    (0x78, 256.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_codes_from_format_definition(code, value):
    assert decode_e4m3fn(np.array([code], dtype=np.uint8))[0] == value


def test_nan_codes_and_no_infinity():
    v = decode_e4m3fn(ALL)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    assert not np.isinf(v).any()
    assert math.copysign(1.0, decode_e4m3fn(np.array([0x80]))[0]) == -1.0   # negative zero


def test_positive_codes_are_monotone_and_step_doubles_per_binade():
    v = decode_e4m3fn(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    steps = np.diff(v)
    # within one exponent field (8 codes) the step is constant; it doubles each binade
    for e in range(1, 15):
        s = steps[8 * e: 8 * e + 7]
        assert np.all(s == 2.0 ** (e - 7 - 3))


def test_decoder_matches_torch_float8_e4m3fn():
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = decode_e4m3fn(ALL)
    finite = ~np.isnan(t)
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.array_equal(v[finite], t[finite])


def test_encoder_roundtrip_and_rounding():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    vals = decode_e4m3fn(finite).astype(np.float32)
    assert np.array_equal(encode_e4m3fn(vals), finite)
    # ties to even: 1 + 1/16 lies half way between 1.0 (0x38) and 1.125 (0x39)
    assert encode_e4m3fn(np.array([1.0625], np.float32))[0] == 0x38
    assert encode_e4m3fn(np.array([1.1875], np.float32))[0] == 0x3A
    # saturation at the largest finite magnitude
    assert encode_e4m3fn(np.array([1e4, -1e4], np.float32)).tolist() == [0x7E, 0xFE]


def test_encoder_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000) * 60, rng.standard_normal(100000) * 0.01])
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = encode_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
